// Host build of the GPU geometry (vsa_classify_geom.h, vsa_geom.h) against brute force.
//
// For random grids, token orders (frame-, tile-, position-major, tile-major over a padded
// grid), mask kinds and tile sizes: the boxes of every query and key range are checked
// to hold exactly the range's positions; every (query tile, key tile) class and kept-pair
// count, over box arrays (tile_class, box_pair_kept) and in the streamed form the GPU
// kernel runs (tile_class_range, tile_counts), is compared with an enumeration of all
// pairs under a per-pair predicate written out here; and every bit of the 64-key row
// masks (tile_row_mask, real_key_mask) with the same predicate.  The coordinates of the
// padded and position-major orders are also checked against nested loops that state
// them.
//
// usage: geometry_check TRIALS SEED [focus]; "focus" draws one-column tiles and stripe
// periods of one row or one frame (the closed-form stripe paths).  Exit status 1 on any
// mismatch.
#include "vsa_classify_geom.h"
#include <cstdio>
#include <cstdlib>
#include <vector>
using namespace vsa;
static bool keep_bf(const Geom& g, const DevMask& m, int tq,int yq,int xq,int tk,int yk,int xk){
  if (tk < m.sink) return true;
  switch(m.kind){
    case 0: return true;
    case 1: return (m.rt<0||abs(tk-tq)<=m.rt)&&(m.rh<0||abs(yk-yq)<=m.rh)&&(m.rw<0||abs(xk-xq)<=m.rw);
    case 2: { int sq=yq*g.Wg+xq, sk=yk*g.Wg+xk; return (abs(tk-tq-m.To)%m.Ts)<=m.Tw-1 && (abs(sk-sq-m.So)%m.Ss)<=m.Sw-1; }
    case 3: { auto st=[&](int a,int w,int n){int s=a-w/2; if(s<0)s=0; int mx=n-w<0?0:n-w; if(s>mx)s=mx; return s;};
      int a0=tq/g.bt,b0=tk/g.bt,a1=yq/g.bh,b1=yk/g.bh,a2=xq/g.bw,b2=xk/g.bw;
      int s0=st(a0,m.wt,g.nT),s1=st(a1,m.wh,g.nH),s2=st(a2,m.ww,g.nW);
      return b0>=s0&&b0<s0+m.wt&&b1>=s1&&b1<s1+m.wh&&b2>=s2&&b2<s2+m.ww; }
  }
  return false;
}
int main(int argc, char** argv){
  const int trials = argc > 1 ? atoi(argv[1]) : 3000;
  srand(argc > 2 ? atoi(argv[2]) : 1);
  const int focus = argc > 3;  // one-column tiles and stripe periods of a row or a frame
  long long ntile=0, nbad=0, nmask=0, nmbad=0;
  // division by invariant divisors: every divisor up to 4096 and random ones up to 2^31
  // against the hardware division, at multiples of d and their neighbours, the ends of
  // the 32-bit range and random numerators; floor_div_by on both signs
  for(int i=0;i<4096+20000;++i){
    const uint32_t d = i<4096 ? (uint32_t)(i+1) : 1u+(uint32_t)(((uint64_t)rand()*RAND_MAX+rand())%2147483647u);
    const Divisor v = make_divisor((int)d);
    uint32_t ns[12] = {0u,1u,d-1u,d,d+1u,2u*d-1u,2u*d,0xffffffffu,0x7fffffffu,0x80000000u,
                       (uint32_t)((uint64_t)rand()*RAND_MAX+rand()), (uint32_t)rand()};
    for(uint32_t n: ns){ if(udiv(v,n)!=n/d){ if(nbad<5) printf("BAD udiv %u / %u got %u\n",n,d,udiv(v,n)); nbad++; } }
    if(d<(1u<<20)) for(int a=-3*(int)d-2;a<=3*(int)d+2;a+=1+(int)d/7){ int ref=a>=0?a/(int)d:-((-a+(int)d-1)/(int)d);
      if(floor_div_by(a,v)!=ref){ if(nbad<5) printf("BAD floor_div_by %d / %u\n",a,d); nbad++; } }
  }
  // the query-tile visiting order of the forward's schedule: a bijection on [0, nQ) that
  // reads the W-column grid of tiles (qt = r*W + c) column after column
  for(int nQ=1;nQ<=700;nQ+=(nQ<100?1:7)) for(int W=1;W<=90;++W){
    std::vector<char> seen(nQ,0); int pc=0, pr=-1;  // the previous tile's column and row
    for(int j=0;j<nQ;++j){ int q=qtile_visit(j,W,nQ);
      bool ok = q>=0 && q<nQ && !seen[q];
      if(ok){ seen[q]=1; const int c=q%W, r=q/W;
        ok = (c==pc && r==pr+1) || (c==pc+1 && r==0);  // down the column, or the next one from its top
        pc=c; pr=r; }
      if(!ok){ if(nbad<5) printf("BAD visit nQ %d W %d j %d -> %d\n",nQ,W,j,q); nbad++; break; } } }
  for(int trial=0; trial<trials; ++trial){
    Geom g; int layout = rand()%4;  // 3: tile-major over the padded grid
    g.padded = 0;
    if(layout==1||layout==2){ g.bt=1+rand()%3; g.bh=1+rand()%3; g.bw=1+rand()%4; g.T=g.bt*(1+rand()%3); g.Hg=g.bh*(1+rand()%3); g.Wg=g.bw*(1+rand()%4);} 
    else if(layout==0) { g.bt=g.bh=g.bw=1; g.T=1+rand()%6; g.Hg=1+rand()%8; g.Wg=1+rand()%12; }
    else { g.bt=1+rand()%3; g.bh=1+rand()%3; g.bw=1+rand()%5; g.T=1+rand()%7; g.Hg=1+rand()%7; g.Wg=1+rand()%11; }
    if(layout==2 && rand()%2){ g.bt=g.bh=g.bw=1; g.T=1+rand()%9; g.Hg=1+rand()%6; g.Wg=1+rand()%9; }
    if(focus && layout!=0 && layout!=2){ g.bw=1; g.bh=1+rand()%9; g.bt=1+rand()%2; if(layout==1){ g.T=g.bt*(1+rand()%3); g.Hg=g.bh*(1+rand()%2); g.Wg=1+rand()%9; } else { g.T=1+rand()%5; g.Hg=1+rand()%12; g.Wg=1+rand()%9; } }
    g.nT=(g.T+g.bt-1)/g.bt; g.nH=(g.Hg+g.bh-1)/g.bh; g.nW=(g.Wg+g.bw-1)/g.bw; g.HW=g.Hg*g.Wg; g.S=g.T*g.HW; g.layout=layout;
    if(layout==3){ g.layout=1; g.padded=1; g.S=g.nT*g.bt*g.nH*g.bh*g.nW*g.bw; }
    DevMask m{}; m.kind = rand()% (layout?4:3); m.sink = rand()%3; m.layout = g.layout;
    if(m.kind==1){ m.rt=rand()%5-1; m.rh=rand()%5-1; m.rw=rand()%5-1; }
    if(focus && m.kind!=2 && rand()%2) m.kind=2;
    if(m.kind==2){ m.Tw=rand()%4; m.To=rand()%5-2; m.Ts=1+rand()%5; m.Sw=rand()%5; m.So=rand()%7-3; m.Ss=1+rand()%40;
      if(focus){ int r=rand()%3; if(r==0) m.Ss=g.Wg; else if(r==1) m.Ss=g.Wg*g.Hg; else if(rand()%2) m.Ss=g.Wg*(1+rand()%3); } }
    if(m.kind==3){ m.wt=1+rand()%3; m.wh=1+rand()%3; m.ww=1+rand()%3; if(m.wt>g.nT)m.wt=g.nT; if(m.wh>g.nH)m.wh=g.nH; if(m.ww>g.nW)m.ww=g.nW;}
    g = head_geom(g, m);
    int Bq = 1+rand()%20, Bk = 1+rand()%20; if(rand()%4==0){Bq=64;Bk=64;}
    int S=g.S; std::vector<int> T(S),Y(S),X(S);
    for(int p=0;p<S;++p) pos_coords(g,p,T[p],Y[p],X[p]);
    std::vector<char> real(S, 1);
    if(layout==3){ // independent statement of the padded order: nested loops over tiles
      int p=0;
      for(int a=0;a<g.nT;++a) for(int b=0;b<g.nH;++b) for(int c=0;c<g.nW;++c)
        for(int i=0;i<g.bt;++i) for(int j=0;j<g.bh;++j) for(int l=0;l<g.bw;++l,++p){
          int t=a*g.bt+i, y=b*g.bh+j, x=c*g.bw+l;
          if(T[p]!=t||Y[p]!=y||X[p]!=x){ if(nbad<5) printf("BAD padded coords p %d\n",p); nbad++; }
          real[p] = t<g.T && y<g.Hg && x<g.Wg;
        }
      if(p!=S){ printf("BAD padded length\n"); nbad++; }
    }
    if(layout==2){ // independent statement of the position-major order
      int HW=g.Hg*g.Wg;
      for(int p=0;p<S;++p){ int t,s2; if(p<HW){t=0;s2=p;} else {t=1+(p-HW)%(g.T-1); s2=(p-HW)/(g.T-1);} 
        if(T[p]!=t||Y[p]!=s2/g.Wg||X[p]!=s2%g.Wg){ if(nbad<5) printf("BAD coords p %d\n",p); nbad++; } }
    }
    int nQ=(S+Bq-1)/Bq, nK=(S+Bk-1)/Bk;
    // boxes of every query and key range: they hold exactly the range's positions
    for(int pass=0;pass<3;++pass){ int B=pass==2?256:(pass?Bk:Bq);  // 256: the largest query tile
      for(int lo=0;lo<S;lo+=B){ int hi=std::min(S,lo+B); Box bx[256]; int nb=decompose(g,lo,hi,bx);  // at most one box per position
        long long vol=0; for(int i=0;i<nb;++i) vol+=box_volume(bx[i]);
        bool ok = nb<=11 && vol==hi-lo;
        for(int p=lo;p<hi&&ok;++p){ int in=0; for(int i=0;i<nb;++i) in += T[p]>=bx[i].t0&&T[p]<=bx[i].t1&&Y[p]>=bx[i].y0&&Y[p]<=bx[i].y1&&X[p]>=bx[i].x0&&X[p]<=bx[i].x1; ok = in==1; }
        if(!ok){ if(nbad<5) printf("BAD boxes trial %d layout %d range [%d,%d) boxes %d volume %lld\n",trial,layout,lo,hi,nb,vol); nbad++; } } }
    for(int qt=0;qt<nQ;++qt){
      Box R[11]; int nr=decompose(g,qt*Bq,std::min(S,(qt+1)*Bq),R);
      bool qpad=(qt+1)*Bq>S;
      if(g.padded) nr=clip_real(g,R,nr,qpad);
      const Box qb = nr>0 ? bounding_box(R,nr) : Box{0,0,0,0,0,0};
      for(int kt=0;kt<nK;++kt){
        const int c0=kt*Bk, c1=std::min(S,(kt+1)*Bk);
        Box C[11]; int nc=decompose(g,c0,c1,C);
        bool pad=qpad||(kt+1)*Bk>S;
        bool pad_s=pad;  // the streamed form (the kernel's) sets its own copy
        int cs = tile_class_range(g,m,pair_divs(g,m),R,nr,qb,c0,c1,pad_s);
        if(g.padded) nc=clip_real(g,C,nc,pad);
        int c = tile_class(g,m,R,nr,C,nc,pad);
        long long kept=0;
        for(int i=qt*Bq;i<(qt+1)*Bq;++i) for(int j=kt*Bk;j<(kt+1)*Bk;++j) if(i<S&&j<S&&real[i]&&real[j]&&keep_bf(g,m,T[i],Y[i],X[i],T[j],Y[j],X[j])) kept++;
        int ref = kept==0?0:(kept==(long long)Bq*Bk?1:2);
        long long kr=0; for(int j=kt*Bk;j<c1;++j) kr+=real[j];
        long long ks=0, krs=0; bool pad_c=qpad||(kt+1)*Bk>S;
        tile_counts(g,m,R,nr,c0,c1,m.kind!=2,ks,krs,pad_c);
        if(krs!=kr||pad_c!=pad){ if(nbad<5) printf("BAD real keys trial %d layout %d kt %d got %lld ref %lld\n",trial,layout,kt,krs,kr); nbad++; }
        if(m.kind!=2){ long long kb=0; for(int i=0;i<nr;++i) for(int j=0;j<nc;++j) kb+=box_pair_kept(g,m,R[i],C[j]);
          if(kb!=kept||ks!=kept){ if(nbad<5) printf("BAD box count trial %d kind %d layout %d got %lld/%lld ref %lld\n",trial,m.kind,layout,kb,ks,kept); nbad++; } }
        ntile++; if(c!=ref||cs!=ref){ if(nbad<5) printf("BAD class trial %d kind %d layout %d qt %d kt %d got %d/%d ref %d\n",trial,m.kind,layout,qt,kt,c,cs,ref); nbad++; }
      }
    }
    // element masks for tiles of 64 keys (stripe periods also as prepared divisors)
    const Divisor dss = make_divisor(m.kind==2 ? m.Ss : 1), dts = make_divisor(m.kind==2 ? m.Ts : 1);
    for(int p=0;p<S;++p){
      QueryPos q = make_query(g,m,p);
      for(int c0=0;c0<S;c0+=64){
        uint64_t bits=tile_row_mask(g,m,q,c0,64);
        if(tile_row_mask(g,m,q,c0,64,dss,dts)!=bits){ if(nmbad<5) printf("BAD divisor row mask trial %d p %d c0 %d\n",trial,p,c0); nmbad++; }
        uint64_t rb=real_key_mask(g,c0,64);
        for(int j=0;j<64;++j){ int key=c0+j; bool ref = key<S && real[key] && keep_bf(g,m,T[p],Y[p],X[p],T[key],Y[key],X[key]); bool got=(bits>>j)&1; nmask++; if(got!=ref){ if(nmbad<5) printf("BAD mask trial %d kind %d p %d key %d got %d\n",trial,m.kind,p,key,got); nmbad++; }
          bool rref = key<S && real[key]; if(((rb>>j)&1)!=rref){ if(nmbad<5) printf("BAD real mask trial %d key %d\n",trial,key); nmbad++; } }
      }
    }
  }
  printf("tiles %lld bad %lld; mask bits %lld bad %lld\n",ntile,nbad,nmask,nmbad);
  return (nbad||nmbad)?1:0;
}

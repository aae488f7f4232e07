// Exact geometry of masks over position ranges, shared by the HIP kernels.
//
// Two jobs:
//  1. Tile classification (full / boundary / empty) without an element loop.  A
//     contiguous range of executed positions is a union of at most 2n-1 "boxes",
//     products of coordinate intervals (n = 3 digits (t,y,x) in frame-major order,
//     6 digits (tile t,h,w, in-tile t,h,w) in tile-major order; in position-major
//     order the frame-0 block (digits y,x) and the rest (digits y,x,t-1) each give
//     at most 5).  Every mask kind is
//     a product of per-axis predicates of a coordinate difference (or of tile
//     coordinates, for sliding tiles), OR-ed with the key-only sink predicate.  Over
//     a pair of boxes each difference takes every value of an interval, independently
//     per axis, so "all pairs kept" and "some pair kept" reduce to interval tests:
//     a band |d| <= r, or a counting function for the periodic stripe predicate.
//  2. The element mask of a boundary tile for one query row: the key range is cut
//     into runs of constant (t, y) and contiguous x (or, past the frame-0 block of
//     position-major order, constant (y, x) and contiguous t); in each run the kept
//     keys of a box, stripe or sliding-tile mask form a few contiguous bit ranges.
//
// Mask definitions: Sparse VideoGen on TPU ("how to accelerate attention": spatial
// and temporal heads, frame-F00 sink); PSA notes, key design 1 (six-tuple stripes);
// Sliding Tile Attention explainer, method section 3 (tile-granular window).
#pragma once

#include <stdint.h>

#include "vsa_internal.h"

namespace vsa {

#define VSA_HD __host__ __device__ __forceinline__

VSA_HD int imin(int a, int b) { return a < b ? a : b; }
VSA_HD int imax(int a, int b) { return a > b ? a : b; }
VSA_HD int iabs(int a) { return a < 0 ? -a : a; }
// floor division for a possibly negative numerator and positive divisor
VSA_HD int fdiv(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

struct Box {
  int t0, t1, y0, y1, x0, x1;
};

// (t, y, x) of executed position p.
VSA_HD void pos_coords(const Geom& g, int p, int& t, int& y, int& x) {
  if (g.layout == VSA_LAYOUT_FRAME_MAJOR) {
    t = p / g.HW;
    int r = p - t * g.HW;
    y = r / g.Wg;
    x = r - y * g.Wg;
  } else if (g.layout == VSA_LAYOUT_POSITION_MAJOR) {
    int s;
    if (p < g.HW) {
      t = 0;
      s = p;
    } else {
      const int T1 = g.T - 1, q = p - g.HW;
      s = q / T1;
      t = 1 + (q - s * T1);
    }
    y = s / g.Wg;
    x = s - y * g.Wg;
  } else {
    int vol = g.bt * g.bh * g.bw;
    int tau = p / vol, io = p - tau * vol;
    int nHW = g.nH * g.nW;
    int tt = tau / nHW, r = tau - tt * nHW;
    int th = r / g.nW, tw = r - th * g.nW;
    int it = io / (g.bh * g.bw), r2 = io - it * (g.bh * g.bw);
    int ih = r2 / g.bw, iw = r2 - ih * g.bw;
    t = tt * g.bt + it;
    y = th * g.bh + ih;
    x = tw * g.bw + iw;
  }
}

// Frame-major index of the token at executed position p, or -1 where p is padding.
VSA_HD int frame_index(const Geom& g, int p) {
  int t, y, x;
  pos_coords(g, p, t, y, x);
  if (t >= g.T || y >= g.Hg || x >= g.Wg) return -1;
  return (t * g.Hg + y) * g.Wg + x;
}

// ---------------------------------------------------------------------------
// boxes of a run of executed positions
// ---------------------------------------------------------------------------
// Each order is a mixed-radix numbering with six digits, most significant first:
// frame-major (T, Hg, Wg, 1, 1, 1), tile-major (nT, nH, nW, bt, bh, bw), and the part of
// the position-major order after its frame-0 block (Hg, Wg, T-1, 1, 1, 1), whose frame-0
// block is frame-major.  Axis a is digit a times mul[a] plus digit a+3; `pm` orders
// the axes (y, x, t-1) instead of (t, y, x).
struct Order {
  int radix[6];
  int mul[3];
  bool pm;
};

VSA_HD Order main_order(const Geom& g) {
  Order o;
  if (g.layout == VSA_LAYOUT_TILE_MAJOR) {
    o.radix[0] = g.nT; o.radix[1] = g.nH; o.radix[2] = g.nW;
    o.radix[3] = g.bt; o.radix[4] = g.bh; o.radix[5] = g.bw;
    o.mul[0] = g.bt; o.mul[1] = g.bh; o.mul[2] = g.bw;
  } else {  // frame-major, and the frame-0 block of the position-major order
    o.radix[0] = g.T; o.radix[1] = g.Hg; o.radix[2] = g.Wg;
    o.radix[3] = o.radix[4] = o.radix[5] = 1;
    o.mul[0] = o.mul[1] = o.mul[2] = 1;
  }
  o.pm = false;
  return o;
}

VSA_HD Order pm_rest_order(const Geom& g) {
  Order o;
  o.radix[0] = g.Hg; o.radix[1] = g.Wg; o.radix[2] = g.T - 1;
  o.radix[3] = o.radix[4] = o.radix[5] = 1;
  o.mul[0] = o.mul[1] = o.mul[2] = 1;
  o.pm = true;
  return o;
}

// Visit the boxes of positions [lo, end) of one order, in ascending position order.
// Each box is a run of one digit with the coarser digits fixed and the finer ones full,
// taken at the coarsest digit that the running position is aligned to and whose unit
// still fits before `end` (the mixed-radix range decomposition: at most 2*6-1 boxes, at
// most 5 for three-digit orders).  The digit arrays are indexed by unrolled loop
// counters only, so on the GPU they stay in registers.
template <typename Emit>
VSA_HD void order_boxes(const Order& o, int lo, int end, Emit&& emit) {
  if (lo >= end) return;
  int W[7];  // W[k + 1]: weight of digit k
  W[6] = 1;
#pragma unroll
  for (int k = 5; k >= 0; --k) W[k] = W[k + 1] * o.radix[k];
  int d[6];
  {
    int x = lo;
#pragma unroll
    for (int k = 5; k >= 0; --k) {
      if (o.radix[k] > 1) {
        const int q = x / o.radix[k];
        d[k] = x - q * o.radix[k];
        x = q;
      } else {
        d[k] = 0;
      }
    }
  }
  int cur = lo;
#pragma nounroll
  while (cur < end) {
    const int rem = end - cur;
    int jnz = 0;  // finest nonzero digit: cur is aligned to the weight of every digit >= jnz
#pragma unroll
    for (int k = 0; k < 6; ++k)
      if (d[k] != 0) jnz = k;
    int j = 5, w = 1, r = 1, dj = 0;  // the run's digit, its weight, radix and start
#pragma unroll
    for (int k = 5; k >= 0; --k)
      if (k >= jnz && W[k + 1] <= rem) { j = k; w = W[k + 1]; r = o.radix[k]; dj = d[k]; }
    const int cnt = imin(r - dj, rem / w);
    // digits > j are zero (aligned); the box spans d..hi per digit
    int A0[3], A1[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const int h0 = a < j ? d[a] : (a == j ? d[a] + cnt - 1 : o.radix[a] - 1);
      const int h1 = a + 3 < j ? d[a + 3] : (a + 3 == j ? d[a + 3] + cnt - 1 : o.radix[a + 3] - 1);
      A0[a] = d[a] * o.mul[a] + d[a + 3];
      A1[a] = h0 * o.mul[a] + h1;
    }
    Box b;
    if (o.pm) {
      b.t0 = A0[2] + 1; b.t1 = A1[2] + 1; b.y0 = A0[0]; b.y1 = A1[0]; b.x0 = A0[1]; b.x1 = A1[1];
    } else {
      b.t0 = A0[0]; b.t1 = A1[0]; b.y0 = A0[1]; b.y1 = A1[1]; b.x0 = A0[2]; b.x1 = A1[2];
    }
    emit(b);
    cur += cnt * w;
    int carry = 0;  // digit j advances by cnt, carrying into the coarser digits
#pragma unroll
    for (int k = 5; k >= 0; --k) {
      const int v = d[k] + (k == j ? cnt : 0) + carry;
      carry = v >= o.radix[k] ? 1 : 0;
      d[k] = carry ? v - o.radix[k] : v;
    }
  }
}

// Visit the boxes of executed positions [lo, end): at most 11 for frame- and tile-major
// orders, at most 10 for position-major (frame-0 block, then the rest).  One loop over
// the (at most two) segments, so `emit` is expanded once.
template <typename Emit>
VSA_HD void for_each_box(const Geom& g, int lo, int end, Emit&& emit) {
  const bool pm = g.layout == VSA_LAYOUT_POSITION_MAJOR;
  const int nseg = (pm && lo < g.HW && end > g.HW) ? 2 : 1;
#pragma nounroll
  for (int s = 0; s < nseg; ++s) {
    const bool rest = pm && (s == 1 || lo >= g.HW);
    const Order o = rest ? pm_rest_order(g) : main_order(g);
    const int a = rest ? imax(lo, g.HW) - g.HW : lo;
    const int b = rest ? end - g.HW : (pm ? imin(end, g.HW) : end);
    order_boxes(o, a, b, emit);
  }
}

// The boxes of executed positions [lo, end) as an array (at most 11).
VSA_HD int decompose(const Geom& g, int lo, int end, Box* out) {
  int nb = 0;
  for_each_box(g, lo, end, [&](const Box& b) { out[nb++] = b; });
  return nb;
}

// Padded grid: cut a box of padded coordinates down to the real tokens; false when none
// is left.  `clipped` is set when some position was padding.
VSA_HD bool clip_box(const Geom& g, Box& c, bool& clipped) {
  const int t1 = imin(c.t1, g.T - 1), y1 = imin(c.y1, g.Hg - 1), x1 = imin(c.x1, g.Wg - 1);
  if (t1 != c.t1 || y1 != c.y1 || x1 != c.x1) clipped = true;
  if (c.t0 > t1 || c.y0 > y1 || c.x0 > x1) return false;
  c.t1 = t1; c.y1 = y1; c.x1 = x1;
  return true;
}

VSA_HD int clip_real(const Geom& g, Box* b, int n, bool& clipped) {
  int k = 0;
  for (int i = 0; i < n; ++i) {
    Box c = b[i];
    if (clip_box(g, c, clipped)) b[k++] = c;
  }
  return k;
}

VSA_HD long long box_volume(const Box& b) {
  return (long long)(b.t1 - b.t0 + 1) * (b.y1 - b.y0 + 1) * (b.x1 - b.x0 + 1);
}

// ---------------------------------------------------------------------------
// predicates over intervals of a coordinate difference
// ---------------------------------------------------------------------------
// Division by a positive divisor that stays fixed over many calls (a mask's period, the
// grid width): floor(n / d) for every 32-bit unsigned n by one multiply-high, a
// subtraction, an addition and two shifts (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, unsigned division of section 4):
// with l = ceil(log2 d), mul = floor(2^32 (2^l - d) / d) + 1.
struct Divisor {
  uint32_t d, mul;
  int s1, s2;
};

VSA_HD Divisor make_divisor(int d) {
  Divisor v;
  v.d = (uint32_t)d;
  int l = 0;
  while ((1ull << l) < (unsigned long long)v.d) ++l;
  v.mul = (uint32_t)(((1ull << 32) * ((1ull << l) - v.d)) / v.d + 1);
  v.s1 = l < 1 ? l : 1;
  v.s2 = l > 1 ? l - 1 : 0;
  return v;
}

VSA_HD uint32_t udiv(const Divisor& v, uint32_t n) {
  const uint32_t t = (uint32_t)(((uint64_t)n * v.mul) >> 32);
  return (t + ((n - t) >> v.s1)) >> v.s2;
}

// floor(a / d) for a possibly negative a
VSA_HD int floor_div_by(int a, const Divisor& v) {
  return a >= 0 ? (int)udiv(v, (uint32_t)a) : -(int)udiv(v, (uint32_t)(-a) + v.d - 1);
}

// The divisors of one (head geometry, mask) pair's interval tests.
struct PairDivs {
  Divisor ts, ss, wg;
  int per;  // stripes: rows after which a row's spatial differences repeat mod Ss
};

// #{v in [0, m] : v mod P < w}, m >= -1
VSA_HD int band_prefix(int m, const Divisor& P, int w) {
  if (m < 0) return 0;
  const int wc = imin(w, (int)P.d);
  const uint32_t x = (uint32_t)m + 1u;
  const uint32_t q = udiv(P, x);
  return (int)q * wc + imin((int)(x - q * P.d), wc);
}
// #{u in [a, b] : (|u| mod P) < w}
VSA_HD int band_count(int a, int b, const Divisor& P, int w) {
  if (a > b || w <= 0) return 0;
  int c = 0;
  if (b >= 0) {
    int lo = imax(a, 0);
    c += band_prefix(b, P, w) - band_prefix(lo - 1, P, w);
  }
  if (a < 0) {
    int lo = imax(-b, 1), hi = -a;
    c += band_prefix(hi, P, w) - band_prefix(lo - 1, P, w);
  }
  return c;
}

// |d| <= r over d in [a, b]; r < 0 = unbounded
VSA_HD void radius_test(int a, int b, int r, bool& all, bool& any) {
  if (r < 0) { all = true; any = true; return; }
  all = (a >= -r) && (b <= r);
  any = (a <= r) && (b >= -r);
}

// (|d - o| mod P) <= w - 1 over d in [a, b]
VSA_HD void periodic_test(int a, int b, int o, const Divisor& P, int w, bool& all, bool& any) {
  int c = band_count(a - o, b - o, P, w);
  all = (c == b - a + 1);
  any = (c > 0);
}

VSA_HD int sta_start(int a, int w, int n) { return imin(imax(a - w / 2, 0), imax(n - w, 0)); }

// sliding tile window on one axis: tile coords a in [a0, a1] (queries), b in [b0, b1]
VSA_HD void sta_test(int a0, int a1, int b0, int b1, int w, int n, bool& all, bool& any) {
  int s0 = sta_start(a0, w, n), s1 = sta_start(a1, w, n);
  all = (s1 <= b0) && (b1 <= s0 + w - 1);
  any = (s0 <= b1) && (s1 + w - 1 >= b0);
}

VSA_HD bool s_contiguous(const Geom& g, const Box& b) {
  return b.y0 == b.y1 || (b.x0 == 0 && b.x1 == g.Wg - 1);
}

VSA_HD int igcd(int a, int b) {
  while (b) { const int r = a % b; a = b; b = r; }
  return a;
}

VSA_HD int floor_div(int a, int b) {  // b > 0
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

VSA_HD PairDivs pair_divs(const Geom& g, const DevMask& m) {
  const bool stripe = m.kind == VSA_MASK_STRIPE;
  PairDivs v;
  v.ts = make_divisor(stripe ? m.Ts : 1);
  v.ss = make_divisor(stripe ? m.Ss : 1);
  v.wg = make_divisor(g.Wg);
  v.per = stripe ? m.Ss / igcd(g.Wg, m.Ss) : 1;
  return v;
}

// Stripe test over the spatial differences of two boxes that are not runs of s: the
// rows dy in [dy0, dy1] each contribute the interval d = dy*Wg + [dx0, dx1] - So, kept
// where (|d| mod Ss) < Sw.  While a row's interval lies wholly below 0, or wholly at or
// above 0, moving dy by Ss / gcd(Wg, Ss) moves d by a multiple of Ss and repeats the
// row's result, so each of those two ranges needs at most one period of rows; only the
// rows whose interval contains 0 are tested one by one.
VSA_HD void stripe_rows_test(const Geom& g, const DevMask& m, const PairDivs& dv, int dy0, int dy1, int dx0,
                             int dx1, bool& all, bool& any) {
  // every |d| below Ss (no wrap): kept iff |d| <= Sw - 1, so "any" asks whether some row
  // interval meets [-(Sw-1), Sw-1] and "all" whether the extremes stay inside it
  const int dmin = dy0 * g.Wg + dx0 - m.So, dmax = dy1 * g.Wg + dx1 - m.So;
  if (dmin > -m.Ss && dmax < m.Ss) {
    const int w = m.Sw - 1;
    if (w < 0) { all = false; any = false; return; }
    const int A = dx0 - m.So, B = dx1 - m.So;  // row dy spans [A + dy*Wg, B + dy*Wg]
    const int lo = imax(dy0, -floor_div_by(w + B, dv.wg)), hi = imin(dy1, floor_div_by(w - A, dv.wg));
    any = lo <= hi;
    all = dmin >= -w && dmax <= w;
    return;
  }
  all = true;
  any = false;
  const int per = dv.per;
  // rows with d < 0 throughout: dy*Wg + dx1 - So < 0; rows with d >= 0 throughout:
  // dy*Wg + dx0 - So >= 0
  const int neg_end = imin(dy1, floor_div_by(m.So - dx1 - 1, dv.wg));
  const int pos_begin = imax(dy0, -floor_div_by(dx0 - m.So, dv.wg));
  auto row = [&](int dy) {
    bool a, n;
    periodic_test(dy * g.Wg + dx0, dy * g.Wg + dx1, m.So, dv.ss, m.Sw, a, n);
    all = all && a;
    any = any || n;
  };
  for (int dy = dy0; dy <= imin(neg_end, dy0 + per - 1); ++dy) row(dy);
  for (int dy = imax(dy0, neg_end + 1); dy <= imin(dy1, pos_begin - 1); ++dy) row(dy);
  for (int dy = pos_begin; dy <= imin(dy1, pos_begin + per - 1); ++dy) row(dy);
}

// all / any kept over query box r x key box c for the mask without its sink.
VSA_HD void box_pair_test(const Geom& g, const DevMask& m, const PairDivs& dv, const Box& r, const Box& c,
                          bool& all, bool& any) {
  switch (m.kind) {
    case VSA_MASK_ALL:
      all = true; any = true;
      return;
    case VSA_MASK_BOX: {
      bool a0, n0, a1, n1, a2, n2;
      radius_test(c.t0 - r.t1, c.t1 - r.t0, m.rt, a0, n0);
      radius_test(c.y0 - r.y1, c.y1 - r.y0, m.rh, a1, n1);
      radius_test(c.x0 - r.x1, c.x1 - r.x0, m.rw, a2, n2);
      all = a0 && a1 && a2;
      any = n0 && n1 && n2;
      return;
    }
    case VSA_MASK_STRIPE: {
      bool at, nt;
      periodic_test(c.t0 - r.t1, c.t1 - r.t0, m.To, dv.ts, m.Tw, at, nt);
      if (!nt) {  // no key frame passes the temporal test: nothing kept
        all = false;
        any = false;
        return;
      }
      bool as = true, ns = false;
      if (s_contiguous(g, r) && s_contiguous(g, c)) {
        int sq0 = r.y0 * g.Wg + r.x0, sq1 = r.y1 * g.Wg + r.x1;
        int sk0 = c.y0 * g.Wg + c.x0, sk1 = c.y1 * g.Wg + c.x1;
        periodic_test(sk0 - sq1, sk1 - sq0, m.So, dv.ss, m.Sw, as, ns);
      } else {
        stripe_rows_test(g, m, dv, c.y0 - r.y1, c.y1 - r.y0, c.x0 - r.x1, c.x1 - r.x0, as, ns);
      }
      all = at && as;
      any = nt && ns;
      return;
    }
    case VSA_MASK_STA: {
      bool a0, n0, a1, n1, a2, n2;
      sta_test(r.t0 / g.bt, r.t1 / g.bt, c.t0 / g.bt, c.t1 / g.bt, m.wt, g.nT, a0, n0);
      sta_test(r.y0 / g.bh, r.y1 / g.bh, c.y0 / g.bh, c.y1 / g.bh, m.wh, g.nH, a1, n1);
      sta_test(r.x0 / g.bw, r.x1 / g.bw, c.x0 / g.bw, c.x1 / g.bw, m.ww, g.nW, a2, n2);
      all = a0 && a1 && a2;
      any = n0 && n1 && n2;
      return;
    }
    default:
      all = false; any = false;
      return;
  }
}

// #{(a, b) : a in [a0, a1], b in [b0, b1], |b - a| <= r}; r < 0 = unbounded
VSA_HD long long radius_pairs(int a0, int a1, int b0, int b1, int r) {
  if (r < 0) return (long long)(a1 - a0 + 1) * (b1 - b0 + 1);
  long long n = 0;
  for (int a = a0; a <= a1; ++a) n += imax(0, imin(b1, a + r) - imax(b0, a - r) + 1);
  return n;
}

// #{(a, b) : a in [a0, a1], b in [b0, b1], b's tile inside the sliding window of a's}
VSA_HD long long window_pairs(int a0, int a1, int b0, int b1, int bsz, int w, int n) {
  long long cnt = 0;
  for (int a = a0; a <= a1; ++a) {
    const int s = sta_start(a / bsz, w, n);
    cnt += imax(0, imin(b1, (s + w) * bsz - 1) - imax(b0, s * bsz) + 1);
  }
  return cnt;
}

// Kept pairs of query box r x key box c (sink included) for the kinds whose predicate
// is a product over the three axes (ALL, BOX, STA); -1 for the others.
VSA_HD long long box_pair_kept(const Geom& g, const DevMask& m, const Box& r, Box c) {
  if (m.kind == VSA_MASK_STRIPE) return -1;
  const long long nq = box_volume(r);
  long long kept = 0;
  if (c.t0 < m.sink) {  // key frames below the sink: every pair kept
    const int t1 = imin(c.t1, m.sink - 1);
    kept += nq * (long long)(t1 - c.t0 + 1) * (c.y1 - c.y0 + 1) * (c.x1 - c.x0 + 1);
    if (t1 == c.t1) return kept;
    c.t0 = t1 + 1;
  }
  switch (m.kind) {
    case VSA_MASK_ALL:
      return kept + nq * box_volume(c);
    case VSA_MASK_BOX:
      return kept + radius_pairs(r.t0, r.t1, c.t0, c.t1, m.rt) * radius_pairs(r.y0, r.y1, c.y0, c.y1, m.rh) *
                        radius_pairs(r.x0, r.x1, c.x0, c.x1, m.rw);
    case VSA_MASK_STA:
      return kept + window_pairs(r.t0, r.t1, c.t0, c.t1, g.bt, m.wt, g.nT) *
                        window_pairs(r.y0, r.y1, c.y0, c.y1, g.bh, m.wh, g.nH) *
                        window_pairs(r.x0, r.x1, c.x0, c.x1, g.bw, m.ww, g.nW);
    default:
      return -1;
  }
}

// Frame range [q0, q1] covered by boxes R[nr] (nr > 0).
VSA_HD void frame_range(const Box* R, int nr, int& q0, int& q1) {
  q0 = R[0].t0;
  q1 = R[0].t1;
  for (int i = 1; i < nr; ++i) { q0 = imin(q0, R[i].t0); q1 = imax(q1, R[i].t1); }
}

// Add key box c to a tile pair's class: `all` stays true while every pair seen is kept,
// `any` turns true once one is.  R[nr] are the query boxes, [q0, q1] their frame range.
VSA_HD void class_add(const Geom& g, const DevMask& m, const PairDivs& dv, const Box* R, int nr, int q0, int q1,
                      Box c, bool& all, bool& any) {
  if (nr == 0) return;
  // Frame pre-test: with no sink frame in c and no pair of frames passing the temporal
  // part of the mask, no pair with c is kept.
  if (c.t0 >= m.sink && (m.kind == VSA_MASK_STRIPE || (m.kind == VSA_MASK_BOX && m.rt >= 0))) {
    bool a, n;
    if (m.kind == VSA_MASK_STRIPE)
      periodic_test(c.t0 - q1, c.t1 - q0, m.To, dv.ts, m.Tw, a, n);
    else
      radius_test(c.t0 - q1, c.t1 - q0, m.rt, a, n);
    if (!n) {
      all = false;
      return;
    }
  }
  if (c.t0 < m.sink) {  // key frames below the sink are kept for every query
    any = true;
    if (c.t1 < m.sink) return;
    c.t0 = m.sink;
  }
  for (int i = 0; i < nr; ++i) {
    bool a, n;
    box_pair_test(g, m, dv, R[i], c, a, n);
    all = all && a;
    any = any || n;
    if (!all && any) return;
  }
}

VSA_HD int class_of(bool all, bool any, bool padded) {
  if (!any) return VSA_TILE_EMPTY;
  return (all && !padded) ? VSA_TILE_FULL : VSA_TILE_BOUNDARY;
}

// Tile class of query boxes R[nr] x key boxes C[nc] (padded: the tile reaches past S).
VSA_HD int tile_class(const Geom& g, const DevMask& m, const Box* R, int nr, const Box* C, int nc,
                      bool padded) {
  bool all = true, any = false;
  if (nr == 0) return VSA_TILE_EMPTY;
  int q0, q1;
  frame_range(R, nr, q0, q1);
  const PairDivs dv = pair_divs(g, m);
  for (int j = 0; j < nc && (all || !any); ++j) class_add(g, m, dv, R, nr, q0, q1, C[j], all, any);
  return class_of(all, any, padded);
}

// Tile class of query boxes R[nr] (real tokens, frame range [q0, q1]) x the key tile of
// executed positions [c0, c1), whose boxes are visited one at a time and clipped to the
// real grid.  `padded`: the query tile or the key tile reaches past S.
VSA_HD int tile_class_range(const Geom& g, const DevMask& m, const PairDivs& dv, const Box* R, int nr, int q0,
                            int q1, int c0, int c1, bool padded) {
  bool all = true, any = false;
  if (nr == 0) return VSA_TILE_EMPTY;
  for_each_box(g, c0, c1, [&](Box c) {
    if (!all && any) return;  // boundary whatever follows
    if (g.padded && !clip_box(g, c, padded)) return;
    class_add(g, m, dv, R, nr, q0, q1, c, all, any);
  });
  return class_of(all, any, padded);
}

// Real keys of the key tile [c0, c1) and, for masks that are a product over the axes,
// its pairs kept with query boxes R[nr].  `padded` is set when a key position is padding.
VSA_HD void tile_counts(const Geom& g, const DevMask& m, const Box* R, int nr, int c0, int c1, bool by_boxes,
                        long long& kept, long long& k_real, bool& padded) {
  kept = 0;
  k_real = 0;
  for_each_box(g, c0, c1, [&](Box c) {
    if (g.padded && !clip_box(g, c, padded)) return;
    k_real += box_volume(c);
    if (by_boxes)
      for (int i = 0; i < nr; ++i) kept += box_pair_kept(g, m, R[i], c);
  });
}

// ---------------------------------------------------------------------------
// element mask of one query row over a key tile (bit i = key c0 + i kept)
// ---------------------------------------------------------------------------
struct QueryPos {
  int t, y, x, s;     // coordinates, s = y*Wg + x
  int st, sh, sw;     // STA window starts (tile coordinates)
  uint64_t tkeep;     // stripe masks with T <= 64: bit t set iff key frame t passes the
                      // temporal stripe test for this query
};

// The temporal stripe test of key frame t for query frame tq.
VSA_HD bool stripe_frame_kept(const DevMask& m, int t, int tq) { return (iabs(t - tq - m.To) % m.Ts) < m.Tw; }

VSA_HD QueryPos make_query(const Geom& g, const DevMask& m, int p) {
  QueryPos q;
  pos_coords(g, p, q.t, q.y, q.x);
  q.s = q.y * g.Wg + q.x;
  q.st = q.sh = q.sw = 0;
  q.tkeep = 0;
  if (m.kind == VSA_MASK_STRIPE && g.T <= 64) {
    for (int t = 0; t < g.T; ++t)
      if (stripe_frame_kept(m, t, q.t)) q.tkeep |= 1ull << t;
  }
  if (m.kind == VSA_MASK_STA) {
    q.st = sta_start(q.t / g.bt, m.wt, g.nT);
    q.sh = sta_start(q.y / g.bh, m.wh, g.nH);
    q.sw = sta_start(q.x / g.bw, m.ww, g.nW);
  }
  return q;
}

VSA_HD uint64_t bit_range(int lo, int hi) {  // bits lo..hi inclusive, 0 <= lo <= hi < 64
  uint64_t ones = ~0ull >> (63 - (hi - lo));
  return ones << lo;
}

// Bits off + (u - ua) for the u in [ua, ub] with (|u| mod P) < w (the stripe predicate
// along one run of keys).
VSA_HD uint64_t periodic_bits(int ua, int ub, int P, int w, int off) {
  // one division per sign of u: the periods are stepped from the first one
  uint64_t bits = 0;
  if (ub >= 0) {
    int lo = imax(ua, 0);
    for (int base = (lo / P) * P; base <= ub; base += P) {
      int a = imax(lo, base), b = imin(ub, base + w - 1);
      if (a <= b) bits |= bit_range(off + a - ua, off + b - ua);
    }
  }
  if (ua < 0) {
    int lo = imax(-ub, 1), hi = -ua;  // |u| in [lo, hi]
    for (int base = (lo / P) * P; base <= hi; base += P) {
      int a = imax(lo, base), b = imin(hi, base + w - 1);
      if (a <= b) bits |= bit_range(off - b - ua, off - a - ua);
    }
  }
  return bits;
}

// kept keys of a run (fixed t, y; x in [x0, x1]; bit of x0 is off) for query q
VSA_HD uint64_t run_mask(const Geom& g, const DevMask& m, const QueryPos& q, int t, int y, int x0,
                         int x1, int off) {
  if (g.padded) {  // padding keys are never kept
    if (t >= g.T || y >= g.Hg || x0 >= g.Wg) return 0;
    x1 = imin(x1, g.Wg - 1);
  }
  if (t < m.sink || m.kind == VSA_MASK_ALL) return bit_range(off, off + x1 - x0);
  switch (m.kind) {
    case VSA_MASK_BOX: {
      if (m.rt >= 0 && iabs(t - q.t) > m.rt) return 0;
      if (m.rh >= 0 && iabs(y - q.y) > m.rh) return 0;
      int lo = x0, hi = x1;
      if (m.rw >= 0) { lo = imax(lo, q.x - m.rw); hi = imin(hi, q.x + m.rw); }
      return lo <= hi ? bit_range(off + lo - x0, off + hi - x0) : 0;
    }
    case VSA_MASK_STRIPE: {
      if (g.T <= 64 ? !((q.tkeep >> t) & 1) : !stripe_frame_kept(m, t, q.t)) return 0;
      // u = s_k - s_q - So over the run; kept where (|u| mod Ss) < Sw
      const int ubase = y * g.Wg - q.s - m.So;  // u = x + ubase
      return periodic_bits(x0 + ubase, x1 + ubase, m.Ss, m.Sw, off);
    }
    case VSA_MASK_STA: {
      int at = t / g.bt, ay = y / g.bh;
      if (at < q.st || at >= q.st + m.wt) return 0;
      if (ay < q.sh || ay >= q.sh + m.wh) return 0;
      int lo = imax(x0, q.sw * g.bw), hi = imin(x1, (q.sw + m.ww) * g.bw - 1);
      return lo <= hi ? bit_range(off + lo - x0, off + hi - x0) : 0;
    }
    default:
      return 0;
  }
}

// kept keys of a frame run of position-major order (fixed y, x; t in [t0, t1]; bit of
// t0 is off) for query q
VSA_HD uint64_t run_mask_t(const Geom& g, const DevMask& m, const QueryPos& q, int t0, int t1, int y,
                           int x, int off) {
  uint64_t bits = 0;
  if (t0 < m.sink) {  // sink frames are kept for every query
    const int hi = imin(t1, m.sink - 1);
    bits = bit_range(off, off + hi - t0);
    if (hi == t1) return bits;
    off += hi + 1 - t0;
    t0 = hi + 1;
  }
  switch (m.kind) {
    case VSA_MASK_ALL:
      return bits | bit_range(off, off + t1 - t0);
    case VSA_MASK_BOX: {
      if (m.rh >= 0 && iabs(y - q.y) > m.rh) return bits;
      if (m.rw >= 0 && iabs(x - q.x) > m.rw) return bits;
      int lo = t0, hi = t1;
      if (m.rt >= 0) { lo = imax(lo, q.t - m.rt); hi = imin(hi, q.t + m.rt); }
      return lo <= hi ? bits | bit_range(off + lo - t0, off + hi - t0) : bits;
    }
    case VSA_MASK_STRIPE: {
      const int ds = iabs(y * g.Wg + x - q.s - m.So);
      if ((ds < m.Ss ? ds : ds % m.Ss) >= m.Sw) return bits;
      if (g.T <= 64)  // frames t0 .. t1 of the precomputed temporal test
        return bits | (((q.tkeep >> t0) & (~0ull >> (63 - (t1 - t0)))) << off);
      // v = t_k - t_q - To over the run; kept where (|v| mod Ts) < Tw
      const int vbase = -q.t - m.To;
      return bits | periodic_bits(t0 + vbase, t1 + vbase, m.Ts, m.Tw, off);
    }
    case VSA_MASK_STA: {
      const int ay = y / g.bh, ax = x / g.bw;
      if (ay < q.sh || ay >= q.sh + m.wh || ax < q.sw || ax >= q.sw + m.ww) return bits;
      const int lo = imax(t0, q.st * g.bt), hi = imin(t1, (q.st + m.wt) * g.bt - 1);
      return lo <= hi ? bits | bit_range(off + lo - t0, off + hi - t0) : bits;
    }
    default:
      return bits;
  }
}

// kept keys of a column run of tile-major order over tiles one column wide (fixed t, x;
// y in [y0, y1]; bit of y0 is off) for query q
VSA_HD uint64_t run_mask_y(const Geom& g, const DevMask& m, const QueryPos& q, int t, int x, int y0, int y1,
                           int off) {
  if (g.padded) {  // padding keys are never kept
    if (t >= g.T || x >= g.Wg || y0 >= g.Hg) return 0;
    y1 = imin(y1, g.Hg - 1);
  }
  if (t < m.sink || m.kind == VSA_MASK_ALL) return bit_range(off, off + y1 - y0);
  switch (m.kind) {
    case VSA_MASK_BOX: {
      if (m.rt >= 0 && iabs(t - q.t) > m.rt) return 0;
      if (m.rw >= 0 && iabs(x - q.x) > m.rw) return 0;
      int lo = y0, hi = y1;
      if (m.rh >= 0) { lo = imax(lo, q.y - m.rh); hi = imin(hi, q.y + m.rh); }
      return lo <= hi ? bit_range(off + lo - y0, off + hi - y0) : 0;
    }
    case VSA_MASK_STRIPE: {
      if (g.T <= 64 ? !((q.tkeep >> t) & 1) : !stripe_frame_kept(m, t, q.t)) return 0;
      if (m.Sw <= 0) return 0;
      // u = s_k - s_q - So steps by Wg along the run; kept where (|u| mod Ss) < Sw.
      uint64_t bits = 0;
      int u = y0 * g.Wg + x - q.s - m.So;
      const int u1 = u + (y1 - y0) * g.Wg;
      if (u > -m.Ss && u1 < m.Ss) {  // no wrap: kept iff |u| <= Sw - 1, one range of rows
        const int w = m.Sw - 1, c = u - y0 * g.Wg;  // u = y*Wg + c
        const int lo = imax(y0, -floor_div(w + c, g.Wg)), hi = imin(y1, floor_div(w - c, g.Wg));
        return lo <= hi ? bit_range(off + lo - y0, off + hi - y0) : 0;
      }
      const int step = g.Wg % m.Ss;
      if (step == 0) {  // the residue is fixed on each side of u = 0
        const int yb = imin(imax(y0, -floor_div(x - q.s - m.So, g.Wg)), y1 + 1);  // first row with u >= 0
        if (yb > y0 && (iabs(u) % m.Ss) < m.Sw) bits |= bit_range(off, off + yb - 1 - y0);
        if (yb <= y1 && ((yb * g.Wg + x - q.s - m.So) % m.Ss) < m.Sw) bits |= bit_range(off + yb - y0, off + y1 - y0);
        return bits;
      }
      // otherwise the residue is carried from row to row (one division per sign of u)
      int y = y0;
      if (u < 0) {
        int r = (-u) % m.Ss;  // |u| mod Ss, |u| falling by Wg per row
        for (; y <= y1 && u < 0; ++y, u += g.Wg) {
          if (r < m.Sw) bits |= 1ull << (off + y - y0);
          r -= step;
          if (r < 0) r += m.Ss;
        }
      }
      if (y <= y1) {
        int r = u % m.Ss;  // u >= 0 from here on
        for (; y <= y1; ++y) {
          if (r < m.Sw) bits |= 1ull << (off + y - y0);
          r += step;
          if (r >= m.Ss) r -= m.Ss;
        }
      }
      return bits;
    }
    case VSA_MASK_STA: {
      const int at = t / g.bt, ax = x / g.bw;
      if (at < q.st || at >= q.st + m.wt || ax < q.sw || ax >= q.sw + m.ww) return 0;
      const int lo = imax(y0, q.sh * g.bh), hi = imin(y1, (q.sh + m.wh) * g.bh - 1);
      return lo <= hi ? bit_range(off + lo - y0, off + hi - y0) : 0;
    }
    default:
      return 0;
  }
}

// Run cursor over executed positions: advances through maximal runs of constant
// (t, y) with contiguous x.
struct RunCursor {
  int p;                 // current position
  int t, y, x;           // its coordinates
  int tt, th, tw, it, ih, iw;  // tile-major digits
};

VSA_HD RunCursor run_begin(const Geom& g, int p) {
  RunCursor c;
  c.p = p;
  if (g.layout != VSA_LAYOUT_TILE_MAJOR) {
    pos_coords(g, p, c.t, c.y, c.x);
    c.tt = c.th = c.tw = c.it = c.ih = c.iw = 0;
  } else {
    int vol = g.bt * g.bh * g.bw;
    int tau = p / vol, io = p - tau * vol;
    int nHW = g.nH * g.nW;
    c.tt = tau / nHW;
    int r = tau - c.tt * nHW;
    c.th = r / g.nW;
    c.tw = r - c.th * g.nW;
    c.it = io / (g.bh * g.bw);
    int r2 = io - c.it * (g.bh * g.bw);
    c.ih = r2 / g.bw;
    c.iw = r2 - c.ih * g.bw;
    c.t = c.tt * g.bt + c.it;
    c.y = c.th * g.bh + c.ih;
    c.x = c.tw * g.bw + c.iw;
  }
  return c;
}

// Frame- and tile-major orders: every run is along x.
VSA_HD int run_len_ft(const Geom& g, const RunCursor& c, int end) {
  return imin(g.layout == VSA_LAYOUT_TILE_MAJOR ? g.bw - c.iw : g.Wg - c.x, end - c.p);
}

VSA_HD void run_advance_ft(const Geom& g, RunCursor& c, int len) {
  c.p += len;
  if (g.layout == VSA_LAYOUT_FRAME_MAJOR) {
    c.x += len;
    if (c.x >= g.Wg) {
      c.x = 0;
      if (++c.y >= g.Hg) { c.y = 0; ++c.t; }
    }
  } else {
    c.iw += len;
    if (c.iw >= g.bw) {
      c.iw = 0;
      if (++c.ih >= g.bh) {
        c.ih = 0;
        if (++c.it >= g.bt) {
          c.it = 0;
          if (++c.tw >= g.nW) {
            c.tw = 0;
            if (++c.th >= g.nH) { c.th = 0; ++c.tt; }
          }
        }
      }
    }
    c.t = c.tt * g.bt + c.it;
    c.y = c.th * g.bh + c.ih;
    c.x = c.tw * g.bw + c.iw;
  }
}

// Position-major order: runs along x inside the frame-0 block, then along t (frames
// 1 .. T-1 of one spatial position).
VSA_HD bool run_along_t(const Geom& g, const RunCursor& c) { return c.p >= g.HW; }

VSA_HD int run_len_pm(const Geom& g, const RunCursor& c, int end) {
  return imin(run_along_t(g, c) ? g.T - c.t : g.Wg - c.x, end - c.p);
}

VSA_HD void run_advance_pm(const Geom& g, RunCursor& c, int len) {
  if (run_along_t(g, c)) {
    c.t += len;
    if (c.t >= g.T) {
      c.t = 1;
      if (++c.x >= g.Wg) { c.x = 0; ++c.y; }
    }
  } else {
    c.x += len;
    if (c.x >= g.Wg) {
      c.x = 0;
      if (++c.y >= g.Hg) { c.y = 0; c.t = 1; }  // frame-0 block done: position 0, frame 1
    }
  }
  c.p += len;
}

// keys [c0, c0 + nbits) that are real tokens: before S, and not padding of a padded
// grid (the only element mask of a tile-aligned list)
VSA_HD uint64_t real_key_mask(const Geom& g, int c0, int nbits) {
  const int end = imin(c0 + nbits, g.S);
  if (end <= c0) return 0ull;
  if (!g.padded) return bit_range(0, end - c0 - 1);
  uint64_t bits = 0;
  RunCursor c = run_begin(g, c0);
  while (c.p < end) {
    const int len = run_len_ft(g, c, end);
    if (c.t < g.T && c.y < g.Hg && c.x < g.Wg) {
      const int x1 = imin(c.x + len - 1, g.Wg - 1);
      bits |= bit_range(c.p - c0, c.p - c0 + x1 - c.x);
    }
    run_advance_ft(g, c, len);
  }
  return bits;
}

// Keep bits of keys [c0, min(c0 + nbits, S)) for query q (nbits <= 64): one loop for
// the frame- and tile-major orders, one for position-major, chosen once per call so that
// neither carries the other's per-run tests.
VSA_HD uint64_t tile_row_mask_ft(const Geom& g, const DevMask& m, const QueryPos& q, int c0, int nbits) {
  const int end = imin(c0 + nbits, g.S);
  uint64_t bits = 0;
  RunCursor c = run_begin(g, c0);
  if (g.layout == VSA_LAYOUT_TILE_MAJOR && g.bw == 1 && g.bh > 1) {
    // tiles one column wide: x is fixed inside a tile, so the runs go along y
    while (c.p < end) {
      const int len = imin(g.bh - c.ih, end - c.p);
      bits |= run_mask_y(g, m, q, c.t, c.x, c.y, c.y + len - 1, c.p - c0);
      c.p += len;
      c.ih += len;
      if (c.ih >= g.bh) {
        c.ih = 0;
        if (++c.it >= g.bt) {
          c.it = 0;
          if (++c.tw >= g.nW) {
            c.tw = 0;
            if (++c.th >= g.nH) { c.th = 0; ++c.tt; }
          }
        }
      }
      c.t = c.tt * g.bt + c.it;
      c.y = c.th * g.bh + c.ih;
      c.x = c.tw;  // bw = 1
    }
    return bits;
  }
  while (c.p < end) {
    const int len = run_len_ft(g, c, end);
    bits |= run_mask(g, m, q, c.t, c.y, c.x, c.x + len - 1, c.p - c0);
    run_advance_ft(g, c, len);
  }
  return bits;
}

VSA_HD uint64_t tile_row_mask_pm(const Geom& g, const DevMask& m, const QueryPos& q, int c0, int nbits) {
  const int end = imin(c0 + nbits, g.S);
  uint64_t bits = 0;
  RunCursor c = run_begin(g, c0);
  while (c.p < end) {
    const int len = run_len_pm(g, c, end);
    if (run_along_t(g, c))
      bits |= run_mask_t(g, m, q, c.t, c.t + len - 1, c.y, c.x, c.p - c0);
    else
      bits |= run_mask(g, m, q, c.t, c.y, c.x, c.x + len - 1, c.p - c0);
    run_advance_pm(g, c, len);
  }
  return bits;
}

VSA_HD uint64_t tile_row_mask(const Geom& g, const DevMask& m, const QueryPos& q, int c0, int nbits) {
  return g.layout == VSA_LAYOUT_POSITION_MAJOR ? tile_row_mask_pm(g, m, q, c0, nbits)
                                               : tile_row_mask_ft(g, m, q, c0, nbits);
}

}  // namespace vsa

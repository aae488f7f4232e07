// Tile classification (full / boundary / empty) without an element loop.
//
// A contiguous range of executed positions is a union of at most 2n-1 "boxes",
// products of coordinate intervals (n = 3 digits (t,y,x) in frame-major order, 6
// digits (tile t,h,w, in-tile t,h,w) in tile-major order; in position-major order the
// frame-0 block (digits y,x) and the rest (digits y,x,t-1) each give at most 5).  Every
// mask kind is a product of per-axis predicates of a coordinate difference (or of tile
// coordinates, for sliding tiles), OR-ed with the key-only sink predicate.  Over a pair
// of boxes each difference takes every value of an interval, independently per axis,
// so "all pairs kept" and "some pair kept" reduce to interval tests: a band |d| <= r,
// or a counting function for the periodic stripe predicate.
//
// Mask definitions: Sparse VideoGen on TPU ("how to accelerate attention"); PSA
// notes, key design 1; Sliding Tile Attention explainer, method section 3.  Tile
// classes: Sparse VideoGen on TPU, "logical sparsity is not physical sparsity".
#pragma once

#include "vsa_geom.h"

namespace vsa {

struct Box {
  int t0, t1, y0, y1, x0, x1;
};

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
// floor(a / d) for a possibly negative a
VSA_HD int floor_div_by(int a, const Divisor& v) {
  return a >= 0 ? (int)udiv(v, (uint32_t)a) : -(int)udiv(v, (uint32_t)(-a) + v.d - 1);
}

// The divisors of one (head geometry, mask) pair's interval tests.
struct PairDivs {
  Divisor ts, ss, wg;
  int per;      // stripes: rows after which a row's spatial differences repeat mod Ss
  bool x_only;  // stripes with Ss dividing Wg: s differences mod Ss depend on x alone
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
// Whether some u in [a, b] lies within w - 1 of a multiple of P (w <= 0: none).
VSA_HD bool near_multiple(int a, int b, const Divisor& P, int w) {
  if (w <= 0 || a > b) return false;
  return floor_div_by(b + w - 1, P) >= -floor_div_by(-(a - w + 1), P);
}

VSA_HD void periodic_test(int a, int b, int o, const Divisor& P, int w, bool& all, bool& any) {
  int c = band_count(a - o, b - o, P, w);
  all = (c == b - a + 1);
  any = (c > 0);
}

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

VSA_HD PairDivs pair_divs(const Geom& g, const DevMask& m) {
  const bool stripe = m.kind == VSA_MASK_STRIPE;
  PairDivs v;
  v.ts = make_divisor(stripe ? m.Ts : 1);
  v.ss = make_divisor(stripe ? m.Ss : 1);
  v.wg = make_divisor(g.Wg);
  v.per = stripe ? m.Ss / igcd(g.Wg, m.Ss) : 1;
  v.x_only = stripe && g.Wg % m.Ss == 0;
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

// all / any kept over query box r x key box c for the mask without its sink.  t_all:
// every frame pair of r x c is known to pass the temporal part (its test is skipped).
VSA_HD void box_pair_test(const Geom& g, const DevMask& m, const PairDivs& dv, const Box& r, const Box& c,
                          bool& all, bool& any, bool t_all = false) {
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
      bool at = true, nt = true;
      if (!t_all) periodic_test(c.t0 - r.t1, c.t1 - r.t0, m.To, dv.ts, m.Tw, at, nt);
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

// Bounding box of boxes R[nr] (nr > 0).
VSA_HD Box bounding_box(const Box* R, int nr) {
  Box q = R[0];
  for (int i = 1; i < nr; ++i) {
    q.t0 = imin(q.t0, R[i].t0); q.t1 = imax(q.t1, R[i].t1);
    q.y0 = imin(q.y0, R[i].y0); q.y1 = imax(q.y1, R[i].y1);
    q.x0 = imin(q.x0, R[i].x0); q.x1 = imax(q.x1, R[i].x1);
  }
  return q;
}

// Add key box c to a tile pair's class: `all` stays true while every pair seen is kept,
// `any` turns true once one is.  R[nr] are the query boxes, qb their bounding box.
VSA_HD void class_add(const Geom& g, const DevMask& m, const PairDivs& dv, const Box* R, int nr, const Box& qb,
                      Box c, bool& all, bool& any) {
  if (nr == 0) return;
  // Frame pre-test: with no sink frame in c and no pair of frames passing the temporal
  // part of the mask, no pair with c is kept; when every pair of frames passes it, the
  // pair tests below skip theirs.
  bool t_all = false;
  if (c.t0 >= m.sink && (m.kind == VSA_MASK_STRIPE || (m.kind == VSA_MASK_BOX && m.rt >= 0))) {
    bool a, n;
    if (m.kind == VSA_MASK_STRIPE)
      periodic_test(c.t0 - qb.t1, c.t1 - qb.t0, m.To, dv.ts, m.Tw, a, n);
    else
      radius_test(c.t0 - qb.t1, c.t1 - qb.t0, m.rt, a, n);
    // Column pre-test for stripes whose period divides the row width: a difference
    // dy*Wg + dx - So is congruent to dx - So mod Ss, so |.| mod Ss < Sw needs dx - So
    // within Sw - 1 of a multiple of Ss.
    if (n && dv.x_only) n = near_multiple(c.x0 - qb.x1 - m.So, c.x1 - qb.x0 - m.So, dv.ss, m.Sw);
    // Position pre-test for stripes: every s = y*Wg + x of a box lies in [y0*Wg + x0,
    // y1*Wg + x1], so the spatial part over the two ranges' differences bounds every pair
    // (narrow, and so deciding, when the tiles hold few positions).
    if (n && m.kind == VSA_MASK_STRIPE) {
      bool as, ns;
      periodic_test(c.y0 * g.Wg + c.x0 - (qb.y1 * g.Wg + qb.x1), c.y1 * g.Wg + c.x1 - (qb.y0 * g.Wg + qb.x0), m.So,
                    dv.ss, m.Sw, as, ns);
      n = ns;
    }
    if (!n) {
      all = false;
      return;
    }
    t_all = a;
  }
  if (c.t0 < m.sink) {  // key frames below the sink are kept for every query
    any = true;
    if (c.t1 < m.sink) return;
    c.t0 = m.sink;
  }
  for (int i = 0; i < nr; ++i) {
    bool a, n;
    box_pair_test(g, m, dv, R[i], c, a, n, t_all);
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
  const Box qb = bounding_box(R, nr);
  const PairDivs dv = pair_divs(g, m);
  for (int j = 0; j < nc && (all || !any); ++j) class_add(g, m, dv, R, nr, qb, C[j], all, any);
  return class_of(all, any, padded);
}

// Tile class of query boxes R[nr] (real tokens, bounding box qb) x the key tile of
// executed positions [c0, c1), whose boxes are visited one at a time and clipped to the
// real grid.  `padded`: the query tile or the key tile reaches past S.
VSA_HD int tile_class_range(const Geom& g, const DevMask& m, const PairDivs& dv, const Box* R, int nr,
                            const Box& qb, int c0, int c1, bool padded) {
  bool all = true, any = false;
  if (nr == 0) return VSA_TILE_EMPTY;
  for_each_box(g, c0, c1, [&](Box c) {
    if (!all && any) return;  // boundary whatever follows
    if (g.padded && !clip_box(g, c, padded)) return;
    class_add(g, m, dv, R, nr, qb, c, all, any);
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

}  // namespace vsa

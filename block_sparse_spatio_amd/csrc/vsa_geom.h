// Geometry of masks over executed positions, shared by the HIP kernels: the
// coordinates of a position in each token order, and the element mask of one query
// row over a key tile.  The key range is cut into runs of constant (t, y) and
// contiguous x (or, past the frame-0 block of position-major order, constant (y, x)
// and contiguous t; or, in tile-major order over one-column tiles, contiguous y); in
// each run the kept keys of a box, stripe or sliding-tile mask form a few contiguous
// bit ranges.  The tile classification built on these definitions is in
// vsa_classify_geom.h.
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
// entries of list row r in a table indexed by an exclusive prefix sum offs, clamped to
// [0, n] (offs comes from the classifier; the clamp keeps a malformed table in bounds)
VSA_HD int row_entries(const int64_t* offs, size_t r, int n) {
  const int64_t d = offs[r + 1] - offs[r];
  return d < 0 ? 0 : d > n ? n : (int)d;
}
// floor division for a possibly negative numerator and a positive divisor
VSA_HD int floor_div(int a, int b) {
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

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

// first tile of the sliding window of width w around tile a on an axis of n tiles
VSA_HD int sta_start(int a, int w, int n) { return imin(imax(a - w / 2, 0), imax(n - w, 0)); }

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
// A stripe period for the row masks: a plain integer (divided on the fly) or a
// multiply-high divisor prepared once per workgroup.
VSA_HD int period_value(int P) { return P; }
VSA_HD int period_value(const Divisor& P) { return (int)P.d; }
VSA_HD int period_div(int a, int P) { return a / P; }  // a >= 0
VSA_HD int period_div(int a, const Divisor& P) { return (int)udiv(P, (uint32_t)a); }

template <typename Per>
VSA_HD uint64_t periodic_bits(int ua, int ub, const Per& Pd, int w, int off) {
  // one division per sign of u: the periods are stepped from the first one
  const int P = period_value(Pd);
  uint64_t bits = 0;
  if (ub >= 0) {
    int lo = imax(ua, 0);
    for (int base = period_div(lo, Pd) * P; base <= ub; base += P) {
      int a = imax(lo, base), b = imin(ub, base + w - 1);
      if (a <= b) bits |= bit_range(off + a - ua, off + b - ua);
    }
  }
  if (ua < 0) {
    int lo = imax(-ub, 1), hi = -ua;  // |u| in [lo, hi]
    for (int base = period_div(lo, Pd) * P; base <= hi; base += P) {
      int a = imax(lo, base), b = imin(hi, base + w - 1);
      if (a <= b) bits |= bit_range(off - b - ua, off - a - ua);
    }
  }
  return bits;
}

// kept keys of a run (fixed t, y; x in [x0, x1]; bit of x0 is off) for query q
template <typename Per>
VSA_HD uint64_t run_mask(const Geom& g, const DevMask& m, const QueryPos& q, int t, int y, int x0,
                         int x1, int off, const Per& ss) {
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
      return periodic_bits(x0 + ubase, x1 + ubase, ss, m.Sw, off);
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
template <typename Per>
VSA_HD uint64_t run_mask_t(const Geom& g, const DevMask& m, const QueryPos& q, int t0, int t1, int y,
                           int x, int off, const Per& ts) {
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
      return bits | periodic_bits(t0 + vbase, t1 + vbase, ts, m.Tw, off);
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
template <typename Per>
VSA_HD uint64_t tile_row_mask_ft(const Geom& g, const DevMask& m, const QueryPos& q, int c0, int nbits,
                                 const Per& ss) {
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
    bits |= run_mask(g, m, q, c.t, c.y, c.x, c.x + len - 1, c.p - c0, ss);
    run_advance_ft(g, c, len);
  }
  return bits;
}

template <typename Per>
VSA_HD uint64_t tile_row_mask_pm(const Geom& g, const DevMask& m, const QueryPos& q, int c0, int nbits,
                                 const Per& ss, const Per& ts) {
  const int end = imin(c0 + nbits, g.S);
  uint64_t bits = 0;
  RunCursor c = run_begin(g, c0);
  while (c.p < end) {
    const int len = run_len_pm(g, c, end);
    if (run_along_t(g, c))
      bits |= run_mask_t(g, m, q, c.t, c.t + len - 1, c.y, c.x, c.p - c0, ts);
    else
      bits |= run_mask(g, m, q, c.t, c.y, c.x, c.x + len - 1, c.p - c0, ss);
    run_advance_pm(g, c, len);
  }
  return bits;
}

template <typename Per>
VSA_HD uint64_t tile_row_mask(const Geom& g, const DevMask& m, const QueryPos& q, int c0, int nbits, const Per& ss,
                              const Per& ts) {
  return g.layout == VSA_LAYOUT_POSITION_MAJOR ? tile_row_mask_pm(g, m, q, c0, nbits, ss, ts)
                                               : tile_row_mask_ft(g, m, q, c0, nbits, ss);
}

// The same with the mask's own periods, divided on the fly.
VSA_HD uint64_t tile_row_mask(const Geom& g, const DevMask& m, const QueryPos& q, int c0, int nbits) {
  return tile_row_mask(g, m, q, c0, nbits, m.Ss, m.Ts);
}

}  // namespace vsa

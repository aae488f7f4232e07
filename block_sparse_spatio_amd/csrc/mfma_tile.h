// Building blocks of the bf16 MFMA attention kernels (gfx950).
//
// A key tile is 64 keys.  Layout conventions (see attn_bf16.hip for the derivation):
//  * K is staged row-major in LDS with the rows permuted by swap_bits23 (so that the
//    S^T = K Q^T output layout hands each lane 8 consecutive keys per register half)
//    and the 16-byte chunks of a row XOR-swizzled by the row index.
//  * V is staged transposed (row = channel, 64 keys per row, 8 chunks of 8 keys) with
//    the chunk index XOR-swizzled by (d ^ d>>3) & 7.
//  * S^T block kb (keys kb*32..kb*32+31) in lane l, register i holds the score of query
//    column l%32 and key kb*32 + (i>>3)*16 + (l>>5)*8 + (i&7).
#pragma once

#include "vsa_geom.h"

namespace vsa {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;

__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // round-to-nearest-even conversion of two fp32 values into one dword
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// key offset (0..63) inside the tile of S^T block kb, register i, lane group g2
__device__ __forceinline__ constexpr int st_key(int kb, int i, int g2) {
  return kb * 32 + (i >> 3) * 16 + g2 * 8 + (i & 7);
}

template <int D>
struct TileSmem {
  static constexpr int KCH = D / 8;
  u32x4 k[BK * KCH];
  u32x4 vt[D * (BK / 8)];
};

// Cooperative global -> register -> LDS staging of one K/V tile by NT threads.
template <int D, int NT>
struct Stager {
  static constexpr int KCH = D / 8;
  static constexpr int K_PER_THREAD = (BK * KCH) / NT;
  static constexpr int VBLK = (BK / 4) * KCH;  // 4-key x 8-channel blocks
  static constexpr int V_PER_THREAD = (VBLK + NT - 1) / NT;
  static_assert((BK * KCH) % NT == 0, "K staging split");

  u32x4 kreg[K_PER_THREAD];
  u32x4 vreg[V_PER_THREAD][4];

  // Load the tile starting at key c0 (rows past S are clamped to S-1: those keys
  // are masked, and clamped rows hold finite data so their zero weights stay zero).
  __device__ __forceinline__ void load(const uint16_t* kp, const uint16_t* vp, size_t base,
                                       size_t tok_stride, int c0, int S, int tid) {
#pragma unroll
    for (int i = 0; i < K_PER_THREAD; ++i) {
      const int cid = tid + i * NT;
      const int r = cid / KCH, c = cid % KCH;
      const int key = imin(c0 + r, S - 1);
      kreg[i] = *(const u32x4*)(kp + base + (size_t)key * tok_stride + c * 8);
    }
#pragma unroll
    for (int i = 0; i < V_PER_THREAD; ++i) {
      const int blk = tid + i * NT;
      if (blk < VBLK) {
        const int kg = blk / KCH, dc = blk % KCH;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = imin(c0 + kg * 4 + j, S - 1);
          vreg[i][j] = *(const u32x4*)(vp + base + (size_t)key * tok_stride + dc * 8);
        }
      }
    }
  }

  __device__ __forceinline__ void store(TileSmem<D>& sm, int tid) const {
#pragma unroll
    for (int i = 0; i < K_PER_THREAD; ++i) {
      const int cid = tid + i * NT;
      const int r = cid / KCH, c = cid % KCH;
      const int row = swap_bits23(r);
      sm.k[row * KCH + (c ^ (row & (KCH - 1)))] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < V_PER_THREAD; ++i) {
      const int blk = tid + i * NT;
      if (blk < VBLK) {
        const int kg = blk / KCH, dc = blk % KCH;
        const int chunk = kg >> 1, half = kg & 1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // dword w of a row holds channels 2w, 2w+1
#pragma unroll
          for (int hi = 0; hi < 2; ++hi) {
            const int d = dc * 8 + 2 * w + hi;
            uint32_t x0, x1;
            if (hi == 0) {
              x0 = (vreg[i][0][w] & 0xffffu) | (vreg[i][1][w] << 16);
              x1 = (vreg[i][2][w] & 0xffffu) | (vreg[i][3][w] << 16);
            } else {
              x0 = (vreg[i][0][w] >> 16) | (vreg[i][1][w] & 0xffff0000u);
              x1 = (vreg[i][2][w] >> 16) | (vreg[i][3][w] & 0xffff0000u);
            }
            const int pc = chunk ^ ((d ^ (d >> 3)) & 7);
            u32x2* dst = (u32x2*)&sm.vt[d * 8 + pc] + half;
            *dst = u32x2{x0, x1};
          }
        }
      }
    }
  }
};

// S^T (64 keys x 32 queries of this wave) = K_tile Q^T
template <int D>
__device__ __forceinline__ void qk_tile(const TileSmem<D>& sm, const bf16x8* qf, int l32, int g2,
                                        f32x16* st) {
  constexpr int KCH = D / 8;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    st[kb] = f32x16{};
    const int row = kb * 32 + l32;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int c = 2 * s + g2;
      const bf16x8 kf = __builtin_bit_cast(bf16x8, sm.k[row * KCH + (c ^ (row & (KCH - 1)))]);
      st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[kb], 0, 0, 0);
    }
  }
}

// O^T (D x 32) += V_tile^T P^T, with P packed as bf16 pairs: pk[kb][0..7]
template <int D>
__device__ __forceinline__ void pv_tile(const TileSmem<D>& sm, const uint32_t (*pk)[8], int l32,
                                        int g2, f32x16* acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kb = j >> 1, hf = j & 1;
    const bf16x8 pf = __builtin_bit_cast(
        bf16x8, u32x4{pk[kb][hf * 4 + 0], pk[kb][hf * 4 + 1], pk[kb][hf * 4 + 2], pk[kb][hf * 4 + 3]});
    const int c = 2 * j + g2;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + l32;
      const bf16x8 vf = __builtin_bit_cast(bf16x8, sm.vt[d * 8 + (c ^ ((d ^ (d >> 3)) & 7))]);
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[db], 0, 0, 0);
    }
  }
}

// Apply the element mask (bit = key offset in the tile) to an S^T tile.
__device__ __forceinline__ void apply_mask(f32x16* st, uint64_t bits, int g2) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!((bits >> st_key(kb, i, g2)) & 1ull)) st[kb][i] = -INFINITY;
}

// One online-softmax step for the row held by this lane and lane^32: updates the
// running max m_run (raw score units) and partial sum l_run, returns the rescale
// factor for the accumulator and packs P = exp(scale*(s - m)) as bf16 pairs.
__device__ __forceinline__ float softmax_step(const f32x16* st, float c_log2, float& m_run,
                                              float& l_run, uint32_t (*pk)[8]) {
  float mt = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, st[kb][i]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float m_new = fmaxf(m_run, mt);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c_log2);
  const float mc = m_use * c_log2;
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(st[kb][i], c_log2, -mc));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(st[kb][i + 1], c_log2, -mc));
      lsum += p0 + p1;
      pk[kb][i >> 1] = pack_bf16x2(p0, p1);
    }
  l_run = l_run * alpha + lsum;
  m_run = m_new;
  return alpha;
}

}  // namespace mfma
}  // namespace vsa

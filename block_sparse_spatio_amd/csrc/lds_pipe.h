// Device building blocks shared by the bf16 attention kernel and the head profiler:
// tile geometry, LDS swizzles, the global -> LDS DMA, barriers and small lane
// reductions (CDNA4, gfx950).
#pragma once

#include "vsa_geom.h"

namespace vsa {
namespace pipe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BK = 64;
constexpr float kLazyLog2 = 8.0f;  // rescale only when the max grows by more than 2^8

template <int D, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = D * 2;                   // bytes of one K/V row
  static constexpr int CH = D / 8;                     // 16-byte chunks per row
  static constexpr int TILE_B = BK * ROWB;             // one K (or V) tile
  static constexpr int STAGE_B = 2 * TILE_B;           // K + V
  static constexpr int ROWS_PER_DMA = 1024 / ROWB;     // rows written by one wave-wide DMA
  static constexpr int DMA_PER_TENSOR = BK / ROWS_PER_DMA;
  static constexpr int NI = DMA_PER_TENSOR / NW;       // DMAs per wave per tensor per tile
  static constexpr int ROWS_PER_BANKLINE = 256 / ROWB; // rows sharing one 256-byte bank line
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static_assert(NI >= 1 && DMA_PER_TENSOR % NW == 0, "DMA split");
};

__device__ __forceinline__ int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// K chunk swizzle: the 16 rows read by one quarter-wave land on distinct banks
template <int D, int NW>
__device__ __forceinline__ int ksw(int row) {
  using C = Cfg<D, NW>;
  return (row / C::ROWS_PER_BANKLINE) & (C::CH - 1);
}
// V^T chunk swizzle (rows of 64 keys = 128 bytes, two rows per 256-byte bank line): the
// 16 channel rows read by one quarter-wave land on distinct banks
__device__ __forceinline__ int vtsw(int row) { return (row >> 1) & 7; }
// Row-major V chunk swizzle for transposing reads (ds_read_b64_tr_b16): the 4 rows of
// one transposing read land on distinct 64-byte segments
template <int D>
__device__ __forceinline__ int vsw(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One wave-wide 16-byte-per-lane DMA from global memory (wave-uniform base + per-lane
// 32-bit byte offset) into LDS at m0 + 16*lane (global_load_lds_dwordx4).  Issued through
// asm so that the compiler does not guard every later LDS read with a wait for all DMAs in
// flight: the kernel waits for the DMAs of a stage itself (wait_vmcnt) before the barrier
// that publishes the stage.
// m0 is written here without being named as clobbered: the compiler reserves m0 (it
// refuses it in a clobber list) and allocates no value to it, and nothing else in the
// kernels that include this header reads m0, so no live value can be overwritten.
// tests/test_asm_m0.py keeps that true: it builds the kernels to gfx950 assembly and
// checks that every m0 reference is one of these writes, directly followed by its DMA.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory");
}

// The same for 4 bytes per lane (global_load_lds_dword): LDS at m0 + 4*lane.
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (whose release fence
// would also wait for every DMA in flight).  LDS reads issued before it are complete
// (lgkmcnt(0)); DMA completion is waited for explicitly with wait_vmcnt.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> one dword of bf16 (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ bf16x2 pack_bf16x2(float lo, float hi) {
  return __builtin_convertvector(f32x2{lo, hi}, bf16x2);
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace pipe
}  // namespace vsa

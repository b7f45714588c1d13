// Device helpers shared by the matrix-core kernels (forward and backward):
// element traits, LDS swizzles, LDS-DMA, transposed LDS reads, cross-half
// reductions and wait helpers.  gfx950 only.
#pragma once

#include "gvattn_internal.h"

namespace gvattn {
namespace mfma {

using namespace dev;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Element type of Q/K/V/O: the matrix-core instruction and the rounding
// conversions (round to nearest even) for P and O.
template <typename T> struct Elem;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <> struct Elem<__bf16> {
  using v8 = bf16x8;
  using v4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // acc + the sum of the eight 16-bit values (v_dot2 with ones, FP32 sum)
  static __device__ __forceinline__ float sum8(v8 p, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
  }
};
template <> struct Elem<_Float16> {
  using v8 = f16x8;
  using v4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sum8(v8 p, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 6, 7), one, acc, false);
  }
};
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// XOR swizzles of the 16-byte chunk index inside a row, chosen so that the
// operand reads are free of bank conflicts on the 64 banks x 4 bytes of the
// gfx950 LDS (256 bytes per clock).
//  * K is read 16 bytes per lane, lanes = 16 consecutive rows at one logical
//    chunk per clock: the 16 rows must land on 16 distinct 16-byte slots of
//    the 256-byte bank window.
//  * V is read by ds_read_b64_tr_b16: 32 lanes = 4 consecutive rows x 64
//    bytes (one 32-wide d block) per clock: the four 64-byte groups must land
//    in distinct quarters of the window.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return (D == 64) ? ((row >> 1) & 7) : (row & 15);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return (D == 64) ? (((row >> 1) & 1) << 2) : ((row & 3) << 2);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds_dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, soff, 0, 0);
}

// v_permlane32_swap with both operands equal leaves lanes 0-31 of the
// first result and lanes 32-63 of the second holding the lower half's
// value, and the other two halves holding the upper half's value.
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ i16x4 read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// An empty volatile asm statement cannot be speculated, so a branch that
// contains one stays a branch instead of being if-converted into code that
// runs on every tile.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

__device__ __forceinline__ void wait_vmem() {
  // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace mfma
}  // namespace gvattn

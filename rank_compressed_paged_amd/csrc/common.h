// Shared device types and helpers for the gfx950 kernels of libstarkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace starkv {

typedef _Float16 f16;
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;                    // tokens per paged block
constexpr float kLog2e = 1.4426950408889634f;

// 32x32x16 f16 MFMA (gfx950): D[32x32] += A[32x16] * B[16x32], fp32 accumulate.
// Operand lane layout: lane l supplies row (A) / column (B) l%32 and the eight
// k values 8*(l/32) .. 8*(l/32)+7.  Result: lane l, register r holds
// D[mfma_row(r, l)][l%32].
__device__ __forceinline__ floatx16 mfma32x32x16(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ constexpr int mfma_row(int r, int lane) {
  return (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
}

// 16x16x32 f16 MFMA (gfx950): D[16x16] += A[16x32] * B[32x16], fp32 accumulate.
// Lane l supplies row (A) / column (B) l%16 and the eight k values
// 8*(l/16) .. 8*(l/16)+7; result register r of lane l is D[4*(l/16) + r][l%16].
__device__ __forceinline__ floatx4 mfma16x16x32(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// DPP sum over groups of G consecutive lanes (G = 1, 2, 4, 8, 16); every lane
// of a group ends with the group total.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2)   // quad_perm [1,0,3,2]
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  if constexpr (G >= 4)   // quad_perm [2,3,0,1]
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  if constexpr (G >= 8)   // row_half_mirror: lane i <-> 7-i within 8
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  if constexpr (G >= 16)  // row_mirror: lane i <-> 15-i within 16
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  static_assert(G <= 16, "group_sum supports up to 16 lanes");
  return x;
}

__device__ __forceinline__ float shfl_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Dot product of two fp16 rows of n elements (n % 8 == 0, n <= 256) with fp32
// accumulation.  All 16-byte loads of a 128-element batch are issued before
// the first multiply (one memory round trip per batch instead of one per
// load); loads past n are clamped to the last chunk and masked to zero.
__device__ __forceinline__ float dot_f16(const _Float16* __restrict__ a, const _Float16* __restrict__ b, int n) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  float acc = 0.f;
  for (int i0 = 0; i0 < n; i0 += 128) {
    h8 x[16], y[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int i = min(i0 + 8 * j, n - 8);
      x[j] = *reinterpret_cast<const h8*>(a + i);
      y[j] = *reinterpret_cast<const h8*>(b + i);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the arithmetic
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float live = i0 + 8 * j < n ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += live * ((float)x[j][e] * (float)y[j][e]);
    }
  }
  return acc;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);            // v_exp_f32; exp2(-inf) = 0
}

// Plan written by the query-projection launch and read by the later ones.
// Layout inside the workspace (int32):
//   [0] W  blocks per attention workgroup   [1] total blocks in the batch
//   [2 .. 2+B]        prefix[b]: first global block of sequence b (prefix[B] = total)
//   [3+B .. 3+2B]     slot_base[b]: first partial-state slot of sequence b
struct PlanView {
  const int32_t* p;
  int batch;
  __device__ int W() const { return p[0]; }
  __device__ int total() const { return p[1]; }
  __device__ const int32_t* prefix() const { return p + 2; }
  __device__ const int32_t* slot_base() const { return p + 3 + batch; }
  // sequence holding the first block of each attention workgroup's range
  __device__ const int32_t* first_seq() const { return p + 4 + 2 * batch; }
};

}  // namespace starkv

// Device building blocks for the gfx950 (CDNA4) attention kernels: MFMA
// wrappers, bf16 packing, exp2, wave reductions and LDS ordering.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

// C[16x16] += A[16x32] * B[32x16], bf16 in, fp32 accumulate.
// Lane l holds A row (l % 16) and B column (l % 16), eight k values each; both
// operands must use the same assignment of k values to (l / 16, slot), which
// makes the contraction independent of the hardware's k order. C: lane l holds
// column (l % 16), rows 4 * (l / 16) + r, r = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(const uint4 &a, const uint4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// C[32x32] += A[32x16] * B[16x32]. Lane l holds A row (l % 32) and B column
// (l % 32), eight k values each (same k-assignment rule as above). C: lane l
// holds column (l % 32), rows 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15.
__device__ __forceinline__ f32x16 mfma_32x32x16(const uint4 &a, const uint4 &b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}
__device__ __forceinline__ float wave_xor_sum(float x, int mask) {
  return x + __shfl_xor(x, mask, 64);
}

// Orders this wave's LDS writes before its later LDS reads (and reads before
// later writes) across lanes: waits for outstanding LDS operations and keeps
// the compiler from moving memory operations across the point.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint4 ldg16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint4 lds16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void sts16(uint16_t *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }
__device__ __forceinline__ void sts8(uint16_t *p, uint32_t x, uint32_t y) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(x, y);
}

// Transpose helpers for four rows r0..r3 of eight bf16 (one uint4 each): the
// two dwords holding column e of the four rows, i.e. (r0[e], r1[e]), (r2[e], r3[e]).
__device__ __forceinline__ uint32_t col_pair(uint32_t a, uint32_t b, int odd) {
  return odd ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}
__device__ __forceinline__ uint32_t dword_of(const uint4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

}  // namespace attn

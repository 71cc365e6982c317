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

// Element-type dispatch for the kernels: F16 = false for bfloat16 inputs,
// true for IEEE fp16 inputs. The MFMA operand and accumulator layouts are the
// same for both types; only the instruction and the P/O conversion differ.
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

template <bool F16>
__device__ __forceinline__ f32x4 mma16(const uint4 &a, const uint4 &b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  else
    return mfma_16x16x32(a, b, c);
}

template <bool F16>
__device__ __forceinline__ f32x16 mma32(const uint4 &a, const uint4 &b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                   0, 0);
  else
    return mfma_32x32x16(a, b, c);
}

// Two floats -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Two floats -> the packed pair of the element type, round to nearest even
// (v_cvt_pk_bf16_f32 or v_cvt_pk_f16_f32).
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (F16) {
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  } else {
    return pack_bf16x2(lo, hi);
  }
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_xor_max(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}
// max(x[l], x[l ^ 32]) in every lane l, without LDS: v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second, so with both operands x the two results hold, in every lane, the
// lane's own value and its partner's.
__device__ __forceinline__ float wave_max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_xor_sum(float x, int mask) {
  return x + __shfl_xor(x, mask, 64);
}

// Inclusive prefix sum over the 64 lanes of a wave (lane l gets x[0] + ... + x[l],
// modulo 2^32) through DPP, without LDS: shifts by 1, 2, 4 and 8 lanes within
// each 16-lane row (lanes shifted in from outside the row add 0), then the last
// lane of rows 0 and 2 added to rows 1 and 3 (row_bcast:15), then lane 31
// added to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ unsigned wave_incl_scan_u32(unsigned x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Orders this wave's LDS writes before its later LDS reads (and reads before
// later writes) across lanes: waits for outstanding LDS operations and keeps
// the compiler from moving memory operations across the point.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane k supplies the address of four consecutive bf16; lane i receives, as
// element j (j = 0..3), element (i % 4) of the four values addressed by lane
// 4j + i / 4. If lane k of a group points at row R(k / 4), columns
// c0 + 4 (k % 4) .. +3 of a row-major tile, lane i therefore receives column
// c0 + i of rows R(0..3): a 4 x 16 block comes back transposed, one column per
// lane, which is the k-major operand layout the MFMAs take.
// LDS reads at a byte address within the work-group's LDS allocation.
__device__ __forceinline__ uint4 lds16_at(unsigned a) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, *(const u32x4 __attribute__((address_space(3))) *)(uintptr_t)a);
}
__device__ __forceinline__ unsigned lds_offset(const void *p) { return (unsigned)reinterpret_cast<uintptr_t>(p); }

__device__ __forceinline__ uint2 lds_tr4(const uint16_t *p) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (bf16x4 __attribute__((address_space(3))) *)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(uint2, v);
}

// Direct-to-LDS buffer load: each of the wave's 64 lanes fetches 16 bytes at
// voffset through the descriptor (out-of-range offsets read zero) and the
// wave deposits them in lane order, 1 KB, at LDS byte address lds (wave
// uniform). The compiler does not see the LDS write: the caller waits
// (vmcnt) before the barrier that publishes the data. A load that takes its
// LDS address from M0 needs one wait state after M0 is set. M0 is listed as
// clobbered; the compiler warns because it reserves M0, and the kernels that
// use this leave M0 to these loads alone.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, int voffset, unsigned lds) {
  const unsigned la = __builtin_amdgcn_readfirstlane(lds);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(rs), "s"(la)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// lds_tr4 at an LDS byte address.
__device__ __forceinline__ uint2 lds_tr4_at(unsigned a) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 __attribute__((address_space(3))) *)(uintptr_t)a);
  return __builtin_bit_cast(uint2, v);
}

// XOR swizzle of the 16-byte chunk index of row r of a row-major bf16 tile in
// LDS with D = 128 (16 chunks per 256-byte row) or D = 64 (8 chunks per
// 128-byte row; two rows share a 256-byte bank window). Conflict-free for the
// two read patterns of the prefill tiles: 16 consecutive rows at one logical
// chunk (a 16-lane MFMA A-operand read of K) hit 16 distinct bank groups, and
// 4 consecutive rows (4-aligned) at 4 consecutive chunks (4-aligned) - the 32
// lanes of a transposing read of V - hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
  // D = 256 (32 chunks, 512-byte rows) takes the D = 128 swizzle: it moves the
  // low four chunk bits, which select the bank group.
  if constexpr (D >= 128) return (4 * (r & 3)) | ((r >> 2) & 3);
  else return (4 * ((r >> 1) & 1)) | ((r >> 2) & 3);
}

// f(I), f(I + 1), ..., f(N - 1) with the index a compile-time constant.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// A stream of NG MFMAs g = 0 .. NG - 1 whose LDS operands are read KDEP MFMAs
// ahead through a register ring, so no product waits on LDS latency:
// read(g) returns operand g, mma(g, a) issues product g. With PIN, a schedule
// barrier after each product keeps the compiler from regrouping the reads
// next to their uses.
template <int NG, int KDEP, bool PIN = true, typename R, typename M>
__device__ __forceinline__ void mfma_stream(R &&read, M &&mma) {
  uint4 ring[KDEP];
  static_for<0, (KDEP < NG ? KDEP : NG)>([&](auto gc) { ring[decltype(gc)::value] = read(gc); });
  static_for<0, NG>([&](auto gc) {
    constexpr int g = decltype(gc)::value;
    const uint4 a = ring[g % KDEP];
    if constexpr (g + KDEP < NG) ring[g % KDEP] = read(std::integral_constant<int, g + KDEP>{});
    mma(gc, a);
    if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
  });
}

__device__ __forceinline__ uint4 ldg16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint4 lds16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void sts16(uint16_t *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

// Fourth word of a raw buffer descriptor: 32-bit data format (a nonzero
// format is required for the loads to return data), no swizzle, no stride.
constexpr int kBufferWord3 = 0x00020000;

// Raw buffer descriptor over [base, base + bytes): loads at offsets past the
// end return zero. bytes <= 0 gives an empty range; sizes above 2^31 - 1 are
// clamped (every caller's offsets stay below that).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kBufferWord3);
}

// buffer_rsrc for a base and size that are the same in every lane, read from
// the first lane, so the descriptor is known to sit in scalar registers (the
// direct-to-LDS load takes it as an assembly operand).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_buffer_rsrc(const void *base, long long bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((unsigned long long)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(n), kBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}

}  // namespace attn

// Measurement kernels: the practical ceilings the attention kernels are
// compared against on the device they run on. They are not part of the
// attention path; the benchmark reports its rates beside the published peaks.
//   - probe_read: a streaming read of a large buffer (HBM read bandwidth).
//   - probe_mfma: independent chains of bf16 32x32x16 MFMAs on register
//     operands (matrix-core throughput at the clock the part sustains), with
//     the shader and constant clocks sampled at its start and end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_probe.h"

namespace attn {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// Grid-stride nontemporal 16-byte loads over the n16 chunks of p, U loads in
// flight per thread, XOR-folded into one word per thread (so no load is dead).
template <int U>
__global__ void __launch_bounds__(256) probe_read(const uint4 *__restrict__ p, size_t n16,
                                                  unsigned *__restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + i + u * stride));
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + i));
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave.
// The operands are small bf16 values of alternating sign, so the sums stay
// finite (finite data draws the power real kernels do). clk receives, from
// the first wave, the shader-clock and constant-clock (100 MHz) counters at
// its start and end.
__global__ void __launch_bounds__(256) probe_mfma(float *__restrict__ out, int iters,
                                                  unsigned long long *__restrict__ clk) {
  const unsigned t = threadIdx.x;
  // bf16 0x3c00 = 2^-7, sign bit flipped on alternate elements and lanes.
  const unsigned s0 = (t & 1) ? 0x80008000u : 0u;
  const uint4 a = make_uint4(0x3c003c00u ^ s0, 0x3c00bc00u ^ s0, 0xbc003c00u ^ s0, 0x3c003c00u);
  const uint4 b = make_uint4(0x3c00bc00u, 0x3c003c00u ^ s0, 0x3c003c00u, 0xbc003c00u ^ s0);
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma_32x32x16(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  out[(size_t)blockIdx.x * 256 + t] = s;
  if (blockIdx.x == 0 && t < 4) clk[t] = t == 0 ? c0 : (t == 1 ? c1 : (t == 2 ? r0 : r1));
}

}  // namespace
}  // namespace attn

extern "C" {

int attn_probe_stream_read(const void *buf, size_t bytes, unsigned *out, int grid, void *stream) {
  if (!buf || !out || grid <= 0 || bytes == 0 || (bytes & 15u) != 0) return ATTN_PROBE_INVALID;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return ATTN_PROBE_INVALID;
  hipLaunchKernelGGL(attn::probe_read<8>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : ATTN_PROBE_LAUNCH;
}

int attn_probe_mfma_bf16(float *out, int grid, int iters, unsigned long long *clk, void *stream) {
  if (!out || !clk || grid <= 0 || iters <= 0) return ATTN_PROBE_INVALID;
  if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0 || (reinterpret_cast<uintptr_t>(clk) & 7u) != 0)
    return ATTN_PROBE_INVALID;
  hipLaunchKernelGGL(attn::probe_mfma, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters, clk);
  return hipGetLastError() == hipSuccess ? 0 : ATTN_PROBE_LAUNCH;
}

}  // extern "C"

// GQA KV-cache decode for gfx950: split-KV kernel and log-sum-exp combine.
//
// Pages cited by title and section:
//   [FA4-decode] "Optimization diaries: S/P ping-pong for FlashAttention-4 decode"
//   [GQA-SM100]  "Building a Faster GQA Decode Kernel for Blackwell SM100"
//   [FA4-edges]  "Flash Attention 4 — warp-role choreography and the edges"
//
// Operand swap ([GQA-SM100] §Starting with the simple pipeline and the
// introduction): S^T = K Q^T / sqrt(d) and O^T = V^T P^T, so key positions
// run along the MFMA's M dimension and the small packed query group (the
// G = Hq / Hkv heads of one KV head times the seqlen_q new tokens, at most 16)
// along N. With v_mfma_f32_16x16x32_bf16 a lane then owns one query column:
// the column max and sum over keys are mostly in-lane, the rescale factor of
// O^T is one scalar per lane, and P leaves the S^T accumulator already in the
// layout the P*V MFMA wants as its B operand (it never goes through memory).
//
// Work decomposition: one work-group of four waves per (split, kv head, batch).
// The split's key range is cut into 32-position sub-blocks dealt round-robin to
// the waves; each wave streams its own sub-blocks (no cross-wave barrier in the
// loop) with register double buffering: the loads of sub-block i+1 are issued
// before the MFMA/softmax work of sub-block i. K and V pass through a per-wave
// LDS tile that changes their layout: K row-major with an XOR swizzle of its
// 16-byte chunks, V transposed (d-major) so the P*V A operand is one 16-byte
// LDS read. At the end the four waves merge their (max, sum, O^T) through LDS
// and the work-group writes one split partial (or, with a single split, the
// final O and LSE).
//
// Key order inside a sub-block: MFMA row i of score tile t (0/1) holds key
// 8 * (i / 4) + 4 * t + (i % 4). Lane group g (= lane / 16) then receives the
// scores of keys 8g .. 8g + 7 in its two accumulators, exactly the eight
// contiguous keys its P*V B-operand slots need, so the V^T read is contiguous.
#include "attn_device.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kSub = 32;  // key positions per wave sub-block
constexpr int kCols = 16; // packed query columns per work-group

// XOR swizzle of the 16-byte chunk index of K row r in LDS (row-major [32][D]).
// For D = 128 (16 chunks per 256-byte row) and D = 64 (8 chunks per 128-byte
// row) it makes the 16 rows one QK A-operand read touches land on 16 distinct
// 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 128) {
    return (r & 15) ^ ((r >> 4) << 2);
  } else {
    const int x = r >> 1;
    return (x & 1) | (((x >> 3) & 1) << 1) | (((x >> 2) & 1) << 2);
  }
}

// Swizzle of the 8-key unit of V^T row dd in LDS (d-major [D][32]).
__device__ __forceinline__ int vt_swz(int dd) { return (dd >> 2) & 3; }

template <int D>
struct DecodeSmem {
  static constexpr int kTile = kSub * D;                      // bf16 elements per K or V^T tile
  static constexpr int kLoopBytes = kWaves * 2 * kTile * 2;   // K + V^T per wave
  static constexpr int kMergeBytes = kWaves * kCols * (D + 2) * 4;
  static constexpr int kBytes = kLoopBytes > kMergeBytes ? kLoopBytes : kMergeBytes;
};

template <int D>
__global__ void __launch_bounds__(256, 2)
decode_split_kv(const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
                const uint16_t *__restrict__ vc, const int *__restrict__ seqlens,
                uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ ws_o,
                float2 *__restrict__ ws_ml, int Hq, int Hkv, int sq, int max_len, int chunk,
                int n_split, float scale_log2) {
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 64 / CH;    // rows one wave-wide 16-byte load covers
  constexpr int NK = kSub / RPI;  // K loads per lane per sub-block
  constexpr int NVG = CH / 8;     // 4-row V groups per lane per sub-block
  constexpr int KST = D / 32;     // k-steps of the QK MFMA
  constexpr int MT = D / 16;      // row tiles of O^T
  __shared__ __attribute__((aligned(16))) unsigned char smem[DecodeSmem<D>::kBytes];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = Hq / Hkv, ncol = G * sq;
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int lo = s * chunk;
  const int hi = min(lo + chunk, L);

  // Packed query column of this lane: n = t * G + hh ([FA4-edges] §Edge 2 · GQA:
  // row -> (seq_pos = row / G, q_head = row % G)).
  const int n = lane & 15, gq = lane >> 4;
  const bool col_ok = n < ncol;
  const int tn = col_ok ? n / G : 0;
  const int head = g * G + (col_ok ? n % G : 0);

  if (lo >= hi) {
    // Empty split. With a single split this is an empty sequence: O = 0 and
    // LSE = -inf. With several, the combine step skips splits past the end.
    if (n_split == 1) {
      for (int idx = threadIdx.x; idx < ncol * D; idx += blockDim.x) {
        const int c = idx / D, e = idx % D;
        o[((size_t)(b * sq + c / G) * Hq + g * G + c % G) * D + e] = 0;
      }
      if (lse != nullptr && threadIdx.x < ncol)
        lse[((size_t)b * Hq + g * G + threadIdx.x % G) * sq + threadIdx.x / G] = kNegInf;
    }
    return;
  }

  // Keys visible to this column: j < bound (tail of the split, and the
  // bottom-right causal limit j <= L - sq + t among the new tokens).
  const int bound = min(hi, L - sq + tn + 1);

  uint16_t *klds = reinterpret_cast<uint16_t *>(smem) + w * 2 * DecodeSmem<D>::kTile;
  uint16_t *vlds = klds + DecodeSmem<D>::kTile;

  // Q^T B operand, resident for the whole split: slot k of lane group gq at
  // k-step kk covers chunk 4 * kk + gq of the query row.
  uint4 qop[KST];
  {
    const uint16_t *qrow = q + ((size_t)(b * sq + tn) * Hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      qop[kk] = col_ok ? ldg16(qrow + (4 * kk + gq) * 8) : make_uint4(0, 0, 0, 0);
  }

  const size_t rstride = (size_t)Hkv * D;
  const uint16_t *kbase = kc + ((size_t)b * max_len * Hkv + g) * D;
  const uint16_t *vbase = vc + ((size_t)b * max_len * Hkv + g) * D;

  uint4 kreg[NK];
  uint4 vreg[NVG][4];
  auto load_sub = [&](int j0) {
    // Rows past `hi` are never read (they may lie past the allocation or hold
    // garbage); zero-filled V rows keep 0 * garbage out of the P*V product.
#pragma unroll
    for (int qi = 0; qi < NK; ++qi) {
      const int p = j0 + RPI * qi + lane / CH;
      kreg[qi] = p < hi ? ldg16(kbase + (size_t)p * rstride + (lane % CH) * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int hg = 0; hg < NVG; ++hg) {
      const int g4 = lane / CH + (64 / CH) * hg;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int p = j0 + 4 * g4 + qq;
        vreg[hg][qq] = p < hi ? ldg16(vbase + (size_t)p * rstride + (lane % CH) * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int j0 = lo + kSub * w;
  if (j0 < hi) load_sub(j0);
  for (; j0 < hi; j0 += kSub * kWaves) {
    // K registers -> LDS (row-major, swizzled chunks).
#pragma unroll
    for (int qi = 0; qi < NK; ++qi) {
      const int r = RPI * qi + lane / CH, c = lane % CH;
      sts16(klds + r * D + ((c ^ k_swz<D>(r)) * 8), kreg[qi]);
    }
    // V registers -> LDS transposed: V^T[dd][key], keys of a lane's 4-row group
    // stay contiguous (8 bytes).
#pragma unroll
    for (int hg = 0; hg < NVG; ++hg) {
      const int g4 = lane / CH + (64 / CH) * hg, c = lane % CH;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = 8 * c + e;
        const uint32_t x = col_pair(dword_of(vreg[hg][0], e >> 1), dword_of(vreg[hg][1], e >> 1), e & 1);
        const uint32_t y = col_pair(dword_of(vreg[hg][2], e >> 1), dword_of(vreg[hg][3], e >> 1), e & 1);
        sts8(vlds + dd * kSub + (((g4 >> 1) ^ vt_swz(dd)) * 8) + (g4 & 1) * 4, x, y);
      }
    }
    wave_lds_sync();

    // Issue the next sub-block's loads before this one's math.
    const int jn = j0 + kSub * kWaves;
    if (jn < hi) load_sub(jn);

    // S^T tiles: rows = keys (permuted as described above), columns = queries.
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int i = lane & 15;
      const int r = 8 * (i >> 2) + 4 * t + (i & 3);
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) {
        const int c = 4 * kk + gq;
        sacc[t] = mfma_16x16x32(lds16(klds + r * D + ((c ^ k_swz<D>(r)) * 8)), qop[kk], sacc[t]);
      }
    }

    // Online softmax in base 2 ([FA4-edges] §The correction; the 1/sqrt(d) and
    // log2(e) factors are folded into scale_log2 and applied to fp32 scores).
    // Masked keys are set to -inf before the max ([FA4-edges] §Edge 1).
    float sv[8];
    float mloc = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = j0 + 8 * gq + 4 * t + r;
        const float x = pos < bound ? sacc[t][r] * scale_log2 : kNegInf;
        sv[4 * t + r] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = wave_xor_max(mloc, 16);
    mloc = wave_xor_max(mloc, 32);
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = exp2_hw(sv[i] - m_use);
      psum += p[i];
    }
    l_run = l_run * alpha + psum;  // per-lane partial denominator
    m_run = m_new;
    // Rescale O before accumulating into it ([FA4-edges] §The value MMA waits
    // on three gates: P*V must not accumulate into an O in the old scale).
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;

    const uint4 pop = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                 pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int dd = 16 * mt + (lane & 15);
      oacc[mt] = mfma_16x16x32(lds16(vlds + dd * kSub + ((gq ^ vt_swz(dd)) * 8)), pop, oacc[mt]);
    }
    wave_lds_sync();
  }

  // Column denominators: the four lanes of a column hold partial sums.
  float l_col = wave_xor_sum(l_run, 16);
  l_col = wave_xor_sum(l_col, 32);

  // Merge the four waves through LDS.
  __syncthreads();
  float *mo = reinterpret_cast<float *>(smem);  // [wave][col][D]
  float *mm = mo + kWaves * kCols * D;          // [wave][col]
  float *ml = mm + kWaves * kCols;              // [wave][col]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    *reinterpret_cast<f32x4 *>(mo + (w * kCols + n) * D + 16 * mt + 4 * gq) = oacc[mt];
  if (gq == 0) {
    mm[w * kCols + n] = m_run;
    ml[w * kCols + n] = l_col;
  }
  __syncthreads();

  constexpr int SEG = D / 16;  // output elements per thread (16 threads per column)
  const int cn = threadIdx.x >> 4, seg = (threadIdx.x & 15) * SEG;
  if (cn >= ncol) return;
  float M = kNegInf;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, mm[ww * kCols + cn]);
  float acc[SEG];
#pragma unroll
  for (int e = 0; e < SEG; ++e) acc[e] = 0.f;
  float lsum = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float sc = exp2_hw(mm[ww * kCols + cn] - M);
      lsum += sc * ml[ww * kCols + cn];
      const float *src = mo + (ww * kCols + cn) * D + seg;
#pragma unroll
      for (int e = 0; e < SEG; ++e) acc[e] += sc * src[e];
    }
  }
  const int ct = cn / G, chead = g * G + cn % G;
  if (n_split == 1) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint16_t *dst = o + ((size_t)(b * sq + ct) * Hq + chead) * D + seg;
#pragma unroll
    for (int e = 0; e < SEG; e += 2) {
      *reinterpret_cast<uint32_t *>(dst + e) = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
    }
    if (lse != nullptr && (threadIdx.x & 15) == 0)
      lse[((size_t)b * Hq + chead) * sq + ct] = lsum > 0.f ? kLn2 * (M + __log2f(lsum)) : kNegInf;
  } else {
    const size_t row = ((size_t)b * Hq + chead) * sq + ct;
    float *dst = ws_o + (row * n_split + s) * D + seg;
#pragma unroll
    for (int e = 0; e < SEG; e += 4)
      *reinterpret_cast<float4 *>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    if ((threadIdx.x & 15) == 0) ws_ml[row * n_split + s] = make_float2(M, lsum);
  }
}

// Split-KV combine ([GQA-SM100] §Combining the KV splits, §Removing the max
// reset): per query row, the common maximum is the max of the staged split
// maxima; every split is rescaled by 2^(m_s - M) and the weighted fp32 sum is
// normalised, in a fixed split order. Splits that lie past the sequence end are
// never read (they were not written by this call) and splits with m_s = -inf
// are skipped; an empty row gives O = 0, LSE = -inf. O is overwritten.
template <int D>
__global__ void __launch_bounds__(256)
combine_splits(const float *__restrict__ ws_o, const float2 *__restrict__ ws_ml,
               const int *__restrict__ seqlens, uint16_t *__restrict__ o, float *__restrict__ lse,
               int n_rows, int Hq, int sq, int max_len, int chunk, int n_split) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= n_rows) return;
  const int tr = threadIdx.x % TPR;
  const int b = row / (Hq * sq), rem = row % (Hq * sq), h = rem / sq, t = rem % sq;
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int nv = min(n_split, (L + chunk - 1) / chunk);
  const float2 *ml = ws_ml + (size_t)row * n_split;
  float M = kNegInf;
  for (int sp = 0; sp < nv; ++sp) M = fmaxf(M, ml[sp].x);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  if (M != kNegInf) {
    for (int sp = 0; sp < nv; ++sp) {
      const float2 v = ml[sp];
      if (v.x == kNegInf) continue;
      const float sc = exp2_hw(v.x - M);
      lsum += sc * v.y;
      const float4 x = *reinterpret_cast<const float4 *>(ws_o + ((size_t)row * n_split + sp) * D + 4 * tr);
      acc.x += sc * x.x;
      acc.y += sc * x.y;
      acc.z += sc * x.z;
      acc.w += sc * x.w;
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t *dst = o + ((size_t)(b * sq + t) * Hq + h) * D + 4 * tr;
  *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv),
                                               pack_bf16x2(acc.z * inv, acc.w * inv));
  if (lse != nullptr && tr == 0)
    lse[((size_t)b * Hq + h) * sq + t] = lsum > 0.f ? kLn2 * (M + __log2f(lsum)) : kNegInf;
}

}  // namespace

// Host-side launchers (called by the C ABI after validation).
hipError_t launch_decode(const void *q, const void *k, const void *v, const int32_t *seqlens,
                         void *o, float *lse, float *ws_o, float2 *ws_ml, int batch, int Hq,
                         int Hkv, int d, int sq, int max_len, int chunk, int n_split,
                         float scale_log2, hipStream_t stream) {
  const dim3 grid(n_split, Hkv, batch), block(256);
  const auto *qq = static_cast<const uint16_t *>(q);
  const auto *kk = static_cast<const uint16_t *>(k);
  const auto *vv = static_cast<const uint16_t *>(v);
  auto *oo = static_cast<uint16_t *>(o);
  if (d == 128)
    hipLaunchKernelGGL(decode_split_kv<128>, grid, block, 0, stream, qq, kk, vv, seqlens, oo, lse,
                       ws_o, ws_ml, Hq, Hkv, sq, max_len, chunk, n_split, scale_log2);
  else
    hipLaunchKernelGGL(decode_split_kv<64>, grid, block, 0, stream, qq, kk, vv, seqlens, oo, lse,
                       ws_o, ws_ml, Hq, Hkv, sq, max_len, chunk, n_split, scale_log2);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_split == 1) return err;
  const int n_rows = batch * Hq * sq;
  const int rpb = 256 / (d / 4);
  const dim3 cgrid((n_rows + rpb - 1) / rpb);
  if (d == 128)
    hipLaunchKernelGGL(combine_splits<128>, cgrid, block, 0, stream, ws_o, ws_ml, seqlens, oo, lse,
                       n_rows, Hq, sq, max_len, chunk, n_split);
  else
    hipLaunchKernelGGL(combine_splits<64>, cgrid, block, 0, stream, ws_o, ws_ml, seqlens, oo, lse,
                       n_rows, Hq, sq, max_len, chunk, n_split);
  return hipGetLastError();
}

}  // namespace attn

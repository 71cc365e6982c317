// Prefill attention forward for gfx950 (MFMA-bound).
//
// Pages cited by title and section:
//   [FA4-decode] "Optimization diaries: S/P ping-pong for FlashAttention-4 decode"
//   [GQA-SM100]  "Building a Faster GQA Decode Kernel for Blackwell SM100"
//   [FA4-edges]  "Flash Attention 4 — warp-role choreography and the edges"
//
// Same inner loop as decode, widened: S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_bf16, each wave owning 32 query columns; a work-group of
// four waves owns a 128-row query tile and shares 64-key K / V^T tiles in LDS.
// Tiles are double-buffered: the global loads of key block i+1 are issued into
// registers before block i's math, then written to the other LDS stage, with
// one work-group barrier per block.
//
// Causal masking ([FA4-edges] §Edge 1 · causal masking): per (query tile, key
// block) the block is fully visible, on the diagonal (masked to -inf before the
// max), or skipped; a work-group only walks keys [0, kend) and a wave skips the
// math of blocks entirely in its future.
// Scheduling ([FA4-edges] §Edge 3 · tile scheduling): work-groups are
// numbered heaviest first (last query tile first, longest visible key range),
// a longest-processing-time order that shortens the tail. With batch * heads a
// multiple of 8, all query tiles of one (batch, head) fall on the same XCD
// (work-groups are dealt round-robin to the 8 XCDs), so they share K/V in that
// XCD's L2.
//
// Key order inside a 32-key score tile: MFMA row i holds key pi(i), where pi
// swaps bits 2 and 3 of i. Lane half h (= lane / 32) then finds, in registers
// 8k .. 8k + 7 of its accumulator, keys 16k + 8h .. 16k + 8h + 7: the eight
// contiguous keys of its P*V B operand for that 16-key step.
#include "attn_device.h"

namespace attn {
namespace {

constexpr int kBM = 128;  // query rows per work-group
constexpr int kBN = 64;   // keys per block

__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i >> 1) & 4) | ((i << 1) & 8);
}

// K tile in LDS: row-major [64][D], XOR swizzle of 16-byte chunks so that the
// 16 consecutive rows of an A-operand read hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int kf_swz(int r) {
  if constexpr (D == 128) return r & 15;
  else return (r >> 1) & 7;
}
// V^T tile in LDS: d-major [D][64]; 16-byte unit swizzle per row.
__device__ __forceinline__ int vf_swz(int dd) { return (dd >> 1) & 7; }

template <int D>
__global__ void __launch_bounds__(256, 2)
fwd_tile(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
         const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
         int Sq, int Sk, int Hq, int Hkv, int causal, float scale_log2, int n_mblocks, int BH) {
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int TILE = kBN * D;          // bf16 elements per K or V^T tile
  constexpr int RPT = 256 / CH;          // rows one work-group-wide load covers
  constexpr int NKL = kBN / RPT;         // K loads per thread per block
  constexpr int VTHREADS = (kBN / 4) * CH;  // threads holding one 4-row V group
  constexpr int KST = D / 16;            // QK k-steps
  constexpr int MT = D / 32;             // O^T row tiles
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];

  const int x = blockIdx.x;
  const int mb = n_mblocks - 1 - x / BH;  // heaviest query tile first
  const int u = x % BH;
  const int b = u / Hq, h = u % Hq;
  const int gk = h / (Hq / Hkv);
  const int q0 = mb * kBM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hl = lane >> 5;
  const int qrow = q0 + 32 * w + n;
  const int off = Sk - Sq;  // bottom-right alignment

  int kend = causal ? min(Sk, q0 + kBM + off) : Sk;
  if (kend < 0) kend = 0;
  const int nblk = (kend + kBN - 1) / kBN;
  const int bound = causal ? min(Sk, qrow + off + 1) : Sk;           // this column's keys: j < bound
  const int wave_hi = causal ? min(Sk, q0 + 32 * w + 31 + off + 1) : Sk;  // max bound over the wave

  uint4 qop[KST];
  {
    const bool ok = qrow < Sq;
    const uint16_t *qp = q + ((size_t)(b * Sq + (ok ? qrow : 0)) * Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) qop[kk] = ok ? ldg16(qp + (2 * kk + hl) * 8) : make_uint4(0, 0, 0, 0);
  }

  const size_t rstride = (size_t)Hkv * D;
  const uint16_t *kb = k + ((size_t)b * Sk * Hkv + gk) * D;
  const uint16_t *vb = v + ((size_t)b * Sk * Hkv + gk) * D;
  uint4 kreg[NKL];
  uint4 vreg[4];
  auto load_blk = [&](int j0) {
#pragma unroll
    for (int qi = 0; qi < NKL; ++qi) {
      const int p = j0 + RPT * qi + tid / CH;
      kreg[qi] = p < Sk ? ldg16(kb + (size_t)p * rstride + (tid % CH) * 8) : make_uint4(0, 0, 0, 0);
    }
    if (tid < VTHREADS) {
      const int g4 = tid / CH;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int p = j0 + 4 * g4 + qq;
        vreg[qq] = p < Sk ? ldg16(vb + (size_t)p * rstride + (tid % CH) * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_blk = [&](int st) {
    uint16_t *kl = smem + st * 2 * TILE;
    uint16_t *vl = kl + TILE;
#pragma unroll
    for (int qi = 0; qi < NKL; ++qi) {
      const int r = RPT * qi + tid / CH, c = tid % CH;
      sts16(kl + r * D + ((c ^ kf_swz<D>(r)) * 8), kreg[qi]);
    }
    if (tid < VTHREADS) {
      const int g4 = tid / CH, c = tid % CH;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = 8 * c + e;
        const uint32_t xx = col_pair(dword_of(vreg[0], e >> 1), dword_of(vreg[1], e >> 1), e & 1);
        const uint32_t yy = col_pair(dword_of(vreg[2], e >> 1), dword_of(vreg[3], e >> 1), e & 1);
        sts8(vl + dd * kBN + (((g4 >> 1) ^ vf_swz(dd)) * 8) + (g4 & 1) * 4, xx, yy);
      }
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;

  if (nblk > 0) load_blk(0);
  for (int blk = 0; blk < nblk; ++blk) {
    const int st = blk & 1;
    store_blk(st);
    __syncthreads();
    if (blk + 1 < nblk) load_blk((blk + 1) * kBN);
    const int j0 = blk * kBN;
    if (j0 >= wave_hi) continue;  // whole block in this wave's future
    const uint16_t *kl = smem + st * 2 * TILE;
    const uint16_t *vl = kl + TILE;

    f32x16 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
      const int row = 32 * t + swap_bits23(n);
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) {
        const int c = 2 * kk + hl;
        sacc[t] = mfma_32x32x16(lds16(kl + row * D + ((c ^ kf_swz<D>(row)) * 8)), qop[kk], sacc[t]);
      }
    }

    // Register r of tile t holds key j0 + 32t + pi(8(r/4) + 4hl + r%4)
    //   = j0 + 32t + 16(r/8) + 8hl + (r%8).
    float mloc = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = j0 + 32 * t + 16 * (r >> 3) + 8 * hl + (r & 7);
        const float xs = pos < bound ? sacc[t][r] * scale_log2 : kNegInf;
        sacc[t][r] = xs;
        mloc = fmaxf(mloc, xs);
      }
    mloc = wave_xor_max(mloc, 32);
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_hw(m_run - m_use);
    float psum = 0.f;
    uint4 pop[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          pv[s] = exp2_hw(sacc[t][8 * hh + s] - m_use);
          psum += pv[s];
        }
        pop[2 * t + hh] = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                     pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int dd = 32 * mt + n;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // 16-key step ks covers keys 16ks + 8hl .. 16ks + 8hl + 7 for this lane.
        const int unit = 2 * ks + hl;
        oacc[mt] = mfma_32x32x16(lds16(vl + dd * kBN + ((unit ^ vf_swz(dd)) * 8)), pop[ks], oacc[mt]);
      }
    }
  }

  const float l_col = wave_xor_sum(l_run, 32);
  if (qrow >= Sq) return;
  const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
  uint16_t *dst = o + ((size_t)(b * Sq + qrow) * Hq + h) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dd = 32 * mt + 8 * a + 4 * hl;
      *reinterpret_cast<uint2 *>(dst + dd) =
          make_uint2(pack_bf16x2(oacc[mt][4 * a] * inv, oacc[mt][4 * a + 1] * inv),
                     pack_bf16x2(oacc[mt][4 * a + 2] * inv, oacc[mt][4 * a + 3] * inv));
    }
  if (lse != nullptr && hl == 0)
    lse[((size_t)b * Hq + h) * Sq + qrow] = l_col > 0.f ? kLn2 * (m_run + __log2f(l_col)) : kNegInf;
}

}  // namespace

hipError_t launch_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
                      int batch, int Sq, int Sk, int Hq, int Hkv, int d, float scale_log2,
                      hipStream_t stream) {
  const int n_mblocks = (Sq + kBM - 1) / kBM;
  const int BH = batch * Hq;
  const dim3 grid(n_mblocks * BH), block(256);
  const auto *qq = static_cast<const uint16_t *>(q);
  const auto *kk = static_cast<const uint16_t *>(k);
  const auto *vv = static_cast<const uint16_t *>(v);
  auto *oo = static_cast<uint16_t *>(o);
  if (d == 128)
    hipLaunchKernelGGL(fwd_tile<128>, grid, block, 0, stream, qq, kk, vv, oo, lse, Sq, Sk, Hq, Hkv,
                       causal, scale_log2, n_mblocks, BH);
  else
    hipLaunchKernelGGL(fwd_tile<64>, grid, block, 0, stream, qq, kk, vv, oo, lse, Sq, Sk, Hq, Hkv,
                       causal, scale_log2, n_mblocks, BH);
  return hipGetLastError();
}

}  // namespace attn

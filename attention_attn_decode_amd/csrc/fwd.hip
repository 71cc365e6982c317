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
// registers before block i's math, then written to the other LDS slot, with
// one work-group barrier per block. K and V stay row-major in LDS (16-byte
// writes); the P*V operand, which needs keys along its k dimension, is read
// with the transposing ds_read_b64_tr_b16.
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
#include <type_traits>

#include "attn_device.h"

namespace attn {
namespace {

constexpr int kBM = 128;  // query rows per work-group
constexpr int kBN = 64;   // keys per block (template default; 32 measured equal)

__device__ __forceinline__ int swap_bits23(int i) {
  return (i & ~12) | ((i >> 1) & 4) | ((i << 1) & 8);
}

// Row strides (bf16 elements) of the K and V tiles in LDS. Padding replaces
// an XOR swizzle, so every read address is a per-lane base plus a constant:
//  - K rows of 17 (d=128) or 9 (d=64) 16-byte units: the 16 consecutive rows
//    of an MFMA A-operand read start on 16 distinct bank groups;
//  - V rows of 20 (d=128) or 12 (d=64) units: the 4 rows x 4 chunks that the
//    32 lanes of a transposing read touch land on 16 distinct bank groups.
template <int D> struct KRow { static constexpr int v = D + 8; };
template <int D> struct VRow { static constexpr int v = D == 128 ? 160 : 96; };

// BN keys per block; OCC work-groups of 4 waves per CU the register budget
// is sized for (two: 2 waves per SIMD).
template <int D, int BN, int OCC>
__global__ void __launch_bounds__(256, OCC)
fwd_tile(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
         const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
         int Sq, int Sk, int Hq, int Hkv, int causal, float scale_log2, int n_mblocks, int BH) {
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int KROW = KRow<D>::v, VROW = VRow<D>::v;
  constexpr int KT = BN * KROW, VT = BN * VROW;  // bf16 elements per K / V tile
  constexpr int RPT = 256 / CH;    // rows one work-group-wide load covers
  constexpr int NKL = BN / RPT;   // K (and V) loads per thread per block
  constexpr int KST = D / 16;      // QK k-steps
  constexpr int MT = D / 32;       // O^T row tiles
  constexpr int NT = BN / 32;      // 32-key score tiles per block
  constexpr int NKS = BN / 16;     // 16-key P*V steps per block
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KT + VT)];

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
  const int nblk = (kend + BN - 1) / BN;
  // Keys this column may see: j < bound. Over the wave the bound ranges from
  // wave_lo (first column) to wave_hi (last column).
  const int bound = causal ? min(Sk, qrow + off + 1) : Sk;
  const int wave_lo = causal ? min(Sk, q0 + 32 * w + off + 1) : Sk;
  const int wave_hi = causal ? min(Sk, q0 + 32 * w + 31 + off + 1) : Sk;

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
  uint16_t *ktile = smem;           // K tiles, 2 slots
  uint16_t *vtile = smem + 2 * KT;  // V tiles, 2 slots
  uint4 kreg[NKL], vreg[NKL];
  // Per-thread row pointers of block 0; block i adds i * 64 rows. Rows past
  // Sk (only in a ragged last block) are clamped to Sk - 1: finite data the
  // mask excludes, so the load count per block never changes.
  const size_t blk_stride = (size_t)BN * rstride;
  const int trow = tid / CH, tcol = (tid % CH) * 8;
  auto load_kv = [&](int blk, uint4 (&kr)[NKL], uint4 (&vr)[NKL]) {
    const size_t base = (size_t)blk * blk_stride;
    if (blk * BN + BN <= Sk) {
#pragma unroll
      for (int qi = 0; qi < NKL; ++qi) {
        const size_t o = base + (size_t)(RPT * qi + trow) * rstride + tcol;
        kr[qi] = ldg16(kb + o);
        vr[qi] = ldg16(vb + o);
      }
    } else {
#pragma unroll
      for (int qi = 0; qi < NKL; ++qi) {
        const int p = min(blk * BN + RPT * qi + trow, Sk - 1);
        const size_t o = (size_t)p * rstride + tcol;
        kr[qi] = ldg16(kb + o);
        vr[qi] = ldg16(vb + o);
      }
    }
  };
  auto store_kv = [&](int slot, const uint4 (&kr)[NKL], const uint4 (&vr)[NKL]) {
#pragma unroll
    for (int qi = 0; qi < NKL; ++qi) {
      sts16(ktile + slot * KT + (RPT * qi + trow) * KROW + tcol, kr[qi]);
      sts16(vtile + slot * VT + (RPT * qi + trow) * VROW + tcol, vr[qi]);
    }
  };

  // Lane-dependent parts of the LDS read addresses; the per-instruction parts
  // (tile t, k-step, row tile, key step) are compile-time constants added to
  // them, which the compiler folds into the instructions' offset fields.
  // QK A operand: K row 32t + pi(n), chunk 2kk + hl.
  const int k_lane = swap_bits23(n) * KROW + hl * 8;
  // P*V A operand (transposing reads of V): lane l is lane k = l % 16 of
  // 16-lane group l / 16; the group covers output rows dd = 32mt + 16((l/16)%2)
  // + 0..15 and keys 16ks + 8hl + 4u + 0..3; lane k addresses key row
  // (k / 4) of those, columns 32mt + 16((l/16)%2) + 4(k % 4) .. +3.
  const int trk = lane & 15, trhalf = (lane >> 4) & 1;
  const int v_lane = (8 * hl + (trk >> 2)) * VROW + 16 * trhalf + 4 * (trk & 3);

  auto qk = [&](int slot, f32x16 (&sa)[NT]) {
    const uint16_t *kl = ktile + slot * KT + k_lane;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[t][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        sa[t] = mfma_32x32x16(lds16(kl + 32 * t * KROW + 16 * kk), qop[kk], sa[t]);
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;

  // Softmax of one score block (register r of tile t holds key
  // j0 + 32t + pi(8(r/4) + 4hl + r%4) = j0 + 32t + 16(r/8) + 8hl + (r%8)),
  // producing the bf16 P operands; returns the rescale factor of O.
  auto softmax = [&](f32x16 (&sa)[NT], int j0, uint4 (&pop)[NKS], auto masked) -> float {
    // Masking ([FA4-edges] §Edge 1): keys past this column's bound get -inf
    // before the max. Only blocks reaching past the wave's first bound (the
    // diagonal, the end of the keys, or blocks in the wave's future) pay it.
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pos = j0 + 32 * t + 16 * (r >> 3) + 8 * hl + (r & 7);
          sa[t][r] = pos < bound ? sa[t][r] : kNegInf;
        }
    }
    float mloc = kNegInf;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sa[t][r]);
    mloc = wave_xor_max(mloc, 32);
    // Base-2 online softmax on raw scores: m is kept scaled (scale > 0, so
    // max(scale * s) = scale * max(s)); p = 2^(s * scale - m) is one fma + exp.
    const float m_new = fmaxf(m_run, mloc * scale_log2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pv[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          pv[s2] = exp2_hw(__builtin_fmaf(sa[t][8 * hh + s2], scale_log2, -m_use));
          psum += pv[s2];
        }
        pop[2 * t + hh] = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                     pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7]));
      }
    const float alpha = exp2_hw(m_run - m_use);  // exactly 1 where the max did not move
    l_run = l_run * alpha + psum;
    m_run = m_new;
    return alpha;
  };

  // P*V for one block. O^T is rescaled before any accumulation ([FA4-edges]
  // §The value MMA waits on three gates: P*V must not add into an O that is
  // still in the old scale).
  auto pv = [&](int slot, const uint4 (&pop)[NKS], float alpha) {
    const uint16_t *vl = vtile + slot * VT + v_lane;
    // Rescale O only when some column's maximum moved ([FA4-edges] §The
    // correction); O is register-resident, so the test is one wave vote.
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        // 16-key step ks: this lane's B slots hold keys 16ks + 8hl + 0..7;
        // the A operand is the same keys at column 32mt + n, read transposed.
        const uint2 t0 = lds_tr4(vl + 16 * ks * VROW + 32 * mt);
        const uint2 t1 = lds_tr4(vl + (16 * ks + 4) * VROW + 32 * mt);
        oacc[mt] = mfma_32x32x16(make_uint4(t0.x, t0.y, t1.x, t1.y), pop[ks], oacc[mt]);
      }
    }
  };

  // Block i: its K/V move from registers into LDS slot i % 2 (whose previous
  // tile, block i - 2, every wave finished before the last barrier); then the
  // loads of block i + 1 go out, and block i is computed. One barrier per
  // block.
  if (nblk > 0) load_kv(0, kreg, vreg);
  for (int i = 0; i < nblk; ++i) {
    store_kv(i & 1, kreg, vreg);
    __syncthreads();
    if (i + 1 < nblk) load_kv(i + 1, kreg, vreg);
    if (i * BN >= wave_hi) continue;  // whole block in this wave's future
    // Wave priority follows the phase: the MFMA phases run at high priority,
    // so when both waves of a SIMD are ready the one feeding the matrix unit
    // issues first and the other's softmax fills the gaps.
    f32x16 S[NT];
    __builtin_amdgcn_s_setprio(2);
    qk(i & 1, S);
    __builtin_amdgcn_s_setprio(0);
    uint4 pop[NKS];
    const float alpha = (i * BN + BN > wave_lo) ? softmax(S, i * BN, pop, std::true_type{})
                                                  : softmax(S, i * BN, pop, std::false_type{});
    __builtin_amdgcn_s_setprio(2);
    pv(i & 1, pop, alpha);
    __builtin_amdgcn_s_setprio(0);
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
    hipLaunchKernelGGL((fwd_tile<128, kBN, 2>), grid, block, 0, stream, qq, kk, vv, oo, lse, Sq, Sk, Hq,
                       Hkv, causal, scale_log2, n_mblocks, BH);
  else
    hipLaunchKernelGGL((fwd_tile<64, kBN, 2>), grid, block, 0, stream, qq, kk, vv, oo, lse, Sq, Sk, Hq,
                       Hkv, causal, scale_log2, n_mblocks, BH);
  return hipGetLastError();
}

}  // namespace attn

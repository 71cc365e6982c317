// Attention backward for gfx950: dQ, dK, dV from Q, K, V, O, LSE and dO.
//
// Pages cited by title and section:
//   [FA4-bwd]   "Optimization diaries: Improving FlashAttention-4 backward pass
//                kernel design for head dimension 64"
//   [FA4-edges] "Flash Attention 4 — warp-role choreography and the edges"
//
// With s = 1/sqrt(d) and L the natural-log LSE of the forward
// ([FA4-bwd] §Recap on the FA4 backward pass):
//   P = exp(s Q K^T - L),  dP = dO V^T,  dS = P o (dP - D),
//   dV = P^T dO,  dK = s dS^T Q,  dQ = s dS K,  D = rowsum(dO o O).
//
// Three kernels, no atomics and no zero-initialised memory:
//   bwd_pre   -D and L * log2(e) per query row, into the caller's workspace.
//   bwd_dkdv  one work-group per (batch, KV head, key tile), as in the page's
//             recap: it owns its K and V rows, walks the query tiles of every
//             query head that reads its KV head (GQA heads summed in
//             registers) and writes dK and dV once.
//   bwd_dq    one work-group per (batch, query head, row tile): it owns its Q
//             and dO rows, walks the key tiles and writes dQ once.
// The page sums dQ contributions from the KV-tile owners into an fp32 buffer
// in global memory. Here dQ has its own pass that recomputes S and dP (seven
// products per (query, key) tile instead of five): no atomic traffic (which
// would be about Sk / 128 times the size of dQ), no zeroed accumulator, and
// bitwise-reproducible results.
//
// Each wave owns 32 rows (keys or queries). At d = 64 a work-group is four
// waves (128 rows) and two run per CU; at d = 128 it is eight waves (256 rows),
// one per CU, so each staged tile serves eight waves, and the dK/dV kernel
// keeps its 256 V rows as a resident LDS tile (read as the dP operand)
// instead of registers, which fits the 256-register budget of two waves per
// SIMD. Only steps that cut the visible region run the per-element mask.
//
// Both main kernels use the forward's swap-AB orientation for the tile they
// own: the owned rows (keys in bwd_dkdv, queries in bwd_dq) are the MFMA N
// dimension held in registers, one row per lane, and the streamed tile is
// the LDS operand. Every product is a v_mfma_f32_32x32x16 and every
// probability tile feeds the next product straight from registers: the
// accumulator of a 32 x 32 tile is, lane for lane, the B operand of a product
// contracting over its rows, once the rows are read in the order pi (bits 2
// and 3 of the row index swapped). The streamed tiles are read both row-wise
// (products contracting over d) and transposed (products contracting over
// rows, ds_read_b64_tr_b16); an XOR swizzle of their 16-byte chunks keeps both
// read patterns free of bank conflicts.
//
// Masking ([FA4-edges] §Edge 1 · causal masking) is bottom-right aligned as in
// the forward: query i sees keys j <= i + Sk - Sq. Masked pairs, rows past Sq
// and keys past Sk get P = dS = 0 by selection, so no infinity or NaN from
// padding reaches a product.
#include <type_traits>

#include "attn_device.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// Where the next step's global loads are issued. At d = 64 after the
// probabilities are formed (shorter register lifetimes, measured faster); at
// d = 128 at the top of the step (the later point raises the peak register
// count past the two-work-groups-per-CU budget).
template <int D> constexpr bool kLateLoads = D == 64;

// LDS operands read three MFMAs ahead of their product through a register
// ring (mfma_stream) at d = 64. At d = 128 the ring fits only where direct
// loads free the staging registers (kDqRing, kDkdvRing2 below).
template <int D> constexpr bool kOperandRing = D == 64;

// dQ at d = 128 stages its K and V tiles with direct-to-LDS loads (waves 0-3
// K, waves 4-7 V, 16 rows each), which frees the 16 staging registers per
// thread the operand ring needs there.
template <int D> constexpr bool kDqDma = D == 128;
template <int D> constexpr bool kDqRing = kOperandRing<D> || kDqDma<D>;
// dK/dV at d = 128 likewise: Q and dO tiles by direct loads (waves 0-3 Q,
// 4-7 dO, 8 rows each), and the operand ring on the dV/dK products, whose
// operands all come from LDS.
template <int D> constexpr bool kDkdvDma = D == 128;
template <int D> constexpr bool kDkdvRing2 = kOperandRing<D> || kDkdvDma<D>;

__device__ __forceinline__ int pi_row(int i) { return (i & ~12) | ((i >> 1) & 4) | ((i << 1) & 8); }

// Row-major tile of R rows x D elements in LDS, 16-byte chunks XOR-swizzled
// per row (chunk_swz): element (r, c) lives at r * D + 8 * ((c / 8) ^ swz(r)) + c % 8.
template <int D>
__device__ __forceinline__ int tile_off(int r, int chunk) {
  return r * D + 8 * (chunk ^ chunk_swz<D>(r));
}

// A operand of a product contracting over the tile's rows: lane (m, h) of
// 16-row step ks, M-tile mt gets rows 16 ks + 8 h .. +7 of column 32 mt + m,
// assembled from two transposing reads (rows +0..3 and +4..7).
template <int D>
__device__ __forceinline__ uint4 tile_tr_operand(const uint16_t *tile, int lane, int ks, int mt) {
  const int k = lane & 15, half = (lane >> 4) & 1, hl = lane >> 5;
  const int c = 4 * mt + 2 * half + ((k & 3) >> 1);
  const int r0 = 16 * ks + 8 * hl + (k >> 2);
  const uint2 a = lds_tr4(tile + tile_off<D>(r0, c) + 4 * (k & 1));
  const uint2 b = lds_tr4(tile + tile_off<D>(r0 + 4, c) + 4 * (k & 1));
  return make_uint4(a.x, a.y, b.x, b.y);
}

// A operand of a product contracting over d: lane (n, h) of 32-row tile t,
// k-step kk gets row 32 t + pi(n), elements 16 kk + 8 h .. +7.
template <int D>
__device__ __forceinline__ uint4 tile_row_operand(const uint16_t *tile, int lane, int t, int kk) {
  const int r = 32 * t + pi_row(lane & 31);
  return lds16(tile + tile_off<D>(r, 2 * kk + (lane >> 5)));
}

// ---------------------------------------------------------------------------
// -D = -rowsum(dO o O) and L2 = L * log2(e) (+inf for a row that sees no key)
// per (batch, head, query) row, rows padded to Sq_pad with -D = 0, L2 = +inf.
// D is stored negated: bwd_dkdv starts its dP accumulators from it.
template <int D>
__global__ void __launch_bounds__(256)
bwd_pre(const uint16_t *__restrict__ o, const uint16_t *__restrict__ dout, const float *__restrict__ lse,
        float *__restrict__ l2ws, float *__restrict__ dws, int B, int Sq, int Sq_pad, int Hq, bool f16) {
  constexpr int LPR = D / 8;  // lanes per row
  const int rows_per_block = 256 / LPR;
  const long long total = (long long)B * Hq * Sq_pad;
  const int sub = threadIdx.x % LPR;
  for (long long row = (long long)blockIdx.x * rows_per_block + threadIdx.x / LPR; row < total;
       row += (long long)gridDim.x * rows_per_block) {
    const int i = (int)(row % Sq_pad);
    const long long bh = row / Sq_pad;
    const int h = (int)(bh % Hq), b = (int)(bh / Hq);
    float acc = 0.f, l2 = __builtin_inff();
    if (i < Sq) {
      const size_t off = ((size_t)((size_t)b * Sq + i) * Hq + h) * D + 8 * sub;
      const uint4 ov = ldg16(o + off), gv = ldg16(dout + off);
      const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float o0, o1, g0, g1;
        if (f16) {
          const f16x2 a = __builtin_bit_cast(f16x2, ow[e]), c = __builtin_bit_cast(f16x2, gw[e]);
          o0 = (float)a[0], o1 = (float)a[1], g0 = (float)c[0], g1 = (float)c[1];
        } else {
          o0 = __uint_as_float(ow[e] << 16), o1 = __uint_as_float(ow[e] & 0xffff0000u);
          g0 = __uint_as_float(gw[e] << 16), g1 = __uint_as_float(gw[e] & 0xffff0000u);
        }
        acc = __builtin_fmaf(o0, g0, acc);
        acc = __builtin_fmaf(o1, g1, acc);
      }
      const float L = lse[(size_t)bh * Sq + i];
      l2 = L == kNegInf ? __builtin_inff() : L * kLog2e;
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (sub == 0) {
      dws[row] = i < Sq ? -acc : 0.f;
      l2ws[row] = l2;
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV. Work-group = 4 waves x 32 keys = one 128-key tile of (b, KV head g);
// query tiles of 32 rows of each of the G query heads of g pass through LDS.
constexpr int kQB = 32;   // query rows per dK/dV step
// Keys per dK/dV work-group (32 per wave) and its threads. At d = 128 eight
// waves share each staged Q/dO tile (one work-group per CU, two waves per
// SIMD); at d = 64 four (two work-groups per CU).
template <int D> constexpr int kKT = D == 128 ? 256 : 128;
template <int D> constexpr int kDkdvThreads = 2 * kKT<D>;

template <int D, bool F16>
__global__ void __launch_bounds__(kDkdvThreads<D>, kDkdvThreads<D> == 512 ? 1 : 2)
bwd_dkdv(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
         const uint16_t *__restrict__ dout, const float *__restrict__ l2ws, const float *__restrict__ dws,
         uint16_t *__restrict__ dk, uint16_t *__restrict__ dv, const int *__restrict__ cu_q,
         const int *__restrict__ cu_k, int total_q, int total_k, int Sq, int Sq_pad, int Sk, int Hq, int Hkv,
         int causal, float scale_log2, float scale, int BHkv) {
  constexpr int KST = D / 16, MT = D / 32, CH = D / 8;
  constexpr int QT = kQB * D;                 // one Q (or dO) tile, elements
  constexpr int NTH = kDkdvThreads<D>, KTL = kKT<D>;
  constexpr int LPT = kQB * CH / NTH;         // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * QT];  // {Q, dO} x 2 slots
  __shared__ __attribute__((aligned(16))) float stat[2][2][kQB];       // {L2, D} of the step's rows x 2 slots
  constexpr bool kVinLds = D == 128;  // V rows as an LDS tile instead of registers (register budget)
  __shared__ __attribute__((aligned(16))) uint16_t vres[kVinLds ? KTL * D : 8];

  const int x = blockIdx.x;
  const int kt = x / BHkv;  // key tile 0 first: under a causal mask it has the most queries
  const int u = x % BHkv;
  const int b = u / Hkv, g = u % Hkv;
  const int G = Hq / Hkv;
  // Rows of sequence b (dense [B][S] blocks, or packed offsets clamped to the
  // totals) and its row statistics in the workspace: [B][Hq][Sq_pad] dense,
  // [Hq][Sq_pad] over the packed rows.
  int qbase, kbase;
  size_t stat_b;
  if (cu_q != nullptr) {
    const int a0 = min(max(cu_q[b], 0), total_q), a1 = min(max(cu_q[b + 1], a0), total_q);
    const int c0 = min(max(cu_k[b], 0), total_k), c1 = min(max(cu_k[b + 1], c0), total_k);
    qbase = a0, Sq = a1 - a0, kbase = c0, Sk = c1 - c0, stat_b = (size_t)a0;
    if (kt * KTL >= Sk) return;  // the whole work-group: this sequence has fewer key tiles
  } else {
    qbase = b * Sq, kbase = b * Sk, stat_b = (size_t)b * Hq * Sq_pad;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hl = lane >> 5;
  const int k0 = kt * KTL, kw0 = k0 + 32 * w;  // first key of the tile, of the wave
  const int key = kw0 + n;
  const int off = Sk - Sq;

  // This lane's K and V row as B operands (d contracted), zero past Sk.
  uint4 kop[KST], vop[kVinLds ? 1 : KST];
  {
    const size_t roff = ((size_t)((size_t)kbase + (key < Sk ? key : 0)) * Hkv + g) * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      const bool ok = key < Sk;
      kop[kk] = ok ? ldg16(k + roff + (2 * kk + hl) * 8) : make_uint4(0, 0, 0, 0);
      if constexpr (!kVinLds) vop[kk] = ok ? ldg16(v + roff + (2 * kk + hl) * 8) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (kVinLds) {
      // The work-group's 128 V rows, swizzled like the streamed tiles; read
      // row-wise (16 consecutive rows per chunk) as the dP operand.
      const size_t vbase = ((size_t)kbase * Hkv + g) * D;
      for (int c = tid; c < KTL * CH; c += NTH) {
        const int r = c / CH, ch = c % CH, kr = k0 + r;
        const uint4 val = kr < Sk ? ldg16(v + vbase + (size_t)kr * Hkv * D + ch * 8) : make_uint4(0, 0, 0, 0);
        sts16(vres + tile_off<D>(r, ch), val);
      }
    }
  }
  f32x16 dkT[MT], dvT[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkT[mt][r] = 0.f, dvT[mt][r] = 0.f;

  // Query rows that can see a key of this tile: i >= k0 - off (all if not causal).
  const int i_first = causal ? max(0, k0 - off) : 0;
  const int ib0 = i_first / kQB, nqb = (Sq + kQB - 1) / kQB;
  const int nsteps = ib0 < nqb ? (nqb - ib0) * G : 0;
  const int wave_first_i = causal ? kw0 - off : -0x40000000;  // first query that sees the wave's first key

  const size_t rstride = (size_t)Hq * D;
  const int tg = tid, trow = tg / CH, tch = tg % CH;
  uint4 sq[kDkdvDma<D> ? 1 : LPT], sdo[kDkdvDma<D> ? 1 : LPT];
  float sst;  // threads 0-63: the L2 (0-31) or D (32-63) value of one of the step's rows
  // Direct loads (d = 128): load i of wave w fills rows 8 (w % 4) + 4 i .. +3
  // of the Q (w < 4) or dO tile; lane l fetches the chunk that the swizzle
  // places at chunk l % 16 of its row.
  int dvoff[kDkdvDma<D> ? 2 : 1];
  if constexpr (kDkdvDma<D>) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * (w & 3) + 4 * i + lane / CH;
      dvoff[i] = (int)((r * rstride + 8 * ((lane % CH) ^ chunk_swz<D>(r))) * 2);
    }
  }
  auto dma_step = [&](int st) {
    const int hh = st / (nqb - ib0), ib = ib0 + st % (nqb - ib0);
    const int h = g * G + hh;
    if (tid < 64) sst = (tid < 32 ? l2ws : dws)[stat_b + (size_t)h * Sq_pad + ib * kQB + (tid & 31)];
    const long long base = ((long long)qbase * Hq + h) * D + (long long)ib * kQB * rstride;
    const long long left = ((long long)Sq * Hq - h) * D * 2 - (long long)ib * kQB * rstride * 2;
    const auto rs = uniform_buffer_rsrc((w < 4 ? q : dout) + base, left);
    const unsigned tile = lds_offset(smem + (st & 1) * 2 * QT + (w < 4 ? 0 : QT)) + 8 * (w & 3) * D * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16(rs, dvoff[i], tile + 4 * i * D * 2);
  };
  auto load_step = [&](int st) {
    const int hh = st / (nqb - ib0), ib = ib0 + st % (nqb - ib0);
    const int h = g * G + hh;
    if (tid < 64) sst = (tid < 32 ? l2ws : dws)[stat_b + (size_t)h * Sq_pad + ib * kQB + (tid & 31)];
    const long long base = ((long long)qbase * Hq + h) * D + (long long)ib * kQB * rstride;
    const long long left = ((long long)Sq * Hq - h) * D * 2 - (long long)ib * kQB * rstride * 2;
    const auto rq = buffer_rsrc(q + base, left), rd = buffer_rsrc(dout + base, left);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int boff = (int)(((trow + i * (NTH / CH)) * rstride + tch * 8) * 2);
      sq[i] = buf_load16(rq, boff);
      sdo[i] = buf_load16(rd, boff);
    }
  };
  auto store_step = [&](int slot) {
    uint16_t *qt = smem + slot * 2 * QT, *dt = qt + QT;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int r = trow + i * (NTH / CH);
      sts16(qt + tile_off<D>(r, tch), sq[i]);
      sts16(dt + tile_off<D>(r, tch), sdo[i]);
    }
    if (tid < 64) stat[slot][tid >> 5][tid & 31] = sst;
  };

  if constexpr (kDkdvDma<D>) {
    if (nsteps > 0) dma_step(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), seen by the compiler: none of its loads is pending in the loop
    if (nsteps > 0 && tid < 64) stat[0][tid >> 5][tid & 31] = sst;
  } else if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    if constexpr (kDkdvDma<D>) {
      if (st + 1 < nsteps) dma_step(st + 1);  // into the slot step st - 1 held, read before the last barrier
    } else if constexpr (!kLateLoads<D>) {
      if (st + 1 < nsteps) load_step(st + 1);
    }
    const int ib = ib0 + st % (nqb - ib0);
    const int i0 = ib * kQB;
    const uint16_t *qt = smem + (st & 1) * 2 * QT, *dt = qt + QT;
    // Skip when every query of the step is before the wave's first visible one.
    const bool active = i0 + kQB - 1 >= wave_first_i && kw0 < Sk;
    if (active) {
      // The two waves of a SIMD share its matrix unit: a wave issuing MFMAs
      // runs at raised priority, so the other's softmax work fills the gaps
      // instead of competing with it.
      __builtin_amdgcn_s_setprio(2);
      // dP starts from -D (stored negated by bwd_pre), so the MFMAs leave
      // dP - D and dS = P o dP needs no subtraction.
      f32x16 S, dP;
      {
        const float *dpn = &stat[st & 1][1][8 * hl];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float4 na = *reinterpret_cast<const float4 *>(dpn + 16 * hf);
          const float4 nb = *reinterpret_cast<const float4 *>(dpn + 16 * hf + 4);
          dP[8 * hf + 0] = na.x, dP[8 * hf + 1] = na.y, dP[8 * hf + 2] = na.z, dP[8 * hf + 3] = na.w;
          dP[8 * hf + 4] = nb.x, dP[8 * hf + 5] = nb.y, dP[8 * hf + 6] = nb.z, dP[8 * hf + 7] = nb.w;
        }
      }
      if constexpr (kOperandRing<D> && !kVinLds) {
        // S^T = K Q^T and dP^T = V dO^T as one stream (Q and dO rows from LDS).
        mfma_stream<2 * KST, 3>(
            [&](auto gc) {
              constexpr int g = decltype(gc)::value;
              return tile_row_operand<D>(g % 2 ? dt : qt, lane, 0, g / 2);
            },
            [&](auto gc, const uint4 &a) {
              constexpr int g = decltype(gc)::value, kk = g / 2;
              if constexpr (g % 2 == 0) S = mma32<F16>(a, kop[kk], kk == 0 ? f32x16{} : S);
              else dP = mma32<F16>(a, vop[kk], dP);
            });
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) {
          S = mma32<F16>(tile_row_operand<D>(qt, lane, 0, kk), kop[kk], S);
          uint4 vb;
          if constexpr (kVinLds) vb = lds16(vres + tile_off<D>(32 * w + n, 2 * kk + hl));
          else vb = vop[kk];
          dP = mma32<F16>(tile_row_operand<D>(dt, lane, 0, kk), vb, dP);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // Register r holds query i0 + 16 (r / 8) + 8 hl + r % 8.
      const float *l2p = &stat[st & 1][0][8 * hl];
      const int lim = causal ? key - off : -0x40000000;  // query i sees this key iff i >= lim
      uint4 pP[2], pS[2];
      {
        // Only steps that cut the visible region (the causal diagonal, rows
        // past Sq, keys past Sk) run the per-element test, which sets masked
        // scores to -inf: P = 0, and dS = 0 * finite (padded rows and keys
        // read zeros). The row statistics are read per half, next to their use.
        if (!(kw0 + 31 < Sk && i0 + kQB - 1 < Sq && (!causal || i0 >= kw0 + 31 - off))) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = i0 + 16 * (r / 8) + 8 * hl + r % 8;
            S[r] = key < Sk && qi < Sq && qi >= lim ? S[r] : kNegInf;
          }
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float pv[8], sv[8];
          const float4 la = *reinterpret_cast<const float4 *>(l2p + 16 * hf);
          const float4 lb = *reinterpret_cast<const float4 *>(l2p + 16 * hf + 4);
          const float lh[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * hf + e;
            const float p = exp2_hw(__builtin_fmaf(S[r], scale_log2, -lh[e]));
            pv[e] = p;
            sv[e] = p * dP[r];
          }
          pP[hf] = make_uint4(pack2<F16>(pv[0], pv[1]), pack2<F16>(pv[2], pv[3]), pack2<F16>(pv[4], pv[5]),
                              pack2<F16>(pv[6], pv[7]));
          pS[hf] = make_uint4(pack2<F16>(sv[0], sv[1]), pack2<F16>(sv[2], sv[3]), pack2<F16>(sv[4], sv[5]),
                              pack2<F16>(sv[6], sv[7]));
        }
      }
      if constexpr (kLateLoads<D>) {
        if (st + 1 < nsteps) load_step(st + 1);
      }
      __builtin_amdgcn_s_setprio(2);
      if constexpr (kDkdvRing2<D>) {
        // dV^T += dO^T P^T and dK^T += Q^T dS^T as one stream.
        mfma_stream<4 * MT, 3>(
            [&](auto gc) {
              constexpr int g = decltype(gc)::value, mt = g / 4, ks = (g / 2) % 2;
              return tile_tr_operand<D>(g % 2 ? qt : dt, lane, ks, mt);
            },
            [&](auto gc, const uint4 &a) {
              constexpr int g = decltype(gc)::value, mt = g / 4, ks = (g / 2) % 2;
              if constexpr (g % 2 == 0) dvT[mt] = mma32<F16>(a, pP[ks], dvT[mt]);
              else dkT[mt] = mma32<F16>(a, pS[ks], dkT[mt]);
            });
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            dvT[mt] = mma32<F16>(tile_tr_operand<D>(dt, lane, ks, mt), pP[ks], dvT[mt]);
            dkT[mt] = mma32<F16>(tile_tr_operand<D>(qt, lane, ks, mt), pS[ks], dkT[mt]);
          }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (kLateLoads<D>) {
      if (!active && st + 1 < nsteps) load_step(st + 1);
    }
    if constexpr (kDkdvDma<D>) {
      if (st + 1 < nsteps) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // step st + 1's tiles are in LDS before the barrier
        if (tid < 64) stat[(st + 1) & 1][tid >> 5][tid & 31] = sst;
      }
    } else {
      if (st + 1 < nsteps) store_step((st + 1) & 1);
    }
    __syncthreads();
  }

  if (key >= Sk) return;
  const size_t ooff = ((size_t)((size_t)kbase + key) * Hkv + g) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dd = 32 * mt + 8 * a + 4 * hl;
      *reinterpret_cast<uint2 *>(dk + ooff + dd) =
          make_uint2(pack2<F16>(dkT[mt][4 * a] * scale, dkT[mt][4 * a + 1] * scale),
                     pack2<F16>(dkT[mt][4 * a + 2] * scale, dkT[mt][4 * a + 3] * scale));
      *reinterpret_cast<uint2 *>(dv + ooff + dd) =
          make_uint2(pack2<F16>(dvT[mt][4 * a], dvT[mt][4 * a + 1]), pack2<F16>(dvT[mt][4 * a + 2], dvT[mt][4 * a + 3]));
    }
}

// ---------------------------------------------------------------------------
// dQ. Work-group = 4 waves x 32 query rows = one 128-row tile of (b, head h);
// 64-key K and V tiles pass through LDS.
// Query rows per dQ work-group (32 per wave) and its threads, as for dK/dV:
// eight waves at d = 128, four at d = 64.
template <int D> constexpr int kQT = D == 128 ? 256 : 128;
template <int D> constexpr int kDqThreads = 2 * kQT<D>;
constexpr int kKB = 64;    // keys per dQ step

constexpr int kPad = 128;  // row padding of the statistics workspace

template <int D, bool F16>
__global__ void __launch_bounds__(kDqThreads<D>, kDqThreads<D> == 512 ? 1 : 2)
bwd_dq(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
       const uint16_t *__restrict__ dout, const float *__restrict__ l2ws, const float *__restrict__ dws,
       uint16_t *__restrict__ dq, const int *__restrict__ cu_q, const int *__restrict__ cu_k, int total_q,
       int total_k, int Sq, int Sq_pad, int Sk, int Hq, int Hkv, int causal, float scale_log2, float scale,
       int n_qtiles, int BH) {
  constexpr int KST = D / 16, MT = D / 32, CH = D / 8;
  constexpr int KTL = kKB * D;          // one K (or V) tile, elements
  constexpr int NTH = kDqThreads<D>, QTL = kQT<D>;
  constexpr int LPT = kKB * CH / NTH;   // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * KTL];  // {K, V} x 2 slots

  const int x = blockIdx.x;
  const int qt_ = n_qtiles - 1 - x / BH;  // last query tile first: the longest key range under a causal mask
  const int u = x % BH;
  const int b = u / Hq, h = u % Hq;
  const int gk = h / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hl = lane >> 5;
  const int q0 = qt_ * QTL, r0 = q0 + 32 * w;
  const int qrow = r0 + n;
  int qbase, kbase;  // as in bwd_dkdv
  size_t stat_b;
  if (cu_q != nullptr) {
    const int a0 = min(max(cu_q[b], 0), total_q), a1 = min(max(cu_q[b + 1], a0), total_q);
    const int c0 = min(max(cu_k[b], 0), total_k), c1 = min(max(cu_k[b + 1], c0), total_k);
    qbase = a0, Sq = a1 - a0, kbase = c0, Sk = c1 - c0, stat_b = (size_t)a0;
    if (q0 >= Sq) return;  // the whole work-group: this sequence has fewer query tiles
  } else {
    qbase = b * Sq, kbase = b * Sk, stat_b = (size_t)b * Hq * Sq_pad;
  }
  const int off = Sk - Sq;

  uint4 qop[KST], doop[KST];
  {
    const bool ok = qrow < Sq;
    const size_t roff = ((size_t)((size_t)qbase + (ok ? qrow : 0)) * Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      qop[kk] = ok ? ldg16(q + roff + (2 * kk + hl) * 8) : make_uint4(0, 0, 0, 0);
      doop[kk] = ok ? ldg16(dout + roff + (2 * kk + hl) * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  // A row past Sq reads the last row's values (it is masked whatever it
  // reads), so every read stays inside the sequence's statistics.
  const int qs = min(qrow, Sq - 1);
  const float l2 = l2ws[stat_b + (size_t)h * Sq_pad + qs];
  const float nDr = dws[stat_b + (size_t)h * Sq_pad + qs];  // -D
  // At d = 64 the dP MFMAs start from -D (the lane's query row), so dS = P o dP
  // needs no addition; at d = 128 the 16 registers are not free.
  constexpr bool kFoldD = D == 64;
  f32x16 ndv;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndv[r] = nDr;
  f32x16 dqT[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqT[mt][r] = 0.f;

  int kend = causal ? min(Sk, q0 + QTL + off) : Sk;  // keys any row of the tile sees
  if (kend < 0) kend = 0;
  const int nblk = (kend + kKB - 1) / kKB;
  // Keys a row of this wave can see: j <= r0 + 31 + off.
  const int wave_kend = causal ? min(Sk, r0 + 32 + off) : Sk;
  const int lim = causal ? qrow + off : 0x3fffffff;  // this row sees keys j <= lim

  const size_t rstride = (size_t)Hkv * D;
  const int trow = tid / CH, tch = tid % CH;
  // Direct loads (d = 128): load i of wave w (group w / 4: K or V) fills rows
  // 16 (w % 4) + 4 i .. +3 of the tile, lane l fetching the chunk that the
  // swizzle places at chunk l % 16 of row 4 i + l / 16.
  int dvoff[kDqDma<D> ? 4 : 1];
  if constexpr (kDqDma<D>) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * (w & 3) + 4 * i + lane / CH;
      dvoff[i] = (int)((r * rstride + 8 * ((lane % CH) ^ chunk_swz<D>(r))) * 2);
    }
  }
  auto dma_blk = [&](int blk) {
    const long long base = ((long long)kbase * Hkv + gk) * D + (long long)blk * kKB * rstride;
    const long long left = ((long long)Sk * Hkv - gk) * D * 2 - (long long)blk * kKB * rstride * 2;
    const auto rs = buffer_rsrc((w < 4 ? k : v) + base, left);
    const unsigned tile = lds_offset(smem + (blk & 1) * 2 * KTL + (w < 4 ? 0 : KTL)) + 16 * (w & 3) * D * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(rs, dvoff[i], tile + 4 * i * D * 2);
  };
  uint4 sk[kDqDma<D> ? 1 : LPT], sv[kDqDma<D> ? 1 : LPT];
  auto load_blk = [&](int blk) {
    const long long base = ((long long)kbase * Hkv + gk) * D + (long long)blk * kKB * rstride;
    const long long left = ((long long)Sk * Hkv - gk) * D * 2 - (long long)blk * kKB * rstride * 2;
    const auto rk = buffer_rsrc(k + base, left), rv = buffer_rsrc(v + base, left);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int boff = (int)(((trow + i * (NTH / CH)) * rstride + tch * 8) * 2);
      sk[i] = buf_load16(rk, boff);
      sv[i] = buf_load16(rv, boff);
    }
  };
  auto store_blk = [&](int slot) {
    uint16_t *ktl = smem + slot * 2 * KTL, *vtl = ktl + KTL;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int r = trow + i * (NTH / CH);
      sts16(ktl + tile_off<D>(r, tch), sk[i]);
      sts16(vtl + tile_off<D>(r, tch), sv[i]);
    }
  };

  if constexpr (kDqDma<D>) {
    if (nblk > 0) dma_blk(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), seen by the compiler: none of its loads is pending in the loop
  } else if (nblk > 0) {
    load_blk(0);
    store_blk(0);
  }
  __syncthreads();
  for (int j = 0; j < nblk; ++j) {
    if constexpr (kDqDma<D>) {
      if (j + 1 < nblk) dma_blk(j + 1);  // into the slot block j - 1 held, read before the last barrier
    } else if constexpr (!kLateLoads<D>) {
      if (j + 1 < nblk) load_blk(j + 1);
    }
    const int j0 = j * kKB;
    const uint16_t *ktl = smem + (j & 1) * 2 * KTL, *vtl = ktl + KTL;
    const bool active = j0 < wave_kend;
    if (active) {
      __builtin_amdgcn_s_setprio(2);
      // S = K Q^T and dP = V dO^T for the two 32-key halves.
      f32x16 S[2], dP[2];
      if constexpr (kDqRing<D>) {
        mfma_stream<4 * KST, 3>(
            [&](auto gc) {
              constexpr int g = decltype(gc)::value, t = g / (2 * KST), kk = (g / 2) % KST;
              return tile_row_operand<D>(g % 2 ? vtl : ktl, lane, t, kk);
            },
            [&](auto gc, const uint4 &a) {
              constexpr int g = decltype(gc)::value, t = g / (2 * KST), kk = (g / 2) % KST;
              if constexpr (g % 2 == 0) S[t] = mma32<F16>(a, qop[kk], kk == 0 ? f32x16{} : S[t]);
              else dP[t] = mma32<F16>(a, doop[kk], kk == 0 ? (kFoldD ? ndv : f32x16{}) : dP[t]);
            });
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int r = 0; r < 16; ++r) S[t][r] = 0.f, dP[t][r] = 0.f;
#pragma unroll
          for (int kk = 0; kk < KST; ++kk) {
            S[t] = mma32<F16>(tile_row_operand<D>(ktl, lane, t, kk), qop[kk], S[t]);
            dP[t] = mma32<F16>(tile_row_operand<D>(vtl, lane, t, kk), doop[kk], dP[t]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // Register r of tile t holds key j0 + 32 t + 16 (r / 8) + 8 hl + r % 8.
      uint4 pS[4];
      {
        // As in bwd_dkdv: the per-element test only where the block cuts the
        // visible region, setting masked scores to -inf.
        if (!(j0 + kKB - 1 < Sk && r0 + 31 < Sq && (!causal || j0 + kKB - 1 <= r0 + off))) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kj = j0 + 32 * t + 16 * (r / 8) + 8 * hl + r % 8;
              S[t][r] = kj < Sk && kj <= lim && qrow < Sq ? S[t][r] : kNegInf;
            }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float sv8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * hf + e;
              sv8[e] = exp2_hw(__builtin_fmaf(S[t][r], scale_log2, -l2)) * (kFoldD ? dP[t][r] : dP[t][r] + nDr);
            }
            pS[2 * t + hf] = make_uint4(pack2<F16>(sv8[0], sv8[1]), pack2<F16>(sv8[2], sv8[3]),
                                        pack2<F16>(sv8[4], sv8[5]), pack2<F16>(sv8[6], sv8[7]));
          }
      }
      if constexpr (kLateLoads<D>) {
        if (j + 1 < nblk) load_blk(j + 1);
      }
      __builtin_amdgcn_s_setprio(2);
      if constexpr (kDqRing<D>) {
        mfma_stream<4 * MT, 3>(
            [&](auto gc) {
              constexpr int g = decltype(gc)::value;
              return tile_tr_operand<D>(ktl, lane, g % 4, g / 4);
            },
            [&](auto gc, const uint4 &a) {
              constexpr int g = decltype(gc)::value;
              dqT[g / 4] = mma32<F16>(a, pS[g % 4], dqT[g / 4]);
            });
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) dqT[mt] = mma32<F16>(tile_tr_operand<D>(ktl, lane, ks, mt), pS[ks], dqT[mt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (kLateLoads<D>) {
      if (!active && j + 1 < nblk) load_blk(j + 1);
    }
    if constexpr (kDqDma<D>) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // block j + 1 is in LDS before the barrier
    } else {
      if (j + 1 < nblk) store_blk((j + 1) & 1);
    }
    __syncthreads();
  }

  if (qrow >= Sq) return;
  uint16_t *dst = dq + ((size_t)((size_t)qbase + qrow) * Hq + h) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dd = 32 * mt + 8 * a + 4 * hl;
      *reinterpret_cast<uint2 *>(dst + dd) =
          make_uint2(pack2<F16>(dqT[mt][4 * a] * scale, dqT[mt][4 * a + 1] * scale),
                     pack2<F16>(dqT[mt][4 * a + 2] * scale, dqT[mt][4 * a + 3] * scale));
    }
}

}  // namespace

int bwd_sq_pad(int Sq) { return (Sq + kPad - 1) / kPad * kPad; }
// Packed batches: one [Hq][pad] statistics block over all rows, padded past
// the last row (a dK/dV step reads its 32 rows from any starting row).
int bwd_varlen_pad(int total_q) { return (total_q + kPad + kPad - 1) / kPad * kPad; }

// Dense when cu_q == nullptr: Sq, Sk are the per-sequence lengths. Packed
// otherwise: Sq, Sk are the longest lengths (they size the grids) and
// total_q, total_k the packed row counts.
hipError_t launch_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                      void *dq, void *dk, void *dv, const int *cu_q, const int *cu_k, int total_q, int total_k,
                      int causal, int batch, int Sq, int Sk, int Hq, int Hkv, int d, float *l2ws, float *dws, bool f16,
                      hipStream_t stream) {
  const auto *qq = static_cast<const uint16_t *>(q);
  const auto *kk = static_cast<const uint16_t *>(k);
  const auto *vv = static_cast<const uint16_t *>(v);
  const auto *oo = static_cast<const uint16_t *>(o);
  const auto *gg = static_cast<const uint16_t *>(dout);
  const bool packed = cu_q != nullptr;
  const int Sq_pad = packed ? bwd_varlen_pad(total_q) : bwd_sq_pad(Sq);
  const float scale = 1.f / sqrtf((float)d), scale_log2 = scale * kLog2e;
  {
    // Row statistics: a packed batch is one sequence of total_q rows here.
    const int pb = packed ? 1 : batch, psq = packed ? total_q : Sq;
    const long long rows = (long long)pb * Hq * Sq_pad;
    const int rows_per_block = 256 / (d / 8);
    const long long blocks = (rows + rows_per_block - 1) / rows_per_block;
    const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
    if (d == 128)
      hipLaunchKernelGGL(bwd_pre<128>, grid, dim3(256), 0, stream, oo, gg, lse, l2ws, dws, pb, psq, Sq_pad, Hq, f16);
    else
      hipLaunchKernelGGL(bwd_pre<64>, grid, dim3(256), 0, stream, oo, gg, lse, l2ws, dws, pb, psq, Sq_pad, Hq, f16);
  }
  const int BHkv = batch * Hkv, BH = batch * Hq;
  const int kt_keys = d == 128 ? kKT<128> : kKT<64>, qt_rows = d == 128 ? kQT<128> : kQT<64>;
  const int n_ktiles = (Sk + kt_keys - 1) / kt_keys, n_qtiles = (Sq + qt_rows - 1) / qt_rows;
  auto dkdv = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(n_ktiles * BHkv), dim3(2 * kt_keys), 0, stream, qq, kk, vv, gg, l2ws, dws,
                       static_cast<uint16_t *>(dk), static_cast<uint16_t *>(dv), cu_q, cu_k, total_q, total_k, Sq,
                       Sq_pad, Sk, Hq, Hkv, causal, scale_log2, scale, BHkv);
  };
  auto dqk = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(n_qtiles * BH), dim3(2 * qt_rows), 0, stream, qq, kk, vv, gg, l2ws, dws,
                       static_cast<uint16_t *>(dq), cu_q, cu_k, total_q, total_k, Sq, Sq_pad, Sk, Hq, Hkv, causal,
                       scale_log2, scale, n_qtiles, BH);
  };
  if (d == 128) {
    if (f16) dkdv(bwd_dkdv<128, true>), dqk(bwd_dq<128, true>);
    else dkdv(bwd_dkdv<128, false>), dqk(bwd_dq<128, false>);
  } else {
    if (f16) dkdv(bwd_dkdv<64, true>), dqk(bwd_dq<64, true>);
    else dkdv(bwd_dkdv<64, false>), dqk(bwd_dq<64, false>);
  }
  return hipGetLastError();
}

}  // namespace attn

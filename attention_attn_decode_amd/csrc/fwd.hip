// Prefill attention forward for gfx950 (MFMA-bound).
//
// Pages cited by title and section:
//   [FA4-decode] "Optimization diaries: S/P ping-pong for FlashAttention-4 decode"
//   [GQA-SM100]  "Building a Faster GQA Decode Kernel for Blackwell SM100"
//   [FA4-edges]  "Flash Attention 4 — warp-role choreography and the edges"
//
// Same inner loop as decode, widened: S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_bf16, each wave owning 32 query columns. A work-group
// of eight waves owns a 256-row query tile and shares 64-key K and V tiles
// in LDS (32-key tiles at d = 256): three slots each of dense, chunk-swizzled
// rows filled by direct-to-LDS loads at d >= 128, two slots of padded rows
// filled through registers at d = 64. K and V stay row-major in LDS; the P*V
// operand, which needs keys along its k dimension, is read with the
// transposing ds_read_b64_tr_b16.
//
// Causal masking ([FA4-edges] §Edge 1 · causal masking): per (query strip,
// key block) the block is fully visible, on the diagonal (masked to -inf
// before the max), or skipped; a work-group only walks keys [0, kend) and a
// wave skips the math of blocks entirely in its future.
// Scheduling ([FA4-edges] §Edge 3 · tile scheduling): tiles are numbered
// heaviest first (last query tile first, longest visible key range), a
// longest-processing-time order that shortens the tail. With batch * heads a
// multiple of 8, the tiles of one (batch, head) that run at the same time fall
// on one XCD (work-groups are dealt round-robin to the 8 XCDs), where they
// share that pair's K/V in the XCD's L2.
//
// Key order inside a 32-key score tile: MFMA row i holds key pi(i), where pi
// swaps bits 2 and 3 of i. Lane half h (= lane / 32) then finds, in registers
// 8k .. 8k + 7 of its accumulator, keys 16k + 8h .. 16k + 8h + 7: the eight
// contiguous keys of its P*V B operand for that 16-key step.
#include <type_traits>

#include "attn_device.h"

namespace attn {
namespace {

constexpr float kRescaleLog2 = 8.f;  // tolerated growth of the row max (base 2)

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

// Ping-pong schedule. A work-group of eight waves covers 256 query rows; waves
// 0-3 form group A and waves 4-7 group B, so every SIMD holds one wave of each.
// Each wave owns 32 query columns and alternates two phases per key block j:
//   MFMA phase j: O^T += V(j-1)^T P(j-1)^T, then S(j) = K(j) Q^T (32 MFMAs),
//                 with the group's share of the K/V staging under them
//   VALU phase j: softmax of S(j) into P(j) and the rescale of O^T.
// Group B runs one phase behind group A, so on each SIMD one wave issues
// MFMAs while the other runs its exponentials: the S/P ping-pong of
// [FA4-decode] §Recap on the FA4 forward pass, played between the two waves
// of a SIMD instead of two register sets. With direct-to-LDS staging
// (d >= 128) the groups meet at one work-group barrier per key block (group A
// runs MFMA(j) then softmax(j), group B softmax(j - 1) then MFMA(j)); with
// register staging (d = 64) at one per phase. K and V tiles are shared by all
// eight waves; group A stages K, group B stages V, each during its MFMA phase,
// ahead of use (one block through registers at d = 64, two half-steps by
// direct-to-LDS loads at d >= 128).
constexpr int kBMP = 256;  // query rows per work-group
// Keys per block: 64, or 32 at d = 256, where a block's score and probability
// registers must shrink to leave room for the 32-row Q operands and O^T; a
// phase still issues 32 MFMAs.
template <int D> constexpr int kBlockKeys = D == 256 ? 32 : 64;

// One 256-row query tile x (heaviest first: x / BH counts the query tiles
// back from the sequence's end, x % BH walks (sequence, head)) in the
// work-group's LDS block smem.
template <int D, bool F16>
__device__ __forceinline__ void
fwd_tile(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
         const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
         const int *__restrict__ cu_q, const int *__restrict__ cu_k, int total_q, int total_k,
         int Sq, int Sk, int Hq, int Hkv, int causal, float scale_log2, int n_mblocks, int BH, int x,
         uint16_t *smem) {
  constexpr int BN = kBlockKeys<D>;
  constexpr int CH = D / 8;        // 16-byte chunks per row
  // d = 128 and 256: K/V staged by direct-to-LDS buffer loads into three
  // slots of dense, chunk-swizzled rows; d = 64: through registers into two
  // slots of padded rows.
  constexpr bool kDma = D >= 128;
  constexpr int NSLOT = kDma ? 3 : 2;
  constexpr int KROW = kDma ? D : KRow<D>::v, VROW = kDma ? D : VRow<D>::v;
  constexpr int KT = BN * KROW, VT = BN * VROW;
  constexpr int RPT = 256 / CH;    // rows one group-wide (256-thread) load covers
  constexpr int NKL = BN / RPT;    // tile loads per thread per block
  constexpr int KST = D / 16;      // QK k-steps
  constexpr int MT = D / 32;       // O^T row tiles
  constexpr int NT = BN / 32;      // 32-key score tiles per block
  constexpr int NKS = BN / 16;     // 16-key P*V steps per block
  uint16_t *const ktile = smem;               // K slots
  uint16_t *const vtile = smem + NSLOT * KT;  // V slots

  const int te = x / BH;  // query tile counted from the sequence's end: the heaviest first
  const int u = x % BH;
  const int b = u / Hq, h = u % Hq;
  const int gk = h / (Hq / Hkv);
  // Rows of sequence b: dense batches are [B][S] blocks; a packed
  // variable-length batch gives each sequence's first row in cu_q / cu_k
  // (clamped to the packed totals, so any offsets stay inside the buffers).
  // LSE is [B][Hq][Sq] dense, [Hq][total_q] packed.
  int qbase, kbase, lse_hs;
  size_t lse_base;
  if (cu_q != nullptr) {
    const int a0 = min(max(cu_q[b], 0), total_q), a1 = min(max(cu_q[b + 1], a0), total_q);
    const int c0 = min(max(cu_k[b], 0), total_k), c1 = min(max(cu_k[b + 1], c0), total_k);
    qbase = a0, Sq = a1 - a0, kbase = c0, Sk = c1 - c0;
    lse_base = (size_t)qbase, lse_hs = total_q;
  } else {
    qbase = b * Sq, kbase = b * Sk;
    lse_base = (size_t)b * Hq * Sq, lse_hs = Sq;
  }
  // Tiles are aligned to the sequence's end, so a length that is not a
  // multiple of the tile leaves its partial tile first, where a causal mask
  // gives it the fewest key blocks; its rows before row 0 are idle like rows
  // past Sq.
  const int q0 = Sq - kBMP * (te + 1);
  if (q0 + kBMP <= 0) return;  // the whole work-group: this sequence has fewer query tiles
  // Wave index in a scalar register: every per-wave condition below (group,
  // key range, skipped blocks) is then a uniform branch, and the barriers
  // inside group-dependent code are passed by whole waves only.
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = w >> 2;  // 0: group A, 1: group B
  const int n = lane & 31, hl = lane >> 5;
  // 32-row strips alternate between the groups, which balances the causal
  // diagonal between them.
  const int r0 = q0 + 64 * (w & 3) + 32 * G;
  const int qrow = r0 + n;
  const int off = Sk - Sq;  // bottom-right alignment

  auto row_bound = [&](int row) {
    const int bnd = causal ? min(Sk, row + off + 1) : Sk;
    return bnd < 0 ? 0 : bnd;
  };
  int kend = causal ? min(Sk, q0 + kBMP + off) : Sk;
  if (kend < 0) kend = 0;
  const int nblk = (kend + BN - 1) / BN;
  const int bound = row_bound(qrow);
  // Blocks this wave computes: up to its last row inside the sequence; none
  // when all its rows lie past Sq or before row 0 (a partial tile), whose
  // results are never stored (the wave still stages its share and meets
  // every barrier).
  const int wave_lo = row_bound(r0), wave_hi = row_bound(min(r0 + 31, Sq - 1));
  const int nbw = r0 >= Sq || r0 + 31 < 0 ? 0 : min(nblk, (wave_hi + BN - 1) / BN);

  uint4 qop[KST];
  {
    const bool ok = qrow >= 0 && qrow < Sq;
    const uint16_t *qp = q + ((size_t)(qbase + (ok ? qrow : 0)) * Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) qop[kk] = ok ? ldg16(qp + (2 * kk + hl) * 8) : make_uint4(0, 0, 0, 0);
  }

  // Staging: group A moves K tiles, group B V tiles, through a buffer
  // descriptor per block whose base is the block's first row and whose size
  // ends with the sequence's last row. Rows past Sk read as zero (the mask
  // excludes them), and the only per-lane address is a constant offset: no
  // vector address arithmetic per load.
  const size_t rstride = (size_t)Hkv * D;
  const uint16_t *src = (G == 0 ? k : v) + ((size_t)kbase * Hkv + gk) * D;
  const long long src_bytes = ((long long)Sk * Hkv - gk) * D * 2;  // src to the end of sequence b
  uint16_t *const dtile = G == 0 ? ktile : vtile;
  const int drow = G == 0 ? KROW : VROW, dsize = G == 0 ? KT : VT;
  const int tg = tid & 255, trow = tg / CH, tcol = (tg % CH) * 8;
  const int voff = (int)((trow * rstride + tcol) * 2);
  auto slot_of = [](int blk) { return kDma ? blk % 3 : blk & 1; };
  auto rsrc_blk = [&](int blk) {
    const long long boff = (long long)blk * BN * (long long)rstride * 2;
    const long long left = src_bytes - boff;
    const int nrec = left <= 0 ? 0 : (left > 0x7fffffffLL ? 0x7fffffff : (int)left);
    return __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const char *>(src) + (left <= 0 ? 0 : boff)), (short)0, nrec, kBufferWord3);
  };
  uint4 sreg[kDma ? 1 : NKL];
  auto load_blk = [&](int blk) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_blk(blk);
#pragma unroll
    for (int qi = 0; qi < NKL; ++qi)
      sreg[qi] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + (int)(qi * RPT * rstride * 2), 0, 0));
  };
  auto store_blk = [&](int blk) {
    uint16_t *dst = dtile + slot_of(blk) * dsize + trow * drow + tcol;
#pragma unroll
    for (int qi = 0; qi < NKL; ++qi) sts16(dst + RPT * qi * drow, sreg[qi]);
  };
  // Direct-to-LDS staging (d >= 128): each wave of a group moves BN / 4 rows
  // of the block with buffer loads whose 64 lanes deposit 16 bytes each, in
  // lane order, at the LDS address in M0 (1 KB: four 256-byte rows at
  // d = 128, two 512-byte rows at d = 256). Lane l of load i therefore
  // fetches the chunk that the swizzle places at chunk l % CH of row
  // RPI i + l / CH. All offsets are per lane, so
  // the descriptor's range check zeroes rows past Sk. The compiler does not
  // see these writes: the waits that publish a slot are explicit.
  constexpr int RPI = 64 / CH;         // rows per load
  constexpr int RPW = BN / 4;          // rows per wave of its group
  constexpr int NI = RPW / RPI;        // loads per wave per block
  const int w4 = w & 3;
  int dvoff[kDma ? NI : 1];
  if constexpr (kDma) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rw = RPW * w4 + RPI * i + lane / CH;
      dvoff[i] = (int)((rw * rstride + 8 * ((lane % CH) ^ chunk_swz<D>(rw))) * 2);
    }
  }
  const unsigned lds_wave = lds_offset(dtile) + (unsigned)(RPW * w4 * D * 2);
  auto dma_blk = [&](int blk) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_blk(blk);
    const unsigned slotb = lds_wave + (unsigned)(slot_of(blk) * dsize * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i) lds_dma16(rs, dvoff[i], slotb + RPI * i * D * 2);
  };
  // Wait until at most one block's direct loads (the newest) are in flight.
  auto dma_wait_one = [&]() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI) : "memory"); };

  // Operand reads. Padded rows (d = 64): a lane base plus constants.
  // Swizzled rows (d = 128): chunk c of row r sits at chunk c ^ chunk_swz(r);
  // the rows one lane reads share their swizzle up to compile-time terms, so
  // each address is a lane base XOR a constant, plus a constant.
  const int pin = swap_bits23(n);
  const int k_lane = pin * KROW + hl * 8;
  const int trk = lane & 15, trhalf = (lane >> 4) & 1;
  const int v_lane = (8 * hl + (trk >> 2)) * VROW + 16 * trhalf + 4 * (trk & 3);
  const unsigned k_lane_b = lds_offset(ktile) + pin * D * 2 + 16 * (hl ^ chunk_swz<D>(pin));
  const unsigned v_lane_b = lds_offset(vtile) + (8 * hl + (trk >> 2)) * D * 2 +
                            16 * (((2 * trhalf + ((trk & 3) >> 1)) ^ (2 * hl)) | ((trk >> 2) << 2)) + 8 * (trk & 1);
  // K rows 32t + pi(n), 16-byte chunk 2kk + hl.
  auto kread = [&](int slot, int t, int kk) {
    if constexpr (kDma) return lds16_at(((k_lane_b + slot * KT * 2) ^ (kk << 5)) + t * 32 * D * 2);
    else return lds16(ktile + slot * KT + k_lane + 32 * t * KROW + 16 * kk);
  };
  // V^T operand of 16-key step ks and O^T row tile mt (two transposing reads
  // of rows 16ks + 8hl + trk/4 and 4 rows further).
  auto vread = [&](int slot, int ks, int mt) {
    uint2 t0, t1;
    if constexpr (kDma) {
      const unsigned bb = v_lane_b + slot * VT * 2;
      t0 = lds_tr4_at((bb ^ (mt << 6)) + 16 * ks * D * 2);
      t1 = lds_tr4_at((bb ^ ((mt << 6) | 16)) + (16 * ks + 4) * D * 2);
    } else {
      const uint16_t *vl = vtile + slot * VT + v_lane;
      t0 = lds_tr4(vl + 16 * ks * VROW + 32 * mt);
      t1 = lds_tr4(vl + (16 * ks + 4) * VROW + 32 * mt);
    }
    return make_uint4(t0.x, t0.y, t1.x, t1.y);
  };

  f32x16 S[NT];
  uint4 pop[NKS];
  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;

  auto qk = [&](int slot) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[t][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) S[t] = mma32<F16>(kread(slot, t, kk), qop[kk], S[t]);
    }
  };
  auto pv = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) oacc[mt] = mma32<F16>(vread(slot, ks, mt), pop[ks], oacc[mt]);
  };
  // Softmax of block j0 (register r of score tile t holds key
  // j0 + 32t + 16(r/8) + 8hl + (r%8)) into the bf16 P operands, with the
  // conditional rescale of O^T ([FA4-edges] §The correction).
  auto softmax = [&](int j0, auto masked) {
    if constexpr (decltype(masked)::value) {
      const int lim = bound - j0 - 8 * hl;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[t][r] = (32 * t + 16 * (r >> 3) + (r & 7)) < lim ? S[t][r] : kNegInf;
    }
    // Row max and row sum as four independent chains each (a single wave
    // issues this phase, so one long dependent chain would stall on latency).
    float mx[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx[r & 3] = fmaxf(mx[r & 3], S[t][r]);
    float mloc = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    mloc = wave_max_halves(mloc);
    const float mblk = mloc * scale_log2;
    const float m_new = mblk > m_run + kRescaleLog2 ? mblk : m_run;
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pv8[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          pv8[s2] = exp2_hw(__builtin_fmaf(S[t][8 * hh + s2], scale_log2, -m_use));
          ps[s2 & 3] += pv8[s2];
        }
        pop[2 * t + hh] = make_uint4(pack2<F16>(pv8[0], pv8[1]), pack2<F16>(pv8[2], pv8[3]),
                                     pack2<F16>(pv8[4], pv8[5]), pack2<F16>(pv8[6], pv8[7]));
      }
    const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    const float alpha = exp2_hw(fmaxf(m_run - m_new, -1e30f));
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // O^T must be in the new scale before P(j) is added ([FA4-edges] §The
    // value MMA waits on three gates).
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] *= alpha;
    }
  };

  // Both products of a phase as one stream of 2 * NPV MFMAs: first P*V(j-1)
  // (16-key step outer, so each P operand dies after its last use), then
  // S(j). Every MFMA's LDS operand (a transposed V pair or a K row chunk) is
  // read KDEP MFMAs ahead through a small register ring, so the S(j) reads
  // already run under the last P*V MFMAs and no read waits on LDS latency.
  constexpr int NPV = MT * NKS;  // P*V MFMAs per block (= QK MFMAs, NT * KST)
  constexpr int KDEP = 3;
  static_assert(NPV == NT * KST, "both products have the same MFMA count");
  // At d = 128 the two products alternate MFMA by MFMA (stream slot 2i is
  // P*V product i, 2i + 1 is score product i), so the transposing V reads and
  // the plain K reads share the LDS over the whole phase (1% faster); at d = 64
  // and 256 that keeps both products' registers live at once and spills.
  constexpr bool PV_QK_INTERLEAVE = D == 128;
  auto pv_qk = [&](int vslot, int kslot, int j) {
    auto rd = [&](int g) {
      const bool is_pv = PV_QK_INTERLEAVE ? (g % 2 == 0) : (g < NPV);
      const int i = PV_QK_INTERLEAVE ? g / 2 : (g < NPV ? g : g - NPV);
      if (is_pv) return vread(vslot, i / MT, i % MT);
      return kread(kslot, i % NT, i / NT);
    };
    uint4 ring[KDEP];
#pragma unroll
    for (int g = 0; g < KDEP; ++g) ring[g] = rd(g);
    static_for<0, 2 * NPV>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      const uint4 a = ring[g % KDEP];
      if constexpr (g + KDEP < 2 * NPV) ring[g % KDEP] = rd(g + KDEP);
      // This group's share of the staging (see stage below), unconditional in
      // the steady range: a block past the work-group's last is loaded (rows
      // past Sk as zeros) into a slot nobody reads again.
      if constexpr (kDma) {
        if constexpr (g == 2) dma_blk(j + 2 - G);
      } else {
        if constexpr (g == 2) store_blk(j + 1 - G);
        if constexpr (g == 6) load_blk(j + 2 - G);
      }
      constexpr bool is_pv = PV_QK_INTERLEAVE ? (g % 2 == 0) : (g < NPV);
      constexpr int i = PV_QK_INTERLEAVE ? g / 2 : (g < NPV ? g : g - NPV);
      if constexpr (is_pv) {
        constexpr int ks = i / MT, mt = i % MT;
        oacc[mt] = mma32<F16>(a, pop[ks], oacc[mt]);
      } else {
        constexpr int t = i % NT, kk = i / NT;
        if constexpr (kk == 0) S[t] = mma32<F16>(a, qop[kk], f32x16{});
        else S[t] = mma32<F16>(a, qop[kk], S[t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Staging, done in the MFMA phase, whose wave mostly waits on the matrix
  // unit: in its phase j group A writes K(j+1) (into the slot K(j-1) held,
  // last read in the previous half-step) and loads K(j+2); group B, half a
  // step later, writes V(j) (into V(j-2)'s slot) and loads V(j+1). Each tile
  // is visible one barrier before its first reader.
  // With direct loads (three slots), group A loads K(j+2) in step j into the
  // slot K(j-1) held and group B loads V(j+1) into the slot of V(j-2), both
  // last read before the barrier that ended step j-1; each block is complete
  // and published one barrier before its first reader. A block past the last
  // loads zeros into a slot nobody reads again.
  auto stage = [&](int j) {
    if constexpr (kDma) {
      if (G == 0 && j == 0) dma_blk(1);
      dma_blk(j + 2 - G);
    } else {
      if (j + 1 - G < nblk) store_blk(j + 1 - G);
      if (j + 2 - G < nblk) load_blk(j + 2 - G);
    }
  };
  auto mfma_phase = [&](int j) {
    __builtin_amdgcn_s_setprio(2);
    stage(j);
    if (j >= 1 && j - 1 < nbw) pv(slot_of(j - 1));
    if (j < nbw) qk(slot_of(j));
    __builtin_amdgcn_s_setprio(0);
  };
  auto valu_phase = [&](int j) {
    if (j >= 0 && j < nbw) {
      if (j * BN + BN > wave_lo) softmax(j * BN, std::true_type{});
      else softmax(j * BN, std::false_type{});
    }
  };

  // Direct loads (d >= 128): one barrier per step. Step j is, for group A,
  // MFMA(j) then softmax(j); for group B, softmax(j - 1) then MFMA(j): within
  // a step each SIMD's two waves still alternate the matrix unit and the
  // vector ALU, and the only point where the groups meet is the step's end.
  // The staging needs nothing more: in step j both groups read K(j) and
  // V(j - 1); group A loads K(j + 2) into K(j - 1)'s slot and group B V(j + 1)
  // into V(j - 2)'s, both last read in step j - 1; each wave's wait before the
  // barrier leaves only the loads it issued in this step in flight, so a block
  // loaded in step j is complete and published by the end of step j + 1.
  if constexpr (kDma) {
    dma_blk(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    // The two groups run separate copies of the loop (the order of softmax
    // and MFMA work differs), so each copy's register assignment only holds
    // what its own order keeps live across the barrier.
    auto run = [&](auto grp) {
      constexpr int GG = decltype(grp)::value;
      auto step = [&](int j, auto steady) {
        if constexpr (GG == 1) valu_phase(j - 1);
        if constexpr (decltype(steady)::value) {
          __builtin_amdgcn_s_setprio(2);
          pv_qk(slot_of(j - 1), slot_of(j), j);
          __builtin_amdgcn_s_setprio(0);
        } else {
          mfma_phase(j);
        }
        if constexpr (GG == 0) valu_phase(j);
        dma_wait_one();
        __syncthreads();
      };
      int j = 0;
      for (; j <= nblk && (j == 0 || j >= nbw); ++j) {  // j = 0, or a wave with nbw <= 1
        step(j, std::false_type{});
        if (j == 0 && nbw > 1) {
          ++j;
          break;
        }
      }
      for (; j < nbw; ++j) step(j, std::true_type{});
      for (; j <= nblk; ++j) step(j, std::false_type{});
    };
    if (G == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
    // Direct loads still in flight (zeros past the last block) land before
    // the slots are reused.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    // Register staging (d = 64): two barriers per step, one per phase, group B
    // one phase behind group A. Prologue: K(0) into slot 0; group A holds
    // K(1), group B V(0) in registers.
    if (nblk > 0) {
      if (G == 0) {
        load_blk(0);
        store_blk(0);
      }
      if (G == 0 && nblk > 1) load_blk(1);
      if (G == 1) load_blk(0);
    }
    __syncthreads();
    // Group B starts one phase later; both groups pass the same number of
    // barriers.
    if (G == 1) __syncthreads();
    // Steps j = 0 .. nblk. The steady range 1 <= j < nbw, where the MFMA phase
    // has both products, is a loop of its own, so its register assignment is
    // not merged with the edge steps'.
    int j = 0;
    for (; j <= nblk && (j == 0 || j >= nbw); ++j) {  // j = 0, or a wave with nbw <= 1
      mfma_phase(j);
      __syncthreads();
      valu_phase(j);
      __syncthreads();
      if (j == 0 && nbw > 1) {
        ++j;
        break;
      }
    }
    for (; j < nbw; ++j) {
      __builtin_amdgcn_s_setprio(2);
      pv_qk(slot_of(j - 1), slot_of(j), j);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      valu_phase(j);
      __syncthreads();
    }
    for (; j <= nblk; ++j) {
      mfma_phase(j);
      __syncthreads();
      valu_phase(j);
      __syncthreads();
    }
    if (G == 0) __syncthreads();
  }

  const float l_col = wave_xor_sum(l_run, 32);
  if (qrow < 0 || qrow >= Sq) return;
  const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
  uint16_t *dst = o + ((size_t)(qbase + qrow) * Hq + h) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int dd = 32 * mt + 8 * a + 4 * hl;
      *reinterpret_cast<uint2 *>(dst + dd) =
          make_uint2(pack2<F16>(oacc[mt][4 * a] * inv, oacc[mt][4 * a + 1] * inv),
                     pack2<F16>(oacc[mt][4 * a + 2] * inv, oacc[mt][4 * a + 3] * inv));
    }
  if (lse != nullptr && hl == 0)
    lse[lse_base + (size_t)h * lse_hs + qrow] = l_col > 0.f ? kLn2 * (m_run + __log2f(l_col)) : kNegInf;
}


template <int D> constexpr int kTileLds =
    D >= 128 ? 3 * 2 * kBlockKeys<D> * D : 2 * 64 * (KRow<D>::v + VRow<D>::v);  // elements
// Waves per SIMD: two (one work-group per CU) at d = 128, four at d = 64,
// where the kernel fits in 128 registers and two work-groups share a CU.
template <int D> constexpr int kPrefillWaves = D == 64 ? 4 : 2;

// One work-group per query tile, dispatched heaviest first.
template <int D, bool F16>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(kPrefillWaves<D>, kPrefillWaves<D>)))
fwd_pp(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
       const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
       const int *__restrict__ cu_q, const int *__restrict__ cu_k, int total_q, int total_k,
       int Sq, int Sk, int Hq, int Hkv, int causal, float scale_log2, int n_mblocks, int BH) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kTileLds<D>];
  fwd_tile<D, F16>(q, k, v, o, lse, cu_q, cu_k, total_q, total_k, Sq, Sk, Hq, Hkv, causal, scale_log2, n_mblocks, BH,
                   blockIdx.x, smem);
}

// Persistent form ([FA4-edges] §Edge 3, tile scheduling): one resident
// work-group per CU walks the heaviest-first tile list in rounds of gridDim.x
// tiles, in snake order (forward in even rounds, backward in odd ones), so
// the heavy and light ends of consecutive rounds pair up on each CU. The
// assignment is static: no counter, nothing to clear between calls. The
// launcher takes it at d = 128, dense or packed (a packed batch's list holds
// only its non-empty tiles); at d = 64 two dispatched work-groups per CU are
// faster, and at d = 256 the loop state would spill.
//
// Sequences a packed persistent launch takes (their tile counts are staged in
// LDS); larger packed batches use one work-group per tile.
constexpr int kPersistMaxSeq = 4096;

template <int D, bool F16>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_persist(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
            const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
            const int *__restrict__ cu_q, const int *__restrict__ cu_k, int total_q, int total_k,
            int Sq, int Sk, int Hq, int Hkv, int causal, float scale_log2, int n_mblocks, int BH) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kTileLds<D>];
  __shared__ int ntl[kPersistMaxSeq];  // packed: query tiles of each sequence
  const int G = gridDim.x, g = blockIdx.x;
  // The next tile's prologue rewrites the LDS slots: every wave must be past
  // its last LDS read and its direct loads must have landed (each wave waited
  // for its own before leaving the tile). The tile's O and LSE stores need
  // not complete first (the next tile reads other memory), so this is a bare
  // barrier, not a release fence that would wait for them.
  auto between_tiles = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  if (cu_q == nullptr) {
    const long long ntiles = (long long)n_mblocks * BH;
    bool odd = false;
    for (long long base = 0; base < ntiles; base += G, odd = !odd) {
      const long long x = base + (odd ? G - 1 - g : g);
      if (x < ntiles)
        fwd_tile<D, F16>(q, k, v, o, lse, cu_q, cu_k, total_q, total_k, Sq, Sk, Hq, Hkv, causal, scale_log2,
                         n_mblocks, BH, (int)x, smem);
      between_tiles();
    }
    return;
  }
  // Packed batch: the non-empty tiles as one list, heaviest first (tile m
  // from a sequence's start carries about m + 1 key blocks under a causal
  // mask): level w = n_mblocks .. 1 holds tile ntl[b] - w (counted from the
  // end) of every sequence b with at least w tiles, in sequence then head
  // order. Work-groups take list positions in snake order as above, and each
  // follows the list with a cursor (level w, sequence cb, head ch) that every
  // wave advances identically from the tile counts, so the assignment is
  // static and the same in every wave: no counter, no sort.
  const int B = BH / Hq, lane = threadIdx.x & 63;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int a0 = min(max(cu_q[b], 0), total_q), a1 = min(max(cu_q[b + 1], a0), total_q);
    ntl[b] = min((a1 - a0 + kBMP - 1) / kBMP, n_mblocks);
  }
  __syncthreads();
  long long ntiles = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    int t = b0 + lane < B ? ntl[b0 + lane] : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) t += __shfl_xor(t, m, 64);
    ntiles += t;
  }
  ntiles *= Hq;
  int w = n_mblocks, cb = 0, ch = 0;
  auto next_valid = [&](int start) {
    for (int b0 = start; b0 < B; b0 += 64) {
      const unsigned long long m = __ballot(b0 + lane < B && ntl[b0 + lane] >= w);
      if (m) return b0 + __ffsll((long long)m) - 1;
    }
    return B;
  };
  auto settle = [&]() {  // the first sequence at or after cb with a tile at level w, else the next level
    while (w > 0) {
      cb = next_valid(cb);
      if (cb < B) return;
      --w;
      cb = 0;
    }
  };
  settle();
  long long cur = 0;
  bool odd = false;
  for (long long base = 0; base < ntiles; base += G, odd = !odd) {
    const long long x = base + (odd ? G - 1 - g : g);
    if (x < ntiles) {
      for (long long kk = x - cur; kk > 0;) {  // move the cursor forward to list position x
        const int left = Hq - ch;
        if (kk < left) {
          ch += (int)kk;
          break;
        }
        kk -= left;
        ch = 0;
        ++cb;
        settle();
      }
      cur = x;
      // The same in every lane (from LDS and wave-wide votes): held in a scalar register.
      const int xt = __builtin_amdgcn_readfirstlane((ntl[cb] - w) * BH + cb * Hq + ch);
      fwd_tile<D, F16>(q, k, v, o, lse, cu_q, cu_k, total_q, total_k, Sq, Sk, Hq, Hkv, causal, scale_log2,
                       n_mblocks, BH, xt, smem);
    }
    between_tiles();
  }
}

}  // namespace

int current_cus();  // compute units of the current device (cached; api.hip)

// Dense when cu_q == nullptr (Sq, Sk the per-sequence lengths); packed
// variable-length otherwise (Sq = the longest query length, which sizes the
// grid; Sk unused; total_q, total_k the packed row counts).
hipError_t launch_fwd(const void *q, const void *k, const void *v, void *o, float *lse, const int *cu_q,
                      const int *cu_k, int total_q, int total_k, int causal, int batch, int Sq, int Sk, int Hq,
                      int Hkv, int d, float scale_log2, bool f16, hipStream_t stream) {
  const int BH = batch * Hq;
  const int n_mblocks = (Sq + kBMP - 1) / kBMP;
  const int ntiles = n_mblocks * BH;
  const dim3 block(512);
  const auto *qq = static_cast<const uint16_t *>(q);
  const auto *kk = static_cast<const uint16_t *>(k);
  const auto *vv = static_cast<const uint16_t *>(v);
  auto *oo = static_cast<uint16_t *>(o);
  auto run = [&](auto kern, int nwg) {
    hipLaunchKernelGGL(kern, dim3(nwg), block, 0, stream, qq, kk, vv, oo, lse, cu_q, cu_k, total_q, total_k, Sq, Sk,
                       Hq, Hkv, causal, scale_log2, n_mblocks, BH);
  };
  if (d == 128 && cu_q == nullptr) {
    const int ncu = current_cus();
    const int nwg = ntiles < ncu ? ntiles : ncu;
    if (f16) run(fwd_persist<128, true>, nwg);
    else run(fwd_persist<128, false>, nwg);
  } else if (d == 128 && batch <= kPersistMaxSeq) {
    const int ncu = current_cus();
    if (f16) run(fwd_persist<128, true>, ncu);
    else run(fwd_persist<128, false>, ncu);
  } else if (d == 256) {  // the persistent form's loop state would spill at d = 256
    if (f16) run(fwd_pp<256, true>, ntiles);
    else run(fwd_pp<256, false>, ntiles);
  } else if (d == 128) {
    if (f16) run(fwd_pp<128, true>, ntiles);
    else run(fwd_pp<128, false>, ntiles);
  } else {
    if (f16) run(fwd_pp<64, true>, ntiles);
    else run(fwd_pp<64, false>, ntiles);
  }
  return hipGetLastError();
}

}  // namespace attn

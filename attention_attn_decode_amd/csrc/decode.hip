// GQA KV-cache decode for gfx950: balanced split-KV kernel and log-sum-exp combine.
//
// Pages cited by title and section:
//   [FA4-decode] "Optimization diaries: S/P ping-pong for FlashAttention-4 decode"
//   [GQA-SM100]  "Building a Faster GQA Decode Kernel for Blackwell SM100"
//   [FA4-edges]  "Flash Attention 4 — warp-role choreography and the edges"
//
// Operand swap ([GQA-SM100] §Starting with the simple pipeline and the
// introduction): S^T = K Q^T / sqrt(d) and O^T = V^T P^T, so key positions run
// along the MFMA's M dimension and the small packed query group (the G = Hq/Hkv
// heads of one KV head times the seqlen_q new tokens, at most 32) along N, in
// one or two groups of 16 columns that share every K and V operand read. With
// v_mfma_f32_16x16x32_bf16 a lane then owns one query column: the column max and
// sum over keys are mostly in-lane, the rescale factor of O^T is one scalar per
// lane, and P leaves the S^T accumulator already in the layout the P*V MFMA
// wants as its B operand (it never goes through memory).
//
// Splitting ([GQA-SM100] §Combining the KV splits: splits give a small batch
// enough parallel work; each returns an unnormalised output, its maximum and
// its denominator). Here the split is balanced on the device, in units of the
// 32-key sub-blocks a wave processes at a time: sequence b has
// n_b = ceil(L_b / 32) sub-blocks, the sub-blocks of all sequences are laid end
// to end (sequence b occupies flattened units [start_b, start_b + n_b)), and
// that range is cut into P_eff equal pieces. Each wave is an independent worker
// owning one (piece, KV head) pair, so every wave runs the same number of
// sub-blocks (to within one) however ragged the lengths, and there are no empty
// work-groups. A piece may cross sequence boundaries; the wave then emits one
// partial per sequence segment it covered. The partial of piece w for sequence
// b goes to slot w + b of its KV head: pieces are contiguous and ordered, so
// (w, b) -> w + b is one-to-one, and P + B slots per head always suffice.
//
// Streaming: one work-group of four independent waves per CU. Each wave keeps
// two sub-blocks of 32 keys in flight in a two-slot register ring (nontemporal
// 16-byte loads; K and V are read exactly once) and, per sub-block, passes K and V
// through a private LDS tile that changes their layout to the MFMA operand
// layouts: K and V row-major with XOR-swizzled 16-byte chunks; the P*V A
// operand, which needs keys along its k dimension, comes from two transposing
// ds_read_b64_tr_b16 reads of V. There is no work-group barrier.
//
// Key order inside a sub-block: MFMA row i of score tile t (0/1) holds key
// 8 * (i / 4) + 4 * t + (i % 4). Lane group g (= lane / 16) then receives the
// scores of keys 8g .. 8g + 7 in its two accumulators, exactly the eight
// contiguous keys its P*V B-operand slots need.
#include "attn_device.h"

namespace attn {
namespace {

constexpr int kWaves = 4;  // waves (independent workers) per work-group
constexpr int kSub = 32;   // keys per sub-block
constexpr int kCols = 16;  // packed query columns per column group
constexpr int kMaxBatch = 8192;  // sequences per call (lengths staged in LDS)
// Pieces per sequence (P / B) above which the combine splits each sequence's
// merge over its output slices instead of one work-group per sequence.
constexpr int kSliceCombine = 16;
// Tolerated growth of a column's running max before O is rescaled (base 2).
constexpr float kRescaleLog2 = 8.f;

// XOR swizzle of the 16-byte chunk index of K row r in the LDS tile [32][D]:
// the 16 rows one QK A-operand read touches land on 16 distinct bank groups.
// At D = 256 the swizzle acts on the low four bits of the chunk index, which
// select the bank group of a 512-byte row as of a 256-byte one.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D >= 128) {
    return (r & 15) ^ ((r >> 4) << 2);
  } else {
    const int x = r >> 1;
    return (x & 1) | (((x >> 3) & 1) << 1) | (((x >> 2) & 1) << 2);
  }
}

// XOR swizzle of the 16-byte chunk index of V row r in the LDS tile [32][D].
// The P*V operand is read transposed: the 32 lanes serviced together read
// rows {4u..4u+3} and {8+4u..8+4u+3} (or the same plus 16) at two adjacent
// chunks; this swizzle puts those 16 pieces on distinct bank groups.
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  if constexpr (D >= 128) return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
  else return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
}

__device__ __forceinline__ int clamp_len(int L, int max_len) {
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

__device__ __forceinline__ uint4 ld_stream(const uint16_t *p) {
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// Sub-blocks of a sequence of L keys.
__device__ __forceinline__ int units_of(int L) { return (L + kSub - 1) / kSub; }

// Sum over all sequences of their sub-block counts (every lane gets it).
__device__ long long total_units(const int *lens, int B) {
  const int lane = threadIdx.x & 63;
  long long t = 0;
  for (int b = lane; b < B; b += 64) t += units_of(lens[b]);
  for (int m = 1; m < 64; m <<= 1) t += __shfl_xor(t, m, 64);
  return t;
}

// Number of pieces per KV head: the requested P, but no piece shorter than
// min_units sub-blocks (so tiny inputs do not fan out into empty work).
__device__ __forceinline__ int pieces_for(long long T, int P, int min_units) {
  const long long by_len = T < (1LL << 31) ? (long long)(((unsigned)T + min_units - 1) / (unsigned)min_units)
                                           : (T + min_units - 1) / min_units;
  return (int)(by_len < P ? (by_len < 1 ? 1 : by_len) : P);
}

// Piece w of P_eff covers flattened units [w*T/P_eff, (w+1)*T/P_eff); the
// piece holding flattened unit x is ((x + 1) * P_eff - 1) / T.
__device__ __forceinline__ long long piece_begin(int w, long long T, int P_eff) {
  return (long long)w * T / P_eff;
}
__device__ __forceinline__ int piece_of(long long x, long long T, int P_eff) {
  return (int)(((x + 1) * P_eff - 1) / T);
}

struct Seg {
  int b;            // sequence
  int lo, hi;       // local key range [lo, hi) of this segment (lo % 32 == 0)
  int L;            // clamped sequence length
  long long start;  // flattened unit where the sequence starts
};

// Key end of a segment of sequence (start, L) cut at flattened unit r1.
__device__ __forceinline__ int seg_hi(long long start, int L, long long r1) {
  const long long e = (r1 - start) * kSub;
  return (int)(e < L ? e : L);
}

// The sequence containing flattened unit x (x < total): wave-wide scan over
// the sub-block counts, 64 sequences at a time.
__device__ Seg find_segment(const int *lens, int B, long long x, long long r1) {
  const int lane = threadIdx.x & 63;
  long long carry = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const int L = b < B ? lens[b] : 0;
    const int n = units_of(L);
    long long incl = n;
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const long long st = carry + incl - n;
    const unsigned long long hit = __ballot(n > 0 && st <= x && x < st + n);
    if (hit) {
      const int h = __ffsll((long long)hit) - 1;
      Seg s;
      s.b = base + h;
      s.start = __shfl(st, h, 64);
      s.L = __shfl(L, h, 64);
      s.lo = (int)(x - s.start) * kSub;
      s.hi = seg_hi(s.start, s.L, r1);
      return s;
    }
    carry += __shfl(incl, 63, 64);
  }
  Seg none = {B, 0, 0, 0, carry};
  return none;
}

// total_units and find_segment for calls whose sub-block counts and their
// sums over 64 sequences fit in 32 bits (max_len <= 2^25): wave scans through
// DPP and lane reads instead of LDS shuffles, the running 64-bit carry in
// scalar registers.
__device__ long long total_units32(const int *lens, int B) {
  const int lane = threadIdx.x & 63;
  long long t = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const unsigned n = b < B ? (unsigned)units_of(lens[b]) : 0u;
    t += __builtin_amdgcn_readlane(wave_incl_scan_u32(n), 63);
  }
  return t;
}

__device__ Seg find_segment32(const int *lens, int B, long long x, long long r1) {
  const int lane = threadIdx.x & 63;
  long long carry = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const int L = b < B ? lens[b] : 0;
    const unsigned n = (unsigned)units_of(L);
    const unsigned incl = wave_incl_scan_u32(n);
    const long long st = carry + (long long)(incl - n);
    const unsigned long long hit = __ballot(n > 0 && st <= x && x < st + (long long)n);
    if (hit) {
      const int h = __ffsll((long long)hit) - 1;
      Seg s;
      s.b = base + h;
      s.start = carry + (long long)__builtin_amdgcn_readlane(incl - n, h);
      s.L = __builtin_amdgcn_readlane(L, h);
      s.lo = (int)(x - s.start) * kSub;
      s.hi = seg_hi(s.start, s.L, r1);
      return s;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  Seg none = {B, 0, 0, 0, carry};
  return none;
}

// Piece bounds w * T / P_eff and (w + 1) * T / P_eff, in 32-bit arithmetic
// when the products fit.
__device__ __forceinline__ void piece_bounds(int w, long long T, int P_eff, long long &r0, long long &r1) {
  if (T * (long long)P_eff < (1LL << 32)) {
    const unsigned t = (unsigned)T, p = (unsigned)P_eff;
    r0 = (unsigned)w * t / p;
    r1 = (unsigned)(w + 1) * t / p;
  } else {
    r0 = piece_begin(w, T, P_eff);
    r1 = piece_begin(w + 1, T, P_eff);
  }
}

// Next non-empty sequence segment before flattened unit r1.
__device__ bool next_segment(Seg &s, const int *lens, int B, long long r1) {
  long long st = s.start + units_of(s.L);
  for (int b = s.b + 1; b < B && st < r1; ++b) {
    const int L = lens[b];
    if (L > 0) {
      s.b = b;
      s.start = st;
      s.L = L;
      s.lo = 0;
      s.hi = seg_hi(st, L, r1);
      return true;
    }
  }
  return false;
}

template <int D, int NC>
struct Slot {
  static constexpr int CH = D / 8;
  static constexpr int RPI = 64 / CH;    // rows one wave-wide 16-byte load covers
  static constexpr int NK = kSub / RPI;  // K loads per lane
  static constexpr int NVG = CH / 8;     // 4-row V groups per lane
  static constexpr int KST = D / 32;     // QK k-steps
  uint4 k[NK];
  uint4 v[NVG][4];
  uint4 q[NC][KST];
};

// NC column groups of 16 packed query columns (1 or 2); the partial
// workspace holds 16 * NC columns per slot. GRP selects the work split:
//   false - balanced pieces: each wave owns one (piece, KV head) of the
//           flattened sub-blocks of all sequences; sequences spread over
//           several pieces leave fp32 partials for the combine kernel.
//   true  - one work-group per (sequence, KV head): its four waves take equal
//           shares of the sequence's sub-blocks and merge their partials
//           through LDS, so the call is one kernel with no workspace and no
//           plan (used when there are enough sequence-head pairs to fill the
//           chip).
template <int D, bool F16, int NC, bool GRP>
__global__ void __launch_bounds__(256, 1)
decode_stream(const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
              const uint16_t *__restrict__ vc, const int *__restrict__ seqlens,
              uint16_t *__restrict__ o, float *__restrict__ lse, float *__restrict__ ws_o,
              float2 *__restrict__ ws_ml, long long *__restrict__ meta, int B, int Hq, int Hkv,
              int sq, int max_len, int P, int min_units, float scale_log2) {
  using S = Slot<D, NC>;
  constexpr int COLS = kCols * NC;
  constexpr int CH = S::CH, RPI = S::RPI, NK = S::NK, NVG = S::NVG, KST = S::KST;
  constexpr int MT = D / 16;
  constexpr int TILE = kSub * D;
  // At D = 256 K and V pass through one tile per wave in turn (V is written
  // once the score MFMAs have read K), which keeps the work-group's LDS at
  // 96 KB; below, each has its own tile.
  constexpr bool kOneTile = D == 256;
  constexpr int NTILE = kOneTile ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kWaves * NTILE * TILE];
  // Clamped sequence lengths, staged once: segment walks then wait on LDS,
  // never on the vector-memory counter that the K/V stream keeps busy.
  __shared__ int lens[GRP ? 1 : kMaxBatch];
  // Grouped work-groups: each wave's (max, denominator) per packed column;
  // the unnormalised outputs go to smem once the stream is done.
  __shared__ float2 s_ml[GRP ? kWaves * COLS : 1];
  static_assert(kWaves * COLS * D * sizeof(float) <= sizeof(smem), "merge area exceeds the K/V tiles");

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int g, wp;
  long long T = 0, r0 = 0, r1 = 0;
  int P_eff = 1;
  Seg first = {0, 0, 0, 0, 0};
  int n_sub = 0;
  if constexpr (GRP) {
    g = blockIdx.x % Hkv;
    wp = 0;
    const int b = blockIdx.x / Hkv;
    const int L = clamp_len(seqlens[b], max_len);
    const int nu = units_of(L);
    const int u0 = wv * nu / kWaves, u1 = (wv + 1) * nu / kWaves;
    first = Seg{b, u0 * kSub, min(u1 * kSub, L), L, 0};
    n_sub = u1 - u0;  // may be 0 for sequences shorter than four sub-blocks
  } else {
    for (int b = threadIdx.x; b < B; b += blockDim.x) lens[b] = clamp_len(seqlens[b], max_len);
    __syncthreads();
    const int item = blockIdx.x * kWaves + wv;  // = piece * Hkv + kv head
    g = item % Hkv;
    wp = item / Hkv;
    // Sub-block counts and their 64-sequence sums fit in 32 bits below 2^25 keys.
    const bool plan32 = max_len <= (1 << 25);
    T = plan32 ? total_units32(lens, B) : total_units(lens, B);
    // The combine step reads the total and every sequence's flattened start
    // from here instead of re-scanning the lengths.
    if (meta != nullptr && item == 0 && lane == 0) meta[0] = T;
    if (T == 0) return;
    P_eff = pieces_for(T, P, min_units);
    if (wp >= P_eff) return;
    piece_bounds(wp, T, P_eff, r0, r1);
    first = plan32 ? find_segment32(lens, B, r0, r1) : find_segment(lens, B, r0, r1);
    if (first.b >= B) return;
    n_sub = (int)(r1 - r0);  // sub-blocks of this piece
  }

  const int G = Hq / Hkv, ncol = G * sq;
  const int n = lane & 15, gq = lane >> 4;
  // Packed column nc[c] = 16 c + n of column group c: new token tn[c], query
  // head head[c] (pad columns read column 0 and are never written out).
  bool col_ok[NC];
  int nc[NC], tn[NC], head[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    nc[c] = kCols * c + n;
    col_ok[c] = nc[c] < ncol;
    tn[c] = col_ok[c] ? nc[c] / G : 0;
    head[c] = g * G + (col_ok[c] ? nc[c] % G : 0);
  }
  const size_t rstride = (size_t)Hkv * D;
  const int slots = P + B;  // partial slots per KV head
  uint16_t *klds = smem + wv * NTILE * TILE;
  uint16_t *vlds = kOneTile ? klds : klds + TILE;

  // Load one sub-block (sequence b, keys [j0, j0 + 32), valid below hi) into
  // ring registers. Rows at or past hi are clamped to hi - 1: every load is
  // issued unconditionally (a fixed count per sub-block keeps the wait counters
  // exact) and reads finite data of this sequence, which the mask then excludes.
  auto load_k = [&](auto &sl, int b, int j0, int hi) __attribute__((always_inline)) {
    const uint16_t *kb = kc + ((size_t)b * max_len * Hkv + g) * D;
#pragma unroll
    for (int qi = 0; qi < NK; ++qi) {
      const int p = min(j0 + RPI * qi + lane / CH, hi - 1);
      sl.k[qi] = ld_stream(kb + (size_t)p * rstride + (lane % CH) * 8);
    }
  };
  auto load_v = [&](auto &sl, int b, int j0, int hi) __attribute__((always_inline)) {
    const uint16_t *vb = vc + ((size_t)b * max_len * Hkv + g) * D;
#pragma unroll
    for (int hg = 0; hg < NVG; ++hg) {
      const int g4 = lane / CH + (64 / CH) * hg;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int p = min(j0 + 4 * g4 + qq, hi - 1);
        sl.v[hg][qq] = ld_stream(vb + (size_t)p * rstride + (lane % CH) * 8);
      }
    }
  };
  // Q^T B operand of sequence b: slot k of lane group gq at k-step kk covers
  // chunk 4 * kk + gq of the query row.
  auto load_q = [&](auto &sl, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint16_t *qrow = q + ((size_t)(b * sq + tn[c]) * Hq + head[c]) * D;
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) sl.q[c][kk] = ldg16(qrow + (4 * kk + gq) * 8);
    }
  };

  float m_run[NC], l_run[NC];
  f32x4 oacc[NC][MT];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    m_run[c] = kNegInf, l_run[c] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K registers -> LDS tile (row-major, swizzled chunks).
  auto store_k = [&](const auto &sl) __attribute__((always_inline)) {
#pragma unroll
    for (int qi = 0; qi < NK; ++qi) {
      const int r = RPI * qi + lane / CH, c = lane % CH;
      sts16(klds + r * D + ((c ^ k_swz<D>(r)) * 8), sl.k[qi]);
    }
  };
  // V registers -> LDS tile (row-major, swizzled chunks).
  auto store_v = [&](const auto &sl) __attribute__((always_inline)) {
#pragma unroll
    for (int hg = 0; hg < NVG; ++hg) {
      const int g4 = lane / CH + (64 / CH) * hg, c = lane % CH;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int r = 4 * g4 + qq;
        sts16(vlds + r * D + ((c ^ v_swz<D>(r)) * 8), sl.v[hg][qq]);
      }
    }
  };
  // S^T = K Q^T of the sub-block whose K is in the LDS tile, with the Q
  // operand in qs (MFMA row i of tile t is key 8 (i / 4) + 4 t + i % 4).
  using Scores = f32x4[NC][2];
  auto scores = [&](const auto &qs, Scores &sacc) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int i = lane & 15;
      const int r = 8 * (i >> 2) + 4 * t + (i & 3);
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) {
        const int ck = 4 * kk + gq;
        const uint4 ka = lds16(klds + r * D + ((ck ^ k_swz<D>(r)) * 8));
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc[c][t] = mma16<F16>(ka, qs.q[c][kk], sacc[c][t]);
      }
    }
  };
  // Online softmax of one sub-block's scores: masks, running max and sum,
  // rescale of O; returns P (element type, the P*V B operand) per group.
  auto softmax = [&](const Scores &sacc, const Seg &cs, int j0, bool live, uint4 (&pop)[NC])
                     __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // Keys visible to this column: below the segment end and, among the sq
      // new tokens, the bottom-right causal limit j <= L - sq + t
      // ([FA4-edges] §Edge 1: masked to -inf before the max).
      const int bound = live ? min(cs.hi, cs.L - sq + tn[c] + 1) : 0;
      float sv[8];
      float mloc = kNegInf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = j0 + 8 * gq + 4 * t + r;
          const float xs = pos < bound ? sacc[c][t][r] * scale_log2 : kNegInf;
          sv[4 * t + r] = xs;
          mloc = fmaxf(mloc, xs);
        }
      mloc = wave_xor_max(mloc, 16);
      mloc = wave_xor_max(mloc, 32);
      // Online softmax in base 2 with the conditional rescale ([FA4-edges]
      // §The correction): the reference max moves only when the sub-block's
      // max exceeds it by more than kRescaleLog2, so P stays below 2^8 and O
      // is rescaled only for the few sub-blocks that raise the max that much.
      const float m_new = mloc > m_run[c] + kRescaleLog2 ? mloc : m_run[c];
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_hw(fmaxf(m_run[c] - m_new, -1e30f));
      float p[8], ps[2] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = exp2_hw(sv[i] - m_use);
        ps[i & 1] += p[i];
      }
      l_run[c] = l_run[c] * alpha + (ps[0] + ps[1]);
      m_run[c] = m_new;
      // Rescale O before accumulating into it ([FA4-edges] §The value MMA waits
      // on three gates); skipped by the whole wave when no column needs it.
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) oacc[c][mt] *= alpha;
      }
      pop[c] = make_uint4(pack2<F16>(p[0], p[1]), pack2<F16>(p[2], p[3]), pack2<F16>(p[4], p[5]),
                          pack2<F16>(p[6], p[7]));
    }
  };
  // O^T += V^T P^T with V in the LDS tile. A operand: the same eight keys
  // 8gq .. 8gq + 7 at column 16mt + (lane % 16), as two transposed 4-key reads.
  auto pv = [&](const uint4 (&pop)[NC]) __attribute__((always_inline)) {
    const int trk = lane & 15;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint2 tr[2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int r = 8 * gq + 4 * uu + (trk >> 2);
        const int c = 2 * mt + ((trk & 3) >> 1);
        tr[uu] = lds_tr4(vlds + r * D + ((c ^ v_swz<D>(r)) * 8) + 4 * (trk & 1));
      }
      const uint4 va = make_uint4(tr[0].x, tr[0].y, tr[1].x, tr[1].y);
#pragma unroll
      for (int c = 0; c < NC; ++c) oacc[c][mt] = mma16<F16>(va, pop[c], oacc[c][mt]);
    }
  };

  // End of a sequence segment. If the segment is the whole sequence, no other
  // piece touches it: write the final O and LSE. Otherwise write this wave's
  // partial for sequence b to slot wp + b of KV head g. Then reset the state.
  auto finalize = [&](const Seg &sg) __attribute__((always_inline)) {
    const int b = sg.b;
    if (meta != nullptr && sg.lo == 0 && g == 0 && lane == 0) meta[1 + b] = sg.start;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float l_col = wave_xor_sum(l_run[c], 16);
      l_col = wave_xor_sum(l_col, 32);
      if (sg.lo == 0 && sg.hi == sg.L) {
        if (col_ok[c]) {
          const float inv = l_col > 0.f ? 1.f / l_col : 0.f;
          uint16_t *dst = o + ((size_t)(b * sq + tn[c]) * Hq + head[c]) * D;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            *reinterpret_cast<uint2 *>(dst + 16 * mt + 4 * gq) =
                make_uint2(pack2<F16>(oacc[c][mt][0] * inv, oacc[c][mt][1] * inv),
                           pack2<F16>(oacc[c][mt][2] * inv, oacc[c][mt][3] * inv));
          if (lse != nullptr && gq == 0)
            lse[((size_t)b * Hq + head[c]) * sq + tn[c]] =
                l_col > 0.f ? kLn2 * (m_run[c] + __log2f(l_col)) : kNegInf;
        }
      } else if (col_ok[c]) {
        const size_t slot = (size_t)g * slots + wp + b;
        float *dst = ws_o + (slot * COLS + nc[c]) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(dst + 16 * mt + 4 * gq) = oacc[c][mt];
        if (gq == 0) ws_ml[slot * COLS + nc[c]] = make_float2(m_run[c], l_col);
      }
      m_run[c] = kNegInf;
      l_run[c] = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Sub-block iterators over this piece's segments. A load iterator past the
  // last sub-block keeps re-reading the last valid rows (its loads are never
  // used), so the loops below have no data-dependent control flow around the
  // ring registers.
  struct Iter {
    Seg s;
    int j;
  };
  auto advance_load = [&](Iter &it) __attribute__((always_inline)) {
    it.j += kSub;
    if (!GRP && it.j >= it.s.hi) {
      Seg nx = it.s;
      if (next_segment(nx, lens, B, r1)) {
        it.s = nx;
        it.j = it.s.lo;
      }
    }
  };
  Seg cs = first;
  int cj = cs.lo;
  auto advance_compute = [&]() __attribute__((always_inline)) {
    cj += kSub;
    if (!GRP && cj >= cs.hi) {
      finalize(cs);
      if (next_segment(cs, lens, B, r1)) cj = cs.lo;
    }
  };

  if (n_sub > 0) {
  if constexpr (kOneTile) {
    // D = 256, one register slot: the next sub-block's K loads are issued as
    // soon as this one's K is in LDS, its V and Q loads once this one's V is,
    // so they run under this sub-block's MFMAs (two slots would exceed the
    // register file). K and V pass through the wave's one LDS tile in turn.
    S r;
    Iter it{first, first.lo};
    load_k(r, it.s.b, it.j, it.s.hi);
    load_v(r, it.s.b, it.j, it.s.hi);
    load_q(r, it.s.b);
    advance_load(it);
    for (int i = 0; i < n_sub; ++i) {
      const int nb = it.s.b, nj = it.j, nhi = it.s.hi;
      store_k(r);
      wave_lds_sync();
      load_k(r, nb, nj, nhi);
      Scores sacc;
      scores(r, sacc);
      uint4 pop[NC];
      softmax(sacc, cs, cj, true, pop);
      wave_lds_sync();  // every K read of the score MFMAs has returned
      store_v(r);
      wave_lds_sync();
      load_v(r, nb, nj, nhi);
      pv(pop);
      load_q(r, nb);
      wave_lds_sync();
      advance_load(it);
      advance_compute();
    }
  } else if constexpr (NC == 1) {
    // One column group: two ring slots, each sub-block's K, V and Q together:
    // sub-block i + 2 is loaded into a slot as soon as sub-block i has left it;
    // its scores, softmax and P*V run in that order. (Removing all score,
    // softmax and P*V work speeds these calls by at most 3% - the stream sets
    // their time - and overlapping scores with softmax, below, made them 1-3%
    // slower.)
    S ra, rb;
    Iter it{first, first.lo};
    auto load_slot = [&](S &sl) __attribute__((always_inline)) {
      load_k(sl, it.s.b, it.j, it.s.hi);
      load_v(sl, it.s.b, it.j, it.s.hi);
      load_q(sl, it.s.b);
      advance_load(it);
    };
    auto compute = [&](S &sl, bool live) __attribute__((always_inline)) {
      store_k(sl);
      store_v(sl);
      wave_lds_sync();
      Scores sacc;
      scores(sl, sacc);
      uint4 pop[NC];
      softmax(sacc, cs, cj, live, pop);
      pv(pop);
      wave_lds_sync();
    };
    load_slot(ra);
    load_slot(rb);
    for (int i = 0; i < n_sub; i += 2) {
      compute(ra, true);
      load_slot(ra);
      advance_compute();
      const bool live_b = i + 1 < n_sub;
      compute(rb, live_b);
      load_slot(rb);
      if (live_b) advance_compute();
    }
  } else {
    // Two column groups (twice the score, softmax and P*V work per byte: with
    // that work removed these calls run 11-17% faster): scores of sub-block
    // i + 1 overlap the softmax of sub-block i ([FA4-decode] §The S/P
    // Ping-Pong, here between two score register sets of one wave): the score
    // MFMAs of i + 1 are issued before the exponentials of i, which do not
    // depend on them, so the matrix unit and the vector ALU work at once. K (with the sequence's Q operand) therefore has to reach LDS
    // one sub-block before V: K and V have their own two-slot register rings
    // and load iterators, K running one sub-block ahead, and each ring slot is
    // refilled (sub-block + 2) as soon as its registers have been used (K once
    // the score MFMAs have read its Q operand).
    struct KSlot {
      uint4 k[NK];
      uint4 q[NC][KST];
    };
    struct VSlot {
      uint4 v[NVG][4];
    };
    KSlot ka, kb;
    VSlot va, vb;
    Iter ik{first, first.lo}, iv{first, first.lo};
    auto load_ks = [&](KSlot &sl) __attribute__((always_inline)) {
      load_k(sl, ik.s.b, ik.j, ik.s.hi);
      load_q(sl, ik.s.b);
      advance_load(ik);
    };
    auto load_vs = [&](VSlot &sl) __attribute__((always_inline)) {
      load_v(sl, iv.s.b, iv.j, iv.s.hi);
      advance_load(iv);
    };
    Scores s_even, s_odd;
    // Prologue: K of sub-blocks 0 and 1, V of 0 and 1 in flight; scores of 0.
    load_ks(ka);
    load_ks(kb);
    load_vs(va);
    load_vs(vb);
    store_k(ka);
    wave_lds_sync();
    scores(ka, s_even);
    wave_lds_sync();
    load_ks(ka);  // K of sub-block 2
    // Step i: K(i + 1) (and its Q operand) is in k_next, V(i) in v_cur, the
    // scores of i in s_cur.
    auto step = [&](KSlot &k_next, VSlot &v_cur, Scores &s_cur, Scores &s_next, bool live)
                    __attribute__((always_inline)) {
      store_k(k_next);
      store_v(v_cur);
      wave_lds_sync();
      load_vs(v_cur);  // V of sub-block i + 2
      scores(k_next, s_next);
      load_ks(k_next);  // K of sub-block i + 3, once the scores have taken its Q operand
      uint4 pop[NC];
      softmax(s_cur, cs, cj, live, pop);
      pv(pop);
      wave_lds_sync();
    };
    for (int i = 0; i < n_sub; i += 2) {
      step(kb, va, s_even, s_odd, true);
      advance_compute();
      const bool live_b = i + 1 < n_sub;
      step(ka, vb, s_odd, s_even, live_b);
      if (live_b) advance_compute();
    }
  }
  }  // n_sub > 0

  if constexpr (GRP) {
    // Merge the four waves' partials of this (sequence, KV head) through LDS
    // in wave order (deterministic), then write O and LSE. A wave with no
    // sub-blocks contributes m = -inf, l = 0, O = 0; an empty sequence thus
    // gets O = 0 and LSE = -inf.
    float *s_o = reinterpret_cast<float *>(smem);  // [kWaves][COLS][D]
    __syncthreads();                               // every wave is done with its K/V tiles
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float l_col = wave_xor_sum(l_run[c], 16);
      l_col = wave_xor_sum(l_col, 32);
      float *dst = s_o + ((size_t)wv * COLS + nc[c]) * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(dst + 16 * mt + 4 * gq) = oacc[c][mt];
      if (gq == 0) s_ml[wv * COLS + nc[c]] = make_float2(m_run[c], l_col);
    }
    __syncthreads();
    constexpr int SEG = D / 16;  // outputs per thread: 16 threads per packed column
    const int b = first.b;
    for (int col = threadIdx.x >> 4; col < ncol; col += 16) {
      const int e0 = (threadIdx.x & 15) * SEG;
      float M = kNegInf, lsum = 0.f;
      float acc[SEG];
#pragma unroll
      for (int e = 0; e < SEG; ++e) acc[e] = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float2 ml = s_ml[w * COLS + col];
        if (ml.x == kNegInf) continue;
        const float Mn = fmaxf(M, ml.x);
        const float a = exp2_hw(M - Mn), cw = exp2_hw(ml.x - Mn);
        lsum = lsum * a + ml.y * cw;
        const float *src = s_o + ((size_t)w * COLS + col) * D + e0;
#pragma unroll
        for (int e = 0; e < SEG; ++e) acc[e] = acc[e] * a + src[e] * cw;
        M = Mn;
      }
      const int ct = col / G, chead = g * G + col % G;
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      uint16_t *dsto = o + ((size_t)(b * sq + ct) * Hq + chead) * D + e0;
#pragma unroll
      for (int e = 0; e < SEG; e += 2)
        *reinterpret_cast<uint32_t *>(dsto + e) = pack2<F16>(acc[e] * inv, acc[e + 1] * inv);
      if (lse != nullptr && (threadIdx.x & 15) == 0)
        lse[((size_t)b * Hq + chead) * sq + ct] = lsum > 0.f ? kLn2 * (M + __log2f(lsum)) : kNegInf;
    }
  }
}

// Split-KV combine ([GQA-SM100] §Combining the KV splits, §Removing the max
// reset): per query row, the common maximum is the max of the staged piece
// maxima, every piece is rescaled by 2^(m_s - M), and the weighted fp32 sum is
// normalised. Only the pieces that overlap the sequence are read (all written
// by this call); pieces whose column was fully masked (m_s = -inf) contribute
// nothing; an empty row gives O = 0 and LSE = -inf; O is overwritten. A
// sequence inside a single piece was finalised by the split kernel and is left
// alone. One work-group per (sequence, KV head); the 16 threads of a column
// each own D/16 outputs, and when the group has fewer than 16 columns the
// idle threads form extra groups that merge disjoint, fixed subsets of the
// pieces (w = w0 + grp, w0 + grp + NG, ...), folded together at the end in
// group order: the result does not depend on timing.
template <int D, bool F16, int NC>
__global__ void __launch_bounds__(256 * NC)
combine_pieces(const float *__restrict__ ws_o, const float2 *__restrict__ ws_ml,
               const long long *__restrict__ meta, const int *__restrict__ seqlens,
               uint16_t *__restrict__ o, float *__restrict__ lse, int B, int Hq, int Hkv, int sq,
               int max_len, int P, int min_units) {
  constexpr int SEG = D / 16;
  constexpr int COLS = kCols * NC;  // columns per partial slot
  __shared__ __attribute__((aligned(16))) float s_acc[COLS][D];
  __shared__ float s_gm[COLS], s_gl[COLS];
  const int b = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, seg = (tid & 15) * SEG, rest = tid >> 4;
  const int G = Hq / Hkv, ncol = G * sq;
  const int NG = COLS / ncol;  // piece groups (>= 1)
  const int col = rest % ncol, grp = rest / ncol;
  // The plan values are read together with the length (one memory round
  // trip, not two); for an empty sequence meta[1 + b] was never written and
  // is not used.
  const int L = clamp_len(seqlens[b], max_len);
  const long long T = P > 1 ? meta[0] : 0, st = P > 1 ? meta[1 + b] : 0;
  int w0 = 0, w1 = -1;
  if (L > 0) {
    if (P <= 1) return;  // every sequence was finished by the split kernel
    const int P_eff = pieces_for(T, P, min_units);
    w0 = piece_of(st, T, P_eff);
    w1 = piece_of(st + units_of(L) - 1, T, P_eff);
    if (w0 == w1) return;
  }
  const size_t base = (size_t)g * (P + B) + b;  // slot of piece w is base + w
  float M = kNegInf, lsum = 0.f;
  float acc[SEG];
#pragma unroll
  for (int e = 0; e < SEG; ++e) acc[e] = 0.f;
  if (grp < NG) {
#pragma unroll 4
    for (int w = w0 + grp; w <= w1; w += NG) {
      const float2 ml = ws_ml[(base + w) * COLS + col];
      const float *src = ws_o + ((base + w) * COLS + col) * D + seg;
      float x[SEG];
#pragma unroll
      for (int e = 0; e < SEG; e += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(src + e);
        x[e] = v.x;
        x[e + 1] = v.y;
        x[e + 2] = v.z;
        x[e + 3] = v.w;
      }
      // A piece whose column was fully masked (m = -inf, l = 0, O = 0)
      // leaves the running state unchanged.
      const bool live = ml.x != kNegInf;
      const float Mn = live ? fmaxf(M, ml.x) : M;
      const float a = live ? exp2_hw(M - Mn) : 1.f;
      const float c = live ? exp2_hw(ml.x - Mn) : 0.f;
      lsum = lsum * a + ml.y * c;
#pragma unroll
      for (int e = 0; e < SEG; ++e) acc[e] = acc[e] * a + x[e] * c;
      M = Mn;
    }
  }
  // Fold the piece groups into group 0, in group order.
  if (NG > 1) {
    for (int k = 1; k < NG; ++k) {
      __syncthreads();
      if (grp == k) {
        if ((tid & 15) == 0) {
          s_gm[col] = M;
          s_gl[col] = lsum;
        }
#pragma unroll
        for (int e = 0; e < SEG; ++e) s_acc[col][seg + e] = acc[e];
      }
      __syncthreads();
      if (grp == 0) {
        const float m2 = s_gm[col];
        if (m2 != kNegInf) {
          const float Mn = fmaxf(M, m2);
          const float a = exp2_hw(M - Mn), c = exp2_hw(m2 - Mn);
          lsum = lsum * a + s_gl[col] * c;
#pragma unroll
          for (int e = 0; e < SEG; ++e) acc[e] = acc[e] * a + s_acc[col][seg + e] * c;
          M = Mn;
        }
      }
    }
  }
  if (grp != 0) return;
  const int ct = col / G, chead = g * G + col % G;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t *dst = o + ((size_t)(b * sq + ct) * Hq + chead) * D + seg;
#pragma unroll
  for (int e = 0; e < SEG; e += 2)
    *reinterpret_cast<uint32_t *>(dst + e) = pack2<F16>(acc[e] * inv, acc[e + 1] * inv);
  if (lse != nullptr && (tid & 15) == 0)
    lse[((size_t)b * Hq + chead) * sq + ct] = lsum > 0.f ? kLn2 * (M + __log2f(lsum)) : kNegInf;
}


// Combine for calls whose sequences spread over many pieces (few sequences
// and KV heads, long keys: the batch-1 decode shapes). The merge of one
// (sequence, KV head) is split over its outputs: one work-group per 16-float
// slice of one packed column. Its 64 piece lanes (4 threads of one float4
// each) merge the disjoint, fixed piece subsets w0 + p, w0 + p + 64, ... with
// the rules of combine_pieces, and the 64 lane states then fold pairwise in a
// fixed tree through LDS (lane p takes lane p + h for h = 32, 16, ..., 1):
// the result does not depend on timing.
template <int D, bool F16, int NC>
__global__ void __launch_bounds__(256)
combine_slices(const float *__restrict__ ws_o, const float2 *__restrict__ ws_ml,
               const long long *__restrict__ meta, const int *__restrict__ seqlens,
               uint16_t *__restrict__ o, float *__restrict__ lse, int B, int Hq, int Hkv, int sq,
               int max_len, int P, int min_units) {
  constexpr int COLS = kCols * NC;  // columns per partial slot
  constexpr int SPC = D / 16;       // 16-float slices per column
  constexpr int NP = 64;            // piece lanes
  constexpr int NB = 4;             // pieces per lane whose loads are in flight together
  __shared__ __attribute__((aligned(16))) float4 s_acc[NP][4];
  __shared__ float s_m[NP], s_l[NP];
  const int b = blockIdx.z, g = blockIdx.y;
  const int col = blockIdx.x / SPC, sl = blockIdx.x % SPC;
  const int G = Hq / Hkv, ncol = G * sq;
  if (col >= ncol) return;
  const int tid = threadIdx.x, f = tid & 3, p = tid >> 2;
  const int L = clamp_len(seqlens[b], max_len);
  const long long T = P > 1 ? meta[0] : 0, st = P > 1 ? meta[1 + b] : 0;
  int w0 = 0, w1 = -1;
  if (L > 0) {
    if (P <= 1) return;
    const int P_eff = pieces_for(T, P, min_units);
    w0 = piece_of(st, T, P_eff);
    w1 = piece_of(st + units_of(L) - 1, T, P_eff);
    if (w0 == w1) return;
  }
  const size_t base = (size_t)g * (P + B) + b;  // slot of piece w is base + w
  const int eoff = 16 * sl + 4 * f;             // this thread's first output element
  float M = kNegInf, lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int w = w0 + p; w <= w1; w += NB * NP) {
    // Pieces past w1 re-read w1's slot and get weight zero.
    float2 ml[NB];
    float4 x[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const size_t slot = base + min(w + j * NP, w1);
      ml[j] = ws_ml[slot * COLS + col];
      x[j] = *reinterpret_cast<const float4 *>(ws_o + (slot * COLS + col) * D + eoff);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool live = w + j * NP <= w1 && ml[j].x != kNegInf;
      const float Mn = live ? fmaxf(M, ml[j].x) : M;
      const float a = live ? exp2_hw(M - Mn) : 1.f;
      const float c = live ? exp2_hw(ml[j].x - Mn) : 0.f;
      lsum = lsum * a + ml[j].y * c;
      acc.x = acc.x * a + x[j].x * c;
      acc.y = acc.y * a + x[j].y * c;
      acc.z = acc.z * a + x[j].z * c;
      acc.w = acc.w * a + x[j].w * c;
      M = Mn;
    }
  }
  s_acc[p][f] = acc;
  if (f == 0) s_m[p] = M, s_l[p] = lsum;
  for (int h = NP / 2; h >= 1; h >>= 1) {
    __syncthreads();
    if (p < h) {
      const float m2 = s_m[p + h];
      if (m2 != kNegInf) {
        const float Mn = fmaxf(M, m2);
        const float a = exp2_hw(M - Mn), c = exp2_hw(m2 - Mn);
        const float4 y = s_acc[p + h][f];
        lsum = lsum * a + s_l[p + h] * c;
        acc.x = acc.x * a + y.x * c;
        acc.y = acc.y * a + y.y * c;
        acc.z = acc.z * a + y.z * c;
        acc.w = acc.w * a + y.w * c;
        M = Mn;
      }
    }
    __syncthreads();
    if (p < h) {
      s_acc[p][f] = acc;
      if (f == 0) s_m[p] = M, s_l[p] = lsum;
    }
  }
  if (p != 0) return;
  const int ct = col / G, chead = g * G + col % G;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t *dst = o + ((size_t)(b * sq + ct) * Hq + chead) * D + eoff;
  *reinterpret_cast<uint2 *>(dst) = make_uint2(pack2<F16>(acc.x * inv, acc.y * inv), pack2<F16>(acc.z * inv, acc.w * inv));
  if (lse != nullptr && sl == 0 && f == 0)
    lse[((size_t)b * Hq + chead) * sq + ct] = lsum > 0.f ? kLn2 * (M + __log2f(lsum)) : kNegInf;
}

}  // namespace

// Work split of a decode call, from host integers only. One work-group per
// (sequence, KV head) needs no plan, partials or combine launch, but each pair
// then streams through a single CU (measured ~33 GB/s for a long pair against
// 7.2 TB/s for the chip), so it is chosen only where that does not bind:
// calls with no workspace (where the alternative is one piece per KV head),
// calls whose whole cache holds at most 256 KB of K/V, and 128 to 512 pairs of
// at most 512 KB each (measured 5-29% faster there, slower above and below).
bool use_grouped(int batch, int Hkv, int d, int max_len, bool have_workspace) {
  if (!have_workspace) return true;
  const long long pair_bytes = (long long)max_len * 4 * d;  // K and V of one pair at capacity, bf16
  const long long pairs = (long long)batch * Hkv;
  if (pairs * pair_bytes <= (256LL << 10)) return true;
  return pair_bytes <= (512LL << 10) && pairs >= 128 && pairs <= 512;
}

// Host-side launcher (called by the C ABI after validation). Work-groups:
// B x Hkv for the grouped kernel (no combine); otherwise ceil(Hkv * P / 4)
// for the split kernel (extra waves exit at once when the keys allow fewer
// pieces) and, for the combine, B x Hkv when the pieces per sequence are few
// (P <= kSliceCombine * B), else one per 16-float output slice of every packed
// column of every (sequence, KV head).
hipError_t launch_decode(const void *q, const void *k, const void *v, const int32_t *seqlens,
                         void *o, float *lse, float *ws_o, float2 *ws_ml, long long *meta,
                         int batch, int Hq,
                         int Hkv, int d, int sq, int max_len, int pieces, int min_piece,
                         float scale_log2, bool f16, hipStream_t stream) {
  const dim3 block(256);
  const dim3 grid((unsigned)(((long)Hkv * pieces + kWaves - 1) / kWaves));
  const int min_units = min_piece > kSub ? min_piece / kSub : 1;
  const auto *qq = static_cast<const uint16_t *>(q);
  const auto *kk = static_cast<const uint16_t *>(k);
  const auto *vv = static_cast<const uint16_t *>(v);
  auto *oo = static_cast<uint16_t *>(o);
  // One column group for up to 16 packed query rows, two for up to 32.
  const bool wide = (Hq / Hkv) * sq > kCols;
  const bool grouped = use_grouped(batch, Hkv, d, max_len, ws_o != nullptr);
  const dim3 ggrid((unsigned)((long)batch * Hkv));
  auto split = [&](auto kern) {
    hipLaunchKernelGGL(kern, grouped ? ggrid : grid, block, 0, stream, qq, kk, vv, seqlens, oo, lse, ws_o, ws_ml,
                       meta, batch, Hq, Hkv, sq, max_len, pieces, min_units, scale_log2);
  };
  auto pick = [&](auto kg, auto ks) {
    if (grouped) split(kg);
    else split(ks);
  };
  if (d == 256) {
    // One column group only (the C ABI rejects more than 16 packed rows here).
    if (f16) pick(decode_stream<256, true, 1, true>, decode_stream<256, true, 1, false>);
    else pick(decode_stream<256, false, 1, true>, decode_stream<256, false, 1, false>);
  } else if (d == 128) {
    if (f16) wide ? pick(decode_stream<128, true, 2, true>, decode_stream<128, true, 2, false>)
                  : pick(decode_stream<128, true, 1, true>, decode_stream<128, true, 1, false>);
    else wide ? pick(decode_stream<128, false, 2, true>, decode_stream<128, false, 2, false>)
              : pick(decode_stream<128, false, 1, true>, decode_stream<128, false, 1, false>);
  } else {
    if (f16) wide ? pick(decode_stream<64, true, 2, true>, decode_stream<64, true, 2, false>)
                  : pick(decode_stream<64, true, 1, true>, decode_stream<64, true, 1, false>);
    else wide ? pick(decode_stream<64, false, 2, true>, decode_stream<64, false, 2, false>)
              : pick(decode_stream<64, false, 1, true>, decode_stream<64, false, 1, false>);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (grouped) return hipSuccess;  // merged in the kernel: no combine step
  // Launched even with one piece per KV head: it writes O = 0 and LSE = -inf
  // for empty sequences, which no split-kernel wave visits.
  if (pieces > kSliceCombine * batch) {
    const int ncol = (Hq / Hkv) * sq;
    const dim3 sgrid((unsigned)(ncol * (d / 16)), Hkv, batch);
    auto slices = [&](auto kern) {
      hipLaunchKernelGGL(kern, sgrid, dim3(256), 0, stream, ws_o, ws_ml, meta, seqlens, oo, lse, batch, Hq, Hkv,
                         sq, max_len, pieces, min_units);
    };
    if (d == 256) {
      if (f16) slices(combine_slices<256, true, 1>);
      else slices(combine_slices<256, false, 1>);
    } else if (d == 128) {
      if (f16) wide ? slices(combine_slices<128, true, 2>) : slices(combine_slices<128, true, 1>);
      else wide ? slices(combine_slices<128, false, 2>) : slices(combine_slices<128, false, 1>);
    } else {
      if (f16) wide ? slices(combine_slices<64, true, 2>) : slices(combine_slices<64, true, 1>);
      else wide ? slices(combine_slices<64, false, 2>) : slices(combine_slices<64, false, 1>);
    }
    return hipGetLastError();
  }
  const dim3 cgrid(batch, Hkv), cblock(wide ? 512 : 256);
  auto combine = [&](auto kern) {
    hipLaunchKernelGGL(kern, cgrid, cblock, 0, stream, ws_o, ws_ml, meta, seqlens, oo, lse, batch, Hq, Hkv, sq,
                       max_len, pieces, min_units);
  };
  if (d == 256) {
    if (f16) combine(combine_pieces<256, true, 1>);
    else combine(combine_pieces<256, false, 1>);
  } else if (d == 128) {
    if (f16) wide ? combine(combine_pieces<128, true, 2>) : combine(combine_pieces<128, true, 1>);
    else wide ? combine(combine_pieces<128, false, 2>) : combine(combine_pieces<128, false, 1>);
  } else {
    if (f16) wide ? combine(combine_pieces<64, true, 2>) : combine(combine_pieces<64, true, 1>);
    else wide ? combine(combine_pieces<64, false, 2>) : combine(combine_pieces<64, false, 1>);
  }
  return hipGetLastError();
}

}  // namespace attn

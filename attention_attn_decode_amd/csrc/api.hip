// C ABI of the attention library: argument validation, split planning and
// kernel launches on the caller's stream. Declarations and the contract of
// every entry point live in include/attn.h.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include <hip/hip_runtime.h>

#include "attn.h"

namespace attn {
// Compute units of the current device, queried once per device and cached
// (256, the MI355X count, if the query fails). Called at launch only, when the
// caller already uses the device: the host-only plan and workspace calls do
// not query the device.
int current_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) return 256;
  if (dev < 64) cache[dev].store(ncu, std::memory_order_relaxed);
  return ncu;
}

hipError_t launch_decode(const void *q, const void *k, const void *v, const int32_t *seqlens,
                         void *o, float *lse, float *ws_o, float2 *ws_ml, long long *meta,
                         int batch, int Hq,
                         int Hkv, int d, int sq, int max_len, int pieces, int min_piece,
                         float scale_log2, bool f16, hipStream_t stream);
hipError_t launch_fwd(const void *q, const void *k, const void *v, void *o, float *lse, const int *cu_q,
                      const int *cu_k, int total_q, int total_k, int causal, int batch, int Sq, int Sk, int Hq,
                      int Hkv, int d, float scale_log2, bool f16, hipStream_t stream);
hipError_t launch_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                      void *dq, void *dk, void *dv, const int *cu_q, const int *cu_k, int total_q, int total_k,
                      int causal, int batch, int Sq, int Sk, int Hq, int Hkv, int d, float *l2ws, float *dws, bool f16,
                      hipStream_t stream);
int bwd_sq_pad(int Sq);
int bwd_varlen_pad(int total_q);
}  // namespace attn

namespace {

// Independent decode workers (waves) the automatic plan spreads over all KV
// heads. Measured on MI355X (256 CUs): d = 64 streams best with one work-group
// of four waves per CU (1024 workers); d = 128, whose sub-blocks keep twice the
// bytes in flight per wave, best with 7/8 of that (896) - more concurrent
// streams lower the achieved HBM bandwidth - unless its pieces would be short:
// below 32 sub-blocks (1024 keys) of capacity per piece at 896 workers, a wave's
// time is its start-up and load latency rather than its share of the bandwidth,
// and 1024 workers finish sooner (batch-1 GQA calls over 32k-128k keys).
int auto_workers(int d, int batch, int n_kv_heads, int max_seqlen_k) {
  if (d < 128) return 1024;
  if (d == 128) {
    const long long units = (long long)batch * ((max_seqlen_k + 31) / 32);  // capacity per KV head
    const long long pieces896 = (896 + n_kv_heads - 1) / n_kv_heads;
    if (units < 32 * pieces896) return 1024;
  }
  return 896;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// log2(e) / sqrt(d): the softmax runs in base 2 on fp32 scores.
float scale_log2_for(int d) { return static_cast<float>(1.4426950408889634 / std::sqrt((double)d)); }

int check_decode_shape(int n_q_heads, int n_kv_heads, int d, int seqlen_q, int batch,
                       int max_seqlen_k) {
  if (n_q_heads <= 0 || n_kv_heads <= 0 || seqlen_q <= 0 || batch <= 0 || max_seqlen_k <= 0)
    return ATTN_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
  if (batch > ATTN_MAX_BATCH || n_kv_heads > 65535) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  // Packed query rows per KV head: two 16-column groups at d <= 128, one at d = 256.
  if ((long)(n_q_heads / n_kv_heads) * seqlen_q > (d == 256 ? 16 : 32)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Packed query columns per partial slot: one group of 16, or two when the
// packed rows (G * seqlen_q) exceed 16.
unsigned decode_cols(int n_q_heads, int n_kv_heads, int seqlen_q) {
  return (n_q_heads / n_kv_heads) * seqlen_q > 16 ? 32u : 16u;
}

int plan_pieces(int batch, int n_kv_heads, int d, int max_seqlen_k, int num_splits) {
  const int w = auto_workers(d, batch, n_kv_heads, max_seqlen_k);
  int p = num_splits > 0 ? num_splits : (w + n_kv_heads - 1) / n_kv_heads;
  if (p > ATTN_MAX_PIECES) p = ATTN_MAX_PIECES;
  return p < 1 ? 1 : p;
}

// Partial outputs, then (max, denominator) pairs, then the key total and the
// flattened start of every sequence (int64).
size_t workspace_bytes_for(int batch, int n_kv_heads, int d, int pieces, unsigned cols) {
  if (pieces <= 1) return 0;
  return (size_t)n_kv_heads * (size_t)(pieces + batch) * cols * (size_t)(d + 2) * 4u +
         (size_t)(batch + 1) * 8u;
}

}  // namespace

extern "C" {

int attn_decode_plan(int batch, int n_q_heads, int n_kv_heads, int d, int seqlen_q,
                     int max_seqlen_k, int num_splits, int *pieces, int *min_piece) {
  if (pieces == nullptr || min_piece == nullptr || num_splits < 0) return ATTN_ERR_INVALID;
  const int st = check_decode_shape(n_q_heads, n_kv_heads, d, seqlen_q, batch, max_seqlen_k);
  if (st != ATTN_OK) return st;
  *pieces = plan_pieces(batch, n_kv_heads, d, max_seqlen_k, num_splits);
  *min_piece = ATTN_MIN_PIECE;
  return ATTN_OK;
}

size_t attn_decode_workspace_size(int batch, int n_q_heads, int n_kv_heads, int seqlen_q, int d,
                                  int max_seqlen_k, int num_splits) {
  if (num_splits < 0 ||
      check_decode_shape(n_q_heads, n_kv_heads, d, seqlen_q, batch, max_seqlen_k) != ATTN_OK)
    return 0;
  return workspace_bytes_for(batch, n_kv_heads, d, plan_pieces(batch, n_kv_heads, d, max_seqlen_k, num_splits),
                             decode_cols(n_q_heads, n_kv_heads, seqlen_q));
}

}  // extern "C"

namespace {

// Device scratch of attn_decode_noalloc: the partial outputs, maxima,
// denominators and plan data of one decode call. HIP places a copy of this
// array on every GPU the library runs on, each at its own address, held until
// the process ends. Host code never passes the array's name to a kernel (on
// the host it only stands for the symbol): it looks up the device address of
// the current GPU's copy once and uses that pointer.
__device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];  // per device id; guarded by scratch_mutex

// Address of the current device's copy of `scratch`, looked up with that
// device current on its first use, then cached. nullptr if HIP cannot report it.
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

int decode_impl(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens_k,
                void *o, float *lse, int n_q_heads, int n_kv_heads, int d, int seqlen_q, int batch,
                int max_seqlen_k, void *workspace, size_t workspace_bytes, void *stream,
                int num_splits, bool f16) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !o || num_splits < 0) return ATTN_ERR_INVALID;
  const int st = check_decode_shape(n_q_heads, n_kv_heads, d, seqlen_q, batch, max_seqlen_k);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned4(seqlens_k) || (lse && !aligned4(lse)) || (workspace && !aligned16(workspace)))
    return ATTN_ERR_MISALIGNED;
  // Without a workspace, one piece per KV head: every sequence is finished by
  // the wave that streams it and no partial is stored.
  const int pieces = workspace ? plan_pieces(batch, n_kv_heads, d, max_seqlen_k, num_splits) : 1;
  const unsigned cols = decode_cols(n_q_heads, n_kv_heads, seqlen_q);
  const size_t need = workspace_bytes_for(batch, n_kv_heads, d, pieces, cols);
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  float *ws_o = nullptr;
  float2 *ws_ml = nullptr;
  long long *meta = nullptr;
  if (need > 0) {
    const size_t slots = (size_t)n_kv_heads * (pieces + batch) * cols;
    ws_o = static_cast<float *>(workspace);
    ws_ml = reinterpret_cast<float2 *>(ws_o + slots * d);
    meta = reinterpret_cast<long long *>(ws_ml + slots);
  }
  const hipError_t err = attn::launch_decode(
      q, k_cache, v_cache, seqlens_k, o, lse, ws_o, ws_ml, meta, batch, n_q_heads, n_kv_heads, d,
      seqlen_q, max_seqlen_k, pieces, ATTN_MIN_PIECE, scale_log2_for(d), f16,
      static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int causal, int batch,
             int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads, int d, void *stream, bool f16) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID;
  if (batch <= 0 || seqlen_q <= 0 || seqlen_k <= 0 || n_q_heads <= 0 || n_kv_heads <= 0)
    return ATTN_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  const long wgs = (long)((seqlen_q + 255) / 256) * batch * n_q_heads;  // 256-row query tiles
  if (wgs > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned4(lse)))
    return ATTN_ERR_MISALIGNED;
  const hipError_t err =
      attn::launch_fwd(q, k, v, o, lse, nullptr, nullptr, 0, 0, causal ? 1 : 0, batch, seqlen_q, seqlen_k,
                       n_q_heads, n_kv_heads, d, scale_log2_for(d), f16, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int fwd_varlen_impl(const void *q, const void *k, const void *v, const int32_t *cu_q, const int32_t *cu_k, void *o,
                    float *lse, int causal, int batch, int max_seqlen_q, int total_q, int total_k, int n_q_heads,
                    int n_kv_heads, int d, void *stream, bool f16) {
  if (!q || !o || !cu_q || !cu_k || (total_k > 0 && (!k || !v))) return ATTN_ERR_INVALID;
  if (batch <= 0 || max_seqlen_q <= 0 || total_q <= 0 || total_k < 0 || n_q_heads <= 0 || n_kv_heads <= 0)
    return ATTN_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  const long wgs = (long)((max_seqlen_q + 255) / 256) * batch * n_q_heads;
  if (wgs > 0x7fffffffL || (long long)total_q * n_q_heads > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || (k && !aligned16(k)) || (v && !aligned16(v)) || !aligned16(o) || (lse && !aligned4(lse)) ||
      !aligned4(cu_q) || !aligned4(cu_k))
    return ATTN_ERR_MISALIGNED;
  const hipError_t err =
      attn::launch_fwd(q, k, v, o, lse, cu_q, cu_k, total_q, total_k, causal ? 1 : 0, batch, max_seqlen_q, 0,
                       n_q_heads, n_kv_heads, d, scale_log2_for(d), f16, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Backward workspace: base-2 LSE and D per (batch, head) row, rows padded to
// a multiple of 128 queries.
size_t bwd_workspace(int batch, int n_q_heads, int seqlen_q) {
  return 2 * (size_t)batch * (size_t)n_q_heads * (size_t)attn::bwd_sq_pad(seqlen_q) * sizeof(float);
}

int bwd_impl(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
             void *dq, void *dk, void *dv, int causal, int batch, int seqlen_q, int seqlen_k, int n_q_heads,
             int n_kv_heads, int d, void *workspace, size_t workspace_bytes, void *stream, bool f16) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return ATTN_ERR_INVALID;
  if (batch <= 0 || seqlen_q <= 0 || seqlen_k <= 0 || n_q_heads <= 0 || n_kv_heads <= 0)
    return ATTN_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (n_q_heads > 65535) return ATTN_ERR_UNSUPPORTED;  // keeps in-tile byte offsets in 32 bits
  const long long qtiles = (long long)(seqlen_q + 127) / 128 * batch * n_q_heads;
  const long long ktiles = (long long)(seqlen_k + 127) / 128 * batch * n_kv_heads;
  const long long rows = (long long)attn::bwd_sq_pad(seqlen_q) * batch * n_q_heads;
  if (qtiles > 0x7fffffffLL || ktiles > 0x7fffffffLL || rows > 0x3fffffffLL) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned4(lse) || !aligned16(workspace))
    return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < bwd_workspace(batch, n_q_heads, seqlen_q)) return ATTN_ERR_WORKSPACE;
  float *l2ws = static_cast<float *>(workspace);
  float *dws = l2ws + rows;
  const hipError_t err =
      attn::launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, 0, 0, causal ? 1 : 0, batch, seqlen_q,
                       seqlen_k, n_q_heads, n_kv_heads, d, l2ws, dws, f16, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

size_t bwd_varlen_workspace(int n_q_heads, int total_q) {
  return 2 * (size_t)n_q_heads * (size_t)attn::bwd_varlen_pad(total_q) * sizeof(float);
}

int bwd_varlen_impl(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                    void *dq, void *dk, void *dv, const int32_t *cu_q, const int32_t *cu_k, int causal, int batch,
                    int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int n_q_heads, int n_kv_heads, int d,
                    void *workspace, size_t workspace_bytes, void *stream, bool f16) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_q || !cu_k || !workspace)
    return ATTN_ERR_INVALID;
  if (batch <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0 || total_q <= 0 || total_k <= 0 || n_q_heads <= 0 ||
      n_kv_heads <= 0)
    return ATTN_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (n_q_heads > 65535) return ATTN_ERR_UNSUPPORTED;
  const long long qtiles = (long long)(max_seqlen_q + 127) / 128 * batch * n_q_heads;
  const long long ktiles = (long long)(max_seqlen_k + 127) / 128 * batch * n_kv_heads;
  const long long rows = (long long)attn::bwd_varlen_pad(total_q) * n_q_heads;
  if (qtiles > 0x7fffffffLL || ktiles > 0x7fffffffLL || rows > 0x3fffffffLL || total_q > 0x3fffff00)
    return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned4(lse) || !aligned4(cu_q) || !aligned4(cu_k) ||
      !aligned16(workspace))
    return ATTN_ERR_MISALIGNED;
  if (workspace_bytes < bwd_varlen_workspace(n_q_heads, total_q)) return ATTN_ERR_WORKSPACE;
  float *l2ws = static_cast<float *>(workspace);
  float *dws = l2ws + rows;
  const hipError_t err =
      attn::launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, cu_q, cu_k, total_q, total_k, causal ? 1 : 0, batch,
                       max_seqlen_q, max_seqlen_k, n_q_heads, n_kv_heads, d, l2ws, dws, f16,
                       static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_size(int batch, int n_q_heads, int seqlen_q) {
  if (batch <= 0 || n_q_heads <= 0 || seqlen_q <= 0) return 0;
  return bwd_workspace(batch, n_q_heads, seqlen_q);
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
             void *dq, void *dk, void *dv, int causal, int batch, int seqlen_q, int seqlen_k, int n_q_heads,
             int n_kv_heads, int d, void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, causal, batch, seqlen_q, seqlen_k, n_q_heads, n_kv_heads, d,
                  workspace, workspace_bytes, stream, false);
}

int attn_bwd_f16(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                 void *dq, void *dk, void *dv, int causal, int batch, int seqlen_q, int seqlen_k, int n_q_heads,
                 int n_kv_heads, int d, void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, causal, batch, seqlen_q, seqlen_k, n_q_heads, n_kv_heads, d,
                  workspace, workspace_bytes, stream, true);
}

size_t attn_bwd_varlen_workspace_size(int n_q_heads, int total_q) {
  if (n_q_heads <= 0 || total_q <= 0) return 0;
  return bwd_varlen_workspace(n_q_heads, total_q);
}

int attn_bwd_varlen(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                    void *dq, void *dk, void *dv, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int causal,
                    int batch, int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int n_q_heads,
                    int n_kv_heads, int d, void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, causal, batch, max_seqlen_q,
                         max_seqlen_k, total_q, total_k, n_q_heads, n_kv_heads, d, workspace, workspace_bytes, stream,
                         false);
}

int attn_bwd_varlen_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dout, void *dq, void *dk, void *dv, const int32_t *cu_seqlens_q,
                        const int32_t *cu_seqlens_k, int causal, int batch, int max_seqlen_q, int max_seqlen_k,
                        int total_q, int total_k, int n_q_heads, int n_kv_heads, int d, void *workspace,
                        size_t workspace_bytes, void *stream) {
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, causal, batch, max_seqlen_q,
                         max_seqlen_k, total_q, total_k, n_q_heads, n_kv_heads, d, workspace, workspace_bytes, stream,
                         true);
}

int attn_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *seqlens_k, void *o, float *lse, int n_q_heads, int n_kv_heads,
                   int d, int seqlen_q, int batch, int max_seqlen_k, void *workspace,
                   size_t workspace_bytes, void *stream, int num_splits) {
  return decode_impl(q, k_cache, v_cache, seqlens_k, o, lse, n_q_heads, n_kv_heads, d, seqlen_q, batch,
                     max_seqlen_k, workspace, workspace_bytes, stream, num_splits, false);
}

int attn_decode_f16(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *seqlens_k, void *o, float *lse, int n_q_heads, int n_kv_heads,
                    int d, int seqlen_q, int batch, int max_seqlen_k, void *workspace,
                    size_t workspace_bytes, void *stream, int num_splits) {
  return decode_impl(q, k_cache, v_cache, seqlens_k, o, lse, n_q_heads, n_kv_heads, d, seqlen_q, batch,
                     max_seqlen_k, workspace, workspace_bytes, stream, num_splits, true);
}

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens_k,
                void *o, float *lse, int n_q_heads, int n_kv_heads, int d, int seqlen_q, int batch,
                int max_seqlen_k, void *workspace, size_t workspace_bytes, void *stream) {
  return attn_decode_ex(q, k_cache, v_cache, seqlens_k, o, lse, n_q_heads, n_kv_heads, d, seqlen_q,
                        batch, max_seqlen_k, workspace, workspace_bytes, stream, 0);
}

int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens_k,
                        void *o, float *lse, int n_q_heads, int n_kv_heads, int d, int seqlen_q, int batch,
                        int max_seqlen_k, void *stream, int num_splits) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !o || num_splits < 0) return ATTN_ERR_INVALID;
  const int st = check_decode_shape(n_q_heads, n_kv_heads, d, seqlen_q, batch, max_seqlen_k);
  if (st != ATTN_OK) return st;
  const size_t need = workspace_bytes_for(batch, n_kv_heads, d, plan_pieces(batch, n_kv_heads, d, max_seqlen_k, num_splits),
                                          decode_cols(n_q_heads, n_kv_heads, seqlen_q));
  if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_TOO_LARGE;
  void *ws = device_scratch();
  if (ws == nullptr) return ATTN_ERR_DEVICE;
  return decode_impl(q, k_cache, v_cache, seqlens_k, o, lse, n_q_heads, n_kv_heads, d, seqlen_q, batch,
                     max_seqlen_k, ws, ATTN_NOALLOC_SCRATCH_BYTES, stream, num_splits, false);
}

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
             int batch, int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads, int d,
             void *stream) {
  return fwd_impl(q, k, v, o, lse, causal, batch, seqlen_q, seqlen_k, n_q_heads, n_kv_heads, d, stream, false);
}

int attn_fwd_f16(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
                 int batch, int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads, int d,
                 void *stream) {
  return fwd_impl(q, k, v, o, lse, causal, batch, seqlen_q, seqlen_k, n_q_heads, n_kv_heads, d, stream, true);
}

int attn_fwd_varlen(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                    const int32_t *cu_seqlens_k, void *o, float *lse, int causal, int batch, int max_seqlen_q,
                    int total_q, int total_k, int n_q_heads, int n_kv_heads, int d, void *stream) {
  return fwd_varlen_impl(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, causal, batch, max_seqlen_q, total_q, total_k,
                         n_q_heads, n_kv_heads, d, stream, false);
}

int attn_fwd_varlen_f16(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                        const int32_t *cu_seqlens_k, void *o, float *lse, int causal, int batch, int max_seqlen_q,
                        int total_q, int total_k, int n_q_heads, int n_kv_heads, int d, void *stream) {
  return fwd_varlen_impl(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, causal, batch, max_seqlen_q, total_q, total_k,
                         n_q_heads, n_kv_heads, d, stream, true);
}

const char *attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported shape (decode and forward: d in {64, 128, 256}; backward: d in {64, 128}; "
             "decode: packed query rows per KV head <= 32, <= 16 at d = 256, batch <= 8192)";
    case ATTN_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case ATTN_ERR_DEVICE: return "no usable HIP device";
    case ATTN_ERR_TOO_LARGE: return "call needs more than the library's fixed decode scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

const char *attn_version(void) { return "attn-mi355x 0.1.0 gfx950"; }

}  // extern "C"

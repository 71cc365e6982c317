// C ABI of the attention library: argument validation, split planning and
// kernel launches on the caller's stream. Declarations and the contract of
// every entry point live in include/attn.h.
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "attn.h"

namespace attn {
hipError_t launch_decode(const void *q, const void *k, const void *v, const int32_t *seqlens,
                         void *o, float *lse, float *ws_o, float2 *ws_ml, int batch, int Hq,
                         int Hkv, int d, int sq, int max_len, int chunk, int n_split,
                         float scale_log2, hipStream_t stream);
hipError_t launch_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
                      int batch, int Sq, int Sk, int Hq, int Hkv, int d, float scale_log2,
                      hipStream_t stream);
}  // namespace attn

namespace {

// Work-groups the automatic decode plan aims for: 16 per CU of a 256-CU part,
// enough that ragged sequence lengths (whose splits past the end exit at once)
// still leave every CU several work-groups.
constexpr long kTargetWorkGroups = 4096;
// Smallest automatic chunk: two 128-key passes of the four-wave work-group.
constexpr int kMinAutoChunk = 256;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int ceil_div(long a, long b) { return static_cast<int>((a + b - 1) / b); }

int split_cap(int max_seqlen_k) {
  const int by_len = ceil_div(max_seqlen_k, ATTN_SPLIT_QUANTUM);
  return by_len < ATTN_MAX_SPLITS ? by_len : ATTN_MAX_SPLITS;
}

// log2(e) / sqrt(d): the softmax runs in base 2 on fp32 scores.
float scale_log2_for(int d) { return static_cast<float>(1.4426950408889634 / std::sqrt((double)d)); }

int check_decode_shape(int n_q_heads, int n_kv_heads, int d, int seqlen_q, int batch,
                       int max_seqlen_k) {
  if (n_q_heads <= 0 || n_kv_heads <= 0 || seqlen_q <= 0 || batch <= 0 || max_seqlen_k <= 0)
    return ATTN_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
  if (n_kv_heads > 65535 || batch > 65535) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long)(n_q_heads / n_kv_heads) * seqlen_q > 16) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_plan(int batch, int n_q_heads, int n_kv_heads, int d, int seqlen_q,
                     int max_seqlen_k, int num_splits, int *n_split, int *chunk) {
  if (n_split == nullptr || chunk == nullptr || num_splits < 0) return ATTN_ERR_INVALID;
  const int st = check_decode_shape(n_q_heads, n_kv_heads, d, seqlen_q, batch, max_seqlen_k);
  if (st != ATTN_OK) return st;
  const int cap = split_cap(max_seqlen_k);
  long n;
  if (num_splits > 0) {
    n = num_splits;
  } else {
    const long units = (long)batch * n_kv_heads;
    n = (kTargetWorkGroups + units - 1) / units;
    const int by_min_chunk = ceil_div(max_seqlen_k, kMinAutoChunk);
    if (n > by_min_chunk) n = by_min_chunk;
  }
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  int c = ceil_div(ceil_div(max_seqlen_k, n), ATTN_SPLIT_QUANTUM) * ATTN_SPLIT_QUANTUM;
  *chunk = c;
  *n_split = ceil_div(max_seqlen_k, c);
  return ATTN_OK;
}

size_t attn_decode_workspace_size(int batch, int n_q_heads, int seqlen_q, int d, int max_seqlen_k) {
  if (batch <= 0 || n_q_heads <= 0 || seqlen_q <= 0 || d <= 0 || max_seqlen_k <= 0) return 0;
  return (size_t)batch * n_q_heads * seqlen_q * split_cap(max_seqlen_k) * (size_t)(d + 2) * 4u;
}

int attn_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *seqlens_k, void *o, float *lse, int n_q_heads, int n_kv_heads,
                   int d, int seqlen_q, int batch, int max_seqlen_k, void *workspace,
                   size_t workspace_bytes, void *stream, int num_splits) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !o) return ATTN_ERR_INVALID;
  int st = check_decode_shape(n_q_heads, n_kv_heads, d, seqlen_q, batch, max_seqlen_k);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned4(seqlens_k) || (lse && !aligned4(lse)) || (workspace && !aligned16(workspace)))
    return ATTN_ERR_MISALIGNED;
  int n_split = 1, chunk = 0;
  st = attn_decode_plan(batch, n_q_heads, n_kv_heads, d, seqlen_q, max_seqlen_k,
                        workspace ? num_splits : 1, &n_split, &chunk);
  if (st != ATTN_OK) return st;
  if (workspace == nullptr) {
    n_split = 1;
    chunk = ceil_div(max_seqlen_k, ATTN_SPLIT_QUANTUM) * ATTN_SPLIT_QUANTUM;
  }
  float *ws_o = nullptr;
  float2 *ws_ml = nullptr;
  if (n_split > 1) {
    const size_t rows = (size_t)batch * n_q_heads * seqlen_q;
    const size_t need = rows * n_split * (size_t)(d + 2) * 4u;
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    ws_o = static_cast<float *>(workspace);
    ws_ml = reinterpret_cast<float2 *>(ws_o + rows * n_split * d);
  }
  const hipError_t err = attn::launch_decode(
      q, k_cache, v_cache, seqlens_k, o, lse, ws_o, ws_ml, batch, n_q_heads, n_kv_heads, d,
      seqlen_q, max_seqlen_k, chunk, n_split, scale_log2_for(d), static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seqlens_k,
                void *o, float *lse, int n_q_heads, int n_kv_heads, int d, int seqlen_q, int batch,
                int max_seqlen_k, void *workspace, size_t workspace_bytes, void *stream) {
  return attn_decode_ex(q, k_cache, v_cache, seqlens_k, o, lse, n_q_heads, n_kv_heads, d, seqlen_q,
                        batch, max_seqlen_k, workspace, workspace_bytes, stream, 0);
}

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
             int batch, int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads, int d,
             void *stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID;
  if (batch <= 0 || seqlen_q <= 0 || seqlen_k <= 0 || n_q_heads <= 0 || n_kv_heads <= 0)
    return ATTN_ERR_INVALID;
  if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_INVALID;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  const long wgs = (long)((seqlen_q + 127) / 128) * batch * n_q_heads;
  if (wgs > 0x7fffffffL) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned4(lse)))
    return ATTN_ERR_MISALIGNED;
  const hipError_t err =
      attn::launch_fwd(q, k, v, o, lse, causal ? 1 : 0, batch, seqlen_q, seqlen_k, n_q_heads,
                       n_kv_heads, d, scale_log2_for(d), static_cast<hipStream_t>(stream));
  return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

const char *attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported shape (d must be 64 or 128; packed query rows <= 16)";
    case ATTN_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case ATTN_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown status";
  }
}

const char *attn_version(void) { return "attn-mi355x 0.1.0 gfx950"; }

}  // extern "C"

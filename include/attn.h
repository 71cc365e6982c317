/*
 * attn.h - fused attention forward for MI355X (gfx950): KV-cache decode with
 * grouped-query attention and split-KV, and (causal) prefill.
 *
 * Pages cited by title and section:
 *   [FA4-decode]  "Optimization diaries: S/P ping-pong for FlashAttention-4 decode"
 *   [FA4-bwd]     "Optimization diaries: Improving FlashAttention-4 backward pass
 *                  kernel design for head dimension 64"
 *   [GQA-SM100]   "Building a Faster GQA Decode Kernel for Blackwell SM100"
 *   [FA4-edges]   "Flash Attention 4 — warp-role choreography and the edges"
 *
 * What every entry point computes ([FA4-decode] §Recap on the FA4 forward pass):
 *   S = Q K^T / sqrt(d),  P = softmax(S) row-wise,  O = P V,
 * without materialising S or P, plus the natural-log log-sum-exp of each score
 * row, LSE = log(sum_j exp(S_j)) (the quantity the backward pass consumes as
 * P = exp(S - LSE), [FA4-bwd] §Recap on the FA4 backward pass).
 *
 * Conventions shared by all calls
 *   - Element types: Q, K, V, O are bfloat16 (passed as raw 16-bit patterns);
 *     LSE is float32. Softmax and accumulation run in fp32; P is rounded to
 *     bf16 (nearest even) before the P*V product; O is rounded to bf16 (nearest
 *     even) once, at the end.
 *   - Layouts are dense, row-major, with the head dimension d innermost:
 *       q, o          [batch][seqlen_q][n_q_heads][d]
 *       k, v (cache)  [batch][seq capacity][n_kv_heads][d]
 *       lse           [batch][n_q_heads][seqlen_q]
 *   - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads); the query
 *     heads sharing one KV head are contiguous ([FA4-edges] §Edge 2 · GQA).
 *   - Causal masking is bottom-right aligned: with L keys and sq queries, query
 *     t sees keys j <= L - sq + t ([FA4-edges] §Edge 1 · causal masking). For
 *     sq == L this is the usual lower triangle.
 *   - A query row with no visible key gets O = 0 and LSE = -inf ([GQA-SM100]
 *     §Removing the max reset: an entirely empty sequence produces zero output).
 *   - Memory: every pointer is device memory owned by the caller. The library
 *     never allocates, frees or memsets. Pointers to bf16/fp32 arrays must be
 *     16-byte aligned. `stream` is a hipStream_t passed as void* (NULL = the
 *     default stream). Work is only enqueued: no host synchronisation and no
 *     host read of device data, so calls may be captured in a hipGraph.
 *   - Errors: calls return synchronously with one of the ATTN_* codes below.
 *     Faults during execution surface at the caller's next synchronisation.
 *     Nothing is enqueued when a call returns an error other than
 *     ATTN_ERR_LAUNCH.
 *   - Thread safety: calls may be made concurrently from several host threads.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_INVALID (-1)     /* NULL pointer, a size <= 0, Hq % Hkv != 0, ... */
#define ATTN_ERR_UNSUPPORTED (-2) /* d not in {64, 128}; packed query rows > 16 */
#define ATTN_ERR_MISALIGNED (-3)  /* a data pointer not 16-byte aligned */
#define ATTN_ERR_WORKSPACE (-4)   /* workspace smaller than the plan needs */
#define ATTN_ERR_LAUNCH (-5)      /* the HIP runtime refused a launch */
#define ATTN_ERR_DEVICE (-6)      /* no usable HIP device */

/* Largest number of KV splits any decode plan uses. */
#define ATTN_MAX_SPLITS 64
/* Every split but the last covers a multiple of this many key positions. */
#define ATTN_SPLIT_QUANTUM 128

/*
 * Split plan of a decode call ([GQA-SM100] §Combining the KV splits: splitting
 * the KV sequence gives a small decode batch enough work-groups; each split
 * returns an unnormalised partial output, its maximum and its denominator).
 *
 * The plan depends only on host integers (never on the device contents of
 * seqlens_k): key range [0, max_seqlen_k) is cut into n_split chunks of
 * `chunk` positions (a multiple of ATTN_SPLIT_QUANTUM). num_splits = 0 asks for
 * the automatic choice; a positive value is honoured after clamping to
 * [1, min(ATTN_MAX_SPLITS, ceil(max_seqlen_k / ATTN_SPLIT_QUANTUM))].
 * Host-only; touches no device. Returns ATTN_OK or ATTN_ERR_INVALID.
 */
int attn_decode_plan(int batch, int n_q_heads, int n_kv_heads, int d, int seqlen_q,
                     int max_seqlen_k, int num_splits, int *n_split, int *chunk);

/*
 * Bytes of workspace any decode plan of this shape may need:
 *   batch * n_q_heads * seqlen_q * S * (d + 2) * 4,
 * S = min(ATTN_MAX_SPLITS, ceil(max_seqlen_k / ATTN_SPLIT_QUANTUM)). The
 * workspace holds per-split fp32 partial outputs, maxima and denominators. It
 * needs no initialisation (e.g. torch.empty): every value the combine step
 * reads is written by the same call ([GQA-SM100] §Removing the max reset).
 * Returns 0 for invalid sizes. Host-only.
 */
size_t attn_decode_workspace_size(int batch, int n_q_heads, int seqlen_q, int d,
                                  int max_seqlen_k);

/*
 * GQA KV-cache decode with split-KV and a log-sum-exp combine.
 *
 *   q          [batch][seqlen_q][n_q_heads][d] bf16, the new queries.
 *   k_cache,   [batch][max_seqlen_k][n_kv_heads][d] bf16, cache tensors at
 *   v_cache    capacity; for sequence b only rows [0, seqlens_k[b]) are read.
 *   seqlens_k  int32[batch] on the device: cached keys per sequence, counting
 *              the seqlen_q new tokens (already appended). Values are clamped
 *              to [0, max_seqlen_k] on the device.
 *   o          [batch][seqlen_q][n_q_heads][d] bf16, overwritten.
 *   lse        [batch][n_q_heads][seqlen_q] fp32 natural-log LSE, overwritten;
 *              may be NULL.
 *   The seqlen_q new tokens are causal among themselves (bottom-right mask).
 *   Requires d in {64, 128} and (n_q_heads / n_kv_heads) * seqlen_q <= 16.
 *   workspace / workspace_bytes: caller scratch of at least
 *   attn_decode_workspace_size(...) bytes; workspace == NULL forces a single
 *   split (no combine step).
 *
 * Device work: one split kernel over (split, kv head, batch) work-groups, then,
 * when the plan has more than one split, one combine kernel over query rows.
 * Both use only fp32 arithmetic on partials, in a fixed split order, with no
 * atomics: results are deterministic and bitwise reproducible.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *seqlens_k, void *o, float *lse, int n_q_heads,
                int n_kv_heads, int d, int seqlen_q, int batch, int max_seqlen_k,
                void *workspace, size_t workspace_bytes, void *stream);

/* attn_decode with an explicit split count (0 = automatic; see attn_decode_plan). */
int attn_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *seqlens_k, void *o, float *lse, int n_q_heads,
                   int n_kv_heads, int d, int seqlen_q, int batch, int max_seqlen_k,
                   void *workspace, size_t workspace_bytes, void *stream,
                   int num_splits);

/*
 * Prefill forward ([FA4-edges] §Edge 1 · causal masking, §Edge 3 · tile
 * scheduling): q [batch][seqlen_q][n_q_heads][d], k and v
 * [batch][seqlen_k][n_kv_heads][d], all bf16; o like q; lse
 * [batch][n_q_heads][seqlen_q] fp32 (may be NULL). causal != 0 applies the
 * bottom-right mask (query i sees keys j <= i + seqlen_k - seqlen_q).
 * Requires d == 128 or d == 64. Work-groups of 128 query rows are launched
 * heaviest first (longest visible key range first).
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
             int batch, int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads, int d,
             void *stream);

/* Static description of a status code; never NULL. */
const char *attn_status_string(int status);

/* Library version string, e.g. "attn-mi355x 0.1.0 gfx950". */
const char *attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */

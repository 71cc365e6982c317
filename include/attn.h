/*
 * attn.h - fused attention for MI355X (gfx950): KV-cache decode with
 * grouped-query attention and split-KV, (causal) prefill, and the backward
 * pass of prefill attention.
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
 *     the *_f16 entry points take IEEE fp16 instead, with the same layouts
 *     ([GQA-SM100] checks its decode kernel in BF16 and FP16; the correctness
 *     test of [FA4-edges] §Does it actually compute attention? runs fp16).
 *     LSE is float32.
 *     Softmax and accumulation run in fp32; P is rounded to the element type
 *     (nearest even) before the P*V product; O is rounded to the element type
 *     (nearest even) once, at the end.
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
#define ATTN_ERR_UNSUPPORTED (-2) /* head size or packed query rows out of range */
#define ATTN_ERR_MISALIGNED (-3)  /* a data pointer not 16-byte aligned */
#define ATTN_ERR_WORKSPACE (-4)   /* workspace smaller than the plan needs */
#define ATTN_ERR_LAUNCH (-5)      /* the HIP runtime refused a launch */
#define ATTN_ERR_DEVICE (-6)      /* no usable HIP device */
#define ATTN_ERR_TOO_LARGE (-7)   /* needs more than the fixed scratch of attn_decode_noalloc */

/* Largest number of key pieces per KV head a decode plan uses. */
#define ATTN_MAX_PIECES 4096
/* Shortest piece the device cuts (fewer pieces are used when keys are few). */
#define ATTN_MIN_PIECE 64
/* Most sequences one decode call accepts (their lengths are staged on chip). */
#define ATTN_MAX_BATCH 8192

/*
 * Split plan of a decode call ([GQA-SM100] §Combining the KV splits: splitting
 * the KV sequence gives a small decode batch enough parallel work; each split
 * returns an unnormalised partial output, its maximum and its denominator).
 *
 * The split is balanced on the device, from seqlens_k, without any host read,
 * in units of the 32-key sub-blocks a worker processes at a time: sequence b
 * has ceil(L_b / 32) of them; for each KV head the sub-blocks of all
 * sequences are laid end to end and cut into
 * P_eff = min(pieces, ceil(total_sub_blocks / (min_piece / 32))) equal pieces,
 * one per independent worker (a 64-lane wave), so every worker runs the same
 * number of sub-blocks to within one. A sequence inside one piece is finished
 * by that worker; a sequence spread over several pieces is merged by the
 * combine step. This call reports the host side of that plan: `pieces`, the
 * number of pieces per KV head (num_splits = 0 asks for the automatic value,
 * ceil(W / n_kv_heads) with W = 1024 workers for d = 64 and 896 for d >= 128,
 * about one work-group of four waves per CU on a 256-CU part, as measured best
 * for HBM streaming; at d = 128 W = 1024 also when the capacity per piece at
 * 896 workers, batch * ceil(max_seqlen_k / 32) / ceil(896 / n_kv_heads), is
 * under 32 sub-blocks of 32 keys, where short pieces are latency-bound; a
 * positive value is honoured up to ATTN_MAX_PIECES) and
 * `min_piece`.
 * Host-only; touches no device. Returns ATTN_OK or an error code.
 */
int attn_decode_plan(int batch, int n_q_heads, int n_kv_heads, int d, int seqlen_q,
                     int max_seqlen_k, int num_splits, int *pieces, int *min_piece);

/*
 * Bytes of workspace attn_decode_ex(..., num_splits) needs for this shape
 * (attn_decode uses num_splits = 0):
 *   n_kv_heads * (pieces + batch) * C * (d + 2) * 4 + (batch + 1) * 8,
 * or 0 when pieces == 1, with C = 16 packed columns per partial when
 * (n_q_heads / n_kv_heads) * seqlen_q <= 16 and C = 32 otherwise. It holds
 * per-(piece, sequence) fp32 partial outputs, maxima and denominators for
 * the (at most) pieces + batch partials of each KV
 * head, then the key total and each sequence's flattened start. It needs no
 * initialisation (e.g. torch.empty): every value the combine step reads is
 * written by the same call ([GQA-SM100] §Removing the max reset).
 * Returns 0 for invalid arguments. Host-only.
 */
size_t attn_decode_workspace_size(int batch, int n_q_heads, int n_kv_heads, int seqlen_q, int d,
                                  int max_seqlen_k, int num_splits);

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
 *   Requires d in {64, 128, 256}; (n_q_heads / n_kv_heads) * seqlen_q <= 32
 *   at d = 64 and 128 (the packed query rows of one KV head: one MFMA column
 *   group of 16, or two that share every K and V read) and <= 16 at d = 256
 *   (one group: a wave streams its keys through a single register slot
 *   there); batch <= ATTN_MAX_BATCH (else ATTN_ERR_UNSUPPORTED).
 *   workspace / workspace_bytes: caller scratch of at least
 *   attn_decode_workspace_size(...) bytes; workspace == NULL selects the
 *   grouped work split below for every shape (slow for few long sequences,
 *   but needs no scratch).
 *
 * Device work, chosen from the host integers alone:
 *   - split (the general case): one split kernel (one work-group of four
 *     independent waves per CU, each wave streaming one balanced piece of one
 *     KV head), then one combine kernel over (sequence, KV head) that merges
 *     the pieces of every sequence spread over several;
 *   - grouped (calls whose whole cache holds at most 256 KB of K/V at
 *     capacity, or 128 to 512 sequence-head pairs of at most 512 KB each, or no
 *     workspace): one kernel, one work-group per (sequence, KV head) whose four
 *     waves share the sequence's keys and merge through LDS; the workspace is
 *     not touched.
 * Both use fp32 arithmetic on partials in a fixed order with no atomics:
 * results are deterministic and bitwise reproducible.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *seqlens_k, void *o, float *lse, int n_q_heads,
                int n_kv_heads, int d, int seqlen_q, int batch, int max_seqlen_k,
                void *workspace, size_t workspace_bytes, void *stream);

/* attn_decode with an explicit number of pieces per KV head (0 = automatic;
 * see attn_decode_plan). */
int attn_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *seqlens_k, void *o, float *lse, int n_q_heads,
                   int n_kv_heads, int d, int seqlen_q, int batch, int max_seqlen_k,
                   void *workspace, size_t workspace_bytes, void *stream,
                   int num_splits);

/* attn_decode_ex for IEEE fp16 q, k_cache, v_cache and o (same layouts, plan,
 * workspace and errors). */
int attn_decode_f16(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *seqlens_k, void *o, float *lse, int n_q_heads,
                    int n_kv_heads, int d, int seqlen_q, int batch, int max_seqlen_k,
                    void *workspace, size_t workspace_bytes, void *stream,
                    int num_splits);

/* Bytes of the fixed device scratch attn_decode_noalloc works in (32 MiB). */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * attn_decode_ex for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, layouts, plan and results as attn_decode_ex (bf16), without
 * the workspace: the partials live in a fixed library array of
 * ATTN_NOALLOC_SCRATCH_BYTES on each device, created when the library's code
 * is loaded on that device and held until the process ends. The call
 * allocates, frees and memsets nothing; the first call on a device looks up
 * that device's copy of the array (a symbol lookup, not an allocation).
 * A call whose plan needs more than the fixed size
 * (attn_decode_workspace_size(...) > ATTN_NOALLOC_SCRATCH_BYTES, e.g. more
 * than about 700 sequences with 8 KV heads at d = 128) returns
 * ATTN_ERR_TOO_LARGE before enqueuing anything. Every call on one device
 * shares its array, and nothing in it needs clearing (each call writes every
 * value it later reads): calls whose execution overlaps on one device - on
 * different streams, or from different host threads without ordering - race
 * on it and give wrong results; calls ordered on one stream are safe.
 */
int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *seqlens_k, void *o, float *lse, int n_q_heads,
                        int n_kv_heads, int d, int seqlen_q, int batch, int max_seqlen_k,
                        void *stream, int num_splits);

/*
 * Prefill forward ([FA4-edges] §Edge 1 · causal masking, §Edge 3 · tile
 * scheduling): q [batch][seqlen_q][n_q_heads][d], k and v
 * [batch][seqlen_k][n_kv_heads][d], all bf16; o like q; lse
 * [batch][n_q_heads][seqlen_q] fp32 (may be NULL). causal != 0 applies the
 * bottom-right mask (query i sees keys j <= i + seqlen_k - seqlen_q).
 * Requires d == 64, 128 or 256 (else ATTN_ERR_UNSUPPORTED). Work-groups of
 * eight waves own 256 query rows and take them heaviest first (longest visible
 * key range first): at d = 128 one persistent work-group per compute unit
 * walks the tile list in rounds (the CU count is read from the current device;
 * ATTN_ERR_LAUNCH if it cannot be), at d = 64 and 256 one work-group is
 * launched per tile. The tile order does not
 * change the result: each row's output is computed by one wave in a fixed
 * order.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
             int batch, int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads, int d,
             void *stream);

/* attn_fwd for IEEE fp16 q, k, v and o (same layouts and errors). */
int attn_fwd_f16(const void *q, const void *k, const void *v, void *o, float *lse, int causal,
                 int batch, int seqlen_q, int seqlen_k, int n_q_heads, int n_kv_heads, int d,
                 void *stream);

/*
 * Prefill forward over a packed variable-length batch (the backward page
 * sweeps variable-length shapes, [FA4-bwd] §Results): sequence b owns query
 * rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q and o and key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]) of k and v, and is an independent
 * attention problem (bottom-right causal within it when causal != 0).
 *   q, o   [total_q][n_q_heads][d] bf16, sequences back to back
 *   k, v   [total_k][n_kv_heads][d] bf16 (may be NULL when total_k == 0)
 *   lse    [n_q_heads][total_q] fp32 natural-log LSE, or NULL
 *   cu_seqlens_q, cu_seqlens_k  int32[batch + 1] on the device, non-decreasing,
 *          starting at 0; offsets are clamped to [0, total] on the device, so
 *          inconsistent values cannot address outside the buffers.
 *   max_seqlen_q  at least the longest query length: it sizes the grid, and
 *          query rows past it are not computed.
 * A sequence with no keys gets O = 0 and LSE = -inf. Requires d == 64, 128
 * or 256 and total_q >= 1. Same tile code as attn_fwd, always one
 * work-group per (256-row query tile, sequence, query head), longest tile
 * index first; a work-group past its sequence's last tile exits at once (a
 * static persistent assignment would not see the lengths, which live on the
 * device).
 */
int attn_fwd_varlen(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                    const int32_t *cu_seqlens_k, void *o, float *lse, int causal, int batch,
                    int max_seqlen_q, int total_q, int total_k, int n_q_heads, int n_kv_heads, int d,
                    void *stream);

/* attn_fwd_varlen for IEEE fp16 q, k, v and o (same layouts and errors). */
int attn_fwd_varlen_f16(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                        const int32_t *cu_seqlens_k, void *o, float *lse, int causal, int batch,
                        int max_seqlen_q, int total_q, int total_k, int n_q_heads, int n_kv_heads,
                        int d, void *stream);

/*
 * Bytes of workspace attn_bwd needs: 2 * batch * n_q_heads * Sq_pad * 4 with
 * Sq_pad = seqlen_q rounded up to a multiple of 128 (a base-2 LSE and the
 * negated row sum D per query row). No initialisation is needed. Returns 0 for invalid
 * arguments. Host-only.
 */
size_t attn_bwd_workspace_size(int batch, int n_q_heads, int seqlen_q);

/*
 * Attention backward ([FA4-bwd] §Recap on the FA4 backward pass): with
 * s = 1/sqrt(d), L = lse and D = rowsum(dO o O) (the row sum of P o dP),
 *   P = exp(s Q K^T - L), dP = dO V^T, dS = P o (dP - D),
 *   dV = P^T dO, dK = s dS^T Q, dQ = s dS K.
 *   q, o, dout, dq  [batch][seqlen_q][n_q_heads][d] bf16
 *   k, v, dk, dv    [batch][seqlen_k][n_kv_heads][d] bf16
 *   lse             [batch][n_q_heads][seqlen_q] fp32, the forward's natural-log
 *                   LSE (-inf for a row that sees no key); required.
 * dq, dk and dv are overwritten (written exactly once each, no accumulation
 * into the caller's memory). GQA: dk and dv of a KV head sum the G query
 * heads that read it. causal != 0 applies the forward's bottom-right mask.
 * Requires d == 64 or d == 128 and a workspace of attn_bwd_workspace_size()
 * bytes (16-byte aligned). Device work: one row-statistics kernel, then a
 * kernel per 128-key tile of each (batch, KV head) for dK and dV and a kernel
 * per 128-row query tile of each (batch, query head) for dQ. No atomics: the
 * results are deterministic and bitwise reproducible.
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dout, void *dq, void *dk, void *dv, int causal, int batch, int seqlen_q,
             int seqlen_k, int n_q_heads, int n_kv_heads, int d, void *workspace,
             size_t workspace_bytes, void *stream);

/* attn_bwd for IEEE fp16 q, k, v, o, dout, dq, dk and dv (same layouts, workspace and errors). */
int attn_bwd_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, int causal, int batch, int seqlen_q,
                 int seqlen_k, int n_q_heads, int n_kv_heads, int d, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace attn_bwd_varlen needs: 2 * n_q_heads * pad * 4 with
 * pad = total_q + 128 rounded up to a multiple of 128. Returns 0 for invalid
 * arguments. Host-only.
 */
size_t attn_bwd_varlen_workspace_size(int n_q_heads, int total_q);

/*
 * attn_bwd over a packed variable-length batch (the layouts, offsets and
 * clamping of attn_fwd_varlen): q, o, dout, dq [total_q][n_q_heads][d];
 * k, v, dk, dv [total_k][n_kv_heads][d]; lse [n_q_heads][total_q], the
 * forward's. max_seqlen_q and max_seqlen_k are at least the longest query
 * and key lengths (they size the grids). Each sequence is an independent
 * problem; dq, dk and dv are written exactly once per row of a sequence.
 * Requires total_q >= 1, total_k >= 1 and a workspace of
 * attn_bwd_varlen_workspace_size() bytes.
 */
int attn_bwd_varlen(const void *q, const void *k, const void *v, const void *o, const float *lse,
                    const void *dout, void *dq, void *dk, void *dv, const int32_t *cu_seqlens_q,
                    const int32_t *cu_seqlens_k, int causal, int batch, int max_seqlen_q,
                    int max_seqlen_k, int total_q, int total_k, int n_q_heads, int n_kv_heads, int d,
                    void *workspace, size_t workspace_bytes, void *stream);

/* attn_bwd_varlen for IEEE fp16 tensors (same layouts, workspace and errors). */
int attn_bwd_varlen_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dout, void *dq, void *dk, void *dv, const int32_t *cu_seqlens_q,
                        const int32_t *cu_seqlens_k, int causal, int batch, int max_seqlen_q,
                        int max_seqlen_k, int total_q, int total_k, int n_q_heads, int n_kv_heads,
                        int d, void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code; never NULL. */
const char *attn_status_string(int status);

/* Library version string, e.g. "attn-mi355x 0.1.0 gfx950". */
const char *attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */

/*
 * A plain C caller of the attention library: no Python and no framework in
 * the process, only the HIP runtime and include/attn.h. The GPU test
 * test_capi_gpu.py feeds it seeded inputs and checks what it writes against
 * the CPU oracle.
 *
 * usage: attn_capi_check IN OUT
 *
 * IN holds one call: eight little-endian int32, then the arrays.
 *   decode:  {1, batch, seqlen_q, n_q_heads, n_kv_heads, d, max_seqlen_k, 0},
 *            q [batch][seqlen_q][n_q_heads][d] bf16, k and v
 *            [batch][max_seqlen_k][n_kv_heads][d] bf16, seqlens_k [batch] int32
 *   prefill: {2, batch, seqlen_q, seqlen_k, n_q_heads, n_kv_heads, d, causal},
 *            q [batch][seqlen_q][n_q_heads][d], k and v
 *            [batch][seqlen_k][n_kv_heads][d], all bf16
 * OUT receives O (bf16, the layout of q) then LSE (fp32,
 * [batch][n_q_heads][seqlen_q]). The exit status is 0 only when every HIP
 * call and the library call succeeded.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "attn.h"

#define HIP_OK(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                     \
      return 1;                                                                       \
    }                                                                                 \
  } while (0)

/* Read `bytes` from f into a new device buffer. */
static int upload(FILE *f, size_t bytes, void **dev) {
  void *host = malloc(bytes ? bytes : 1);
  if (host == NULL || fread(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "input file too short\n");
    free(host);
    return 1;
  }
  if (hipMalloc(dev, bytes ? bytes : 1) != hipSuccess || hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "device upload failed\n");
    free(host);
    return 1;
  }
  free(host);
  return 0;
}

/* Append `bytes` of device memory to f. */
static int download(FILE *f, const void *dev, size_t bytes) {
  void *host = malloc(bytes ? bytes : 1);
  int bad = host == NULL || hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess ||
            fwrite(host, 1, bytes, f) != bytes;
  free(host);
  if (bad) fprintf(stderr, "device download failed\n");
  return bad;
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE *in = fopen(argv[1], "rb");
  int32_t h[8];
  if (in == NULL || fread(h, sizeof(int32_t), 8, in) != 8) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 2;
  }
  HIP_OK(hipSetDevice(0));
  void *q = NULL, *k = NULL, *v = NULL, *o = NULL, *ws = NULL;
  int32_t *seqlens = NULL;
  float *lse = NULL;
  size_t q_elems, lse_elems;
  int status;
  if (h[0] == 1) {
    const int B = h[1], sq = h[2], Hq = h[3], Hkv = h[4], d = h[5], S = h[6];
    q_elems = (size_t)B * sq * Hq * d;
    const size_t kv_elems = (size_t)B * S * Hkv * d;
    lse_elems = (size_t)B * Hq * sq;
    if (upload(in, q_elems * 2, &q) || upload(in, kv_elems * 2, &k) || upload(in, kv_elems * 2, &v) ||
        upload(in, (size_t)B * 4, (void **)&seqlens))
      return 1;
    const size_t ws_bytes = attn_decode_workspace_size(B, Hq, Hkv, sq, d, S, 0);
    HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 16));
    HIP_OK(hipMalloc(&o, q_elems * 2));
    HIP_OK(hipMalloc((void **)&lse, lse_elems * 4));
    status = attn_decode(q, k, v, seqlens, o, lse, Hq, Hkv, d, sq, B, S, ws, ws_bytes, NULL);
  } else if (h[0] == 2) {
    const int B = h[1], Sq = h[2], Sk = h[3], Hq = h[4], Hkv = h[5], d = h[6], causal = h[7];
    q_elems = (size_t)B * Sq * Hq * d;
    const size_t kv_elems = (size_t)B * Sk * Hkv * d;
    lse_elems = (size_t)B * Hq * Sq;
    if (upload(in, q_elems * 2, &q) || upload(in, kv_elems * 2, &k) || upload(in, kv_elems * 2, &v)) return 1;
    HIP_OK(hipMalloc(&o, q_elems * 2));
    HIP_OK(hipMalloc((void **)&lse, lse_elems * 4));
    status = attn_fwd(q, k, v, o, lse, causal, B, Sq, Sk, Hq, Hkv, d, NULL);
  } else {
    fprintf(stderr, "unknown call kind %d\n", (int)h[0]);
    return 2;
  }
  fclose(in);
  if (status != 0) {
    fprintf(stderr, "library call failed: %s (%d)\n", attn_status_string(status), status);
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  FILE *out = fopen(argv[2], "wb");
  if (out == NULL || download(out, o, q_elems * 2) || download(out, lse, lse_elems * 4)) return 1;
  fclose(out);
  void *bufs[] = {q, k, v, o, lse, ws, seqlens};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) (void)hipFree(bufs[i]);
  printf("ok %s\n", attn_version());
  return 0;
}

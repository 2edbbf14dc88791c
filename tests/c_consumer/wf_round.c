/*
 * A plain C program that runs one chunk-wise causal attention round through
 * the C ABI of libwf (include/wf.h), with device memory from the HIP runtime
 * and no other dependency: the ABI carries only pointers, sizes and ints.
 *
 *   wf_round <in.bin> <out.bin>
 *
 * in.bin:  int32 C, H, D, n_hist, n_inflight, dtype (WF_F32 or WF_BF16), then
 *          float32 scale, then q [n_inflight*C][H][D], k_hist and v_hist
 *          [n_hist*C][H][D], k_in and v_in [n_inflight*C][H][D] in the dtype
 *          (bf16 as uint16 bit patterns).
 * out.bin: O of wf_chunk_causal_attn_fwd [n_inflight*C][H][D] in the dtype,
 *          then its LSE float32 [H][n_inflight*C]; for bf16 also O and LSE of
 *          wf_chunk_causal_attn_fwd_ws (with the key-split workspace).
 *
 * The cache holds the history chunks and then the in-flight chunks, appended
 * in order (refresh chunk first). Exit status 0 on success; on any error the
 * failing call and wf_last_error() go to stderr and the status is 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "wf.h"

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

#define WF_OK_OR_FAIL(call)                                                       \
  do {                                                                            \
    int s_ = (call);                                                              \
    if (s_ != WF_OK) {                                                            \
      fprintf(stderr, "%s returned %d: %s\n", #call, s_, wf_last_error());        \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

static void* read_all(const char* path, size_t* size) {
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  fseek(f, 0, SEEK_END);
  long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  void* buf = n > 0 ? malloc((size_t)n) : NULL;
  if (buf && fread(buf, 1, (size_t)n, f) != (size_t)n) {
    free(buf);
    buf = NULL;
  }
  fclose(f);
  *size = buf ? (size_t)n : 0;
  return buf;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <in.bin> <out.bin>\n", argv[0]);
    return 1;
  }
  size_t in_size = 0;
  char* in = (char*)read_all(argv[1], &in_size);
  if (!in || in_size < 6 * sizeof(int) + sizeof(float)) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  int hdr[6];
  float scale;
  memcpy(hdr, in, sizeof(hdr));
  memcpy(&scale, in + sizeof(hdr), sizeof(float));
  const int C = hdr[0], H = hdr[1], D = hdr[2], n_hist = hdr[3], N = hdr[4], dtype = hdr[5];
  const size_t esize = dtype == WF_F32 ? 4 : 2;
  const size_t chunk_bytes = (size_t)C * H * D * esize;
  const size_t q_bytes = (size_t)N * chunk_bytes;
  const size_t need = sizeof(hdr) + sizeof(float) + q_bytes + 2 * (size_t)n_hist * chunk_bytes + 2 * q_bytes;
  if ((dtype != WF_F32 && dtype != WF_BF16) || in_size != need) {
    fprintf(stderr, "%s: %zu bytes, expected %zu for the header's shape\n", argv[1], in_size, need);
    return 1;
  }
  const char* src_q = in + sizeof(hdr) + sizeof(float);
  const char* src_kh = src_q + q_bytes;
  const char* src_vh = src_kh + (size_t)n_hist * chunk_bytes;
  const char* src_ki = src_vh + (size_t)n_hist * chunk_bytes;
  const char* src_vi = src_ki + q_bytes;

  const int n_slots = n_hist + N;
  const size_t pool = wf_kv_pool_bytes(n_slots, C, H, D, dtype);
  if (pool == 0) {
    fprintf(stderr, "wf_kv_pool_bytes rejected the shape\n");
    return 1;
  }
  void *k_pool, *v_pool, *q, *kh, *vh, *ki, *vi, *out, *ws = NULL;
  float* lse;
  HIP_OK(hipMalloc(&k_pool, pool));
  HIP_OK(hipMalloc(&v_pool, pool));
  HIP_OK(hipMalloc(&q, q_bytes));
  HIP_OK(hipMalloc(&kh, n_hist ? (size_t)n_hist * chunk_bytes : 16));
  HIP_OK(hipMalloc(&vh, n_hist ? (size_t)n_hist * chunk_bytes : 16));
  HIP_OK(hipMalloc(&ki, q_bytes));
  HIP_OK(hipMalloc(&vi, q_bytes));
  HIP_OK(hipMalloc(&out, q_bytes));
  HIP_OK(hipMalloc((void**)&lse, (size_t)H * N * C * sizeof(float)));
  HIP_OK(hipMemcpy(q, src_q, q_bytes, hipMemcpyHostToDevice));
  if (n_hist) {
    HIP_OK(hipMemcpy(kh, src_kh, (size_t)n_hist * chunk_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(vh, src_vh, (size_t)n_hist * chunk_bytes, hipMemcpyHostToDevice));
  }
  HIP_OK(hipMemcpy(ki, src_ki, q_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(vi, src_vi, q_bytes, hipMemcpyHostToDevice));

  wf_kv_cache* cache = NULL;
  WF_OK_OR_FAIL(wf_kv_cache_create(&cache, k_pool, v_pool, n_slots, C, H, D, dtype, WF_KV_ZERO_FILL, NULL));
  for (int c = 0; c < n_hist; ++c)
    WF_OK_OR_FAIL(wf_kv_append(cache, (char*)kh + c * chunk_bytes, (char*)vh + c * chunk_bytes, NULL, NULL));
  for (int c = 0; c < N; ++c)
    WF_OK_OR_FAIL(wf_kv_append(cache, (char*)ki + c * chunk_bytes, (char*)vi + c * chunk_bytes, NULL, NULL));

  const size_t lse_bytes = (size_t)H * N * C * sizeof(float);
  const int runs = dtype == WF_BF16 ? 2 : 1;
  char* host = (char*)malloc(runs * (q_bytes + lse_bytes));
  if (!host) return 1;
  for (int run = 0; run < runs; ++run) {
    HIP_OK(hipMemset(out, 0xff, q_bytes));  /* every output element is written by the call */
    HIP_OK(hipMemset(lse, 0xff, lse_bytes));
    if (run == 0) {
      WF_OK_OR_FAIL(wf_chunk_causal_attn_fwd(q, cache, N, scale, out, lse, NULL));
    } else {
      const size_t ws_bytes = wf_attn_fwd_workspace_bytes(cache);
      HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 256));
      WF_OK_OR_FAIL(wf_chunk_causal_attn_fwd_ws(q, cache, N, scale, ws, out, lse, NULL));
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(host + run * (q_bytes + lse_bytes), out, q_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(host + run * (q_bytes + lse_bytes) + q_bytes, lse, lse_bytes, hipMemcpyDeviceToHost));
  }
  WF_OK_OR_FAIL(wf_kv_cache_destroy(cache));

  FILE* f = fopen(argv[2], "wb");
  if (!f || fwrite(host, 1, runs * (q_bytes + lse_bytes), f) != runs * (q_bytes + lse_bytes)) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(f);
  free(host);
  free(in);
  void* bufs[] = {k_pool, v_pool, q, kh, vh, ki, vi, out, lse, ws};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i)
    if (bufs[i]) HIP_OK(hipFree(bufs[i]));
  printf("wf_round: %d run(s) of a %d-chunk round (%d history), C %d, H %d, D %d\n", runs, N, n_hist, C, H, D);
  return 0;
}

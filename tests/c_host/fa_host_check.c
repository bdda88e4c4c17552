/*
 * A plain C host program that drives libfa.so through include/fa.h alone:
 * no Python, no PyTorch. Test infrastructure (tests/test_c_host.py runs it):
 *
 *   fa_host_check IN OUT
 *
 * IN holds six int32 (B, H, Hkv, N, d, causal), one float32 (scale), then
 * Q [B,H,N,d], K and V [B,Hkv,N,d] as raw bf16 bit patterns. The program
 * copies them to device memory it allocates itself, checks that a call with
 * an unsupported head size is refused before any work is enqueued, runs
 * fa_forward_gqa on a stream it creates, and writes O (bf16 bits) and lse
 * (float32) to OUT. Exit status 0 on success; otherwise a message on stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "fa.h"

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      return 2;                                                                \
    }                                                                          \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t hdr[6];
  float scale;
  if (!read_all(in, hdr, sizeof hdr) || !read_all(in, &scale, sizeof scale)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int B = hdr[0], H = hdr[1], Hkv = hdr[2], N = hdr[3], d = hdr[4], causal = hdr[5];
  const size_t nq = (size_t)B * H * N * d, nkv = (size_t)B * Hkv * N * d, nl = (size_t)B * H * N;
  uint16_t* hq = malloc(nq * 2);
  uint16_t* hk = malloc(nkv * 2);
  uint16_t* hv = malloc(nkv * 2);
  uint16_t* ho = malloc(nq * 2);
  float* hl = malloc(nl * 4);
  if (!hq || !hk || !hv || !ho || !hl) {
    fprintf(stderr, "host allocation failed\n");
    return 1;
  }
  if (!read_all(in, hq, nq * 2) || !read_all(in, hk, nkv * 2) || !read_all(in, hv, nkv * 2)) {
    fprintf(stderr, "short tensor data\n");
    return 1;
  }
  fclose(in);

  void *q, *k, *v, *o;
  float* lse;
  HIP_OK(hipMalloc(&q, nq * 2));
  HIP_OK(hipMalloc(&k, nkv * 2));
  HIP_OK(hipMalloc(&v, nkv * 2));
  HIP_OK(hipMalloc(&o, nq * 2));
  HIP_OK(hipMalloc((void**)&lse, nl * 4));
  HIP_OK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, nkv * 2, hipMemcpyHostToDevice));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  /* a head size the library does not support is refused before any launch */
  const int bad = fa_forward_gqa(q, k, v, o, lse, B, H, Hkv, N, 96, causal, scale, stream);
  if (bad == FA_OK) {
    fprintf(stderr, "d = 96 was accepted\n");
    return 3;
  }

  const int rc = fa_forward_gqa(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, stream);
  if (rc != FA_OK) {
    fprintf(stderr, "fa_forward_gqa: %s\n", fa_status_string(rc));
    return 3;
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(ho, o, nq * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl, lse, nl * 4, hipMemcpyDeviceToHost));

  FILE* out = fopen(argv[2], "wb");
  if (!out || fwrite(ho, 2, nq, out) != nq || fwrite(hl, 4, nl, out) != nl) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(out);
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(o));
  HIP_OK(hipFree(lse));
  free(hq);
  free(hk);
  free(hv);
  free(ho);
  free(hl);
  return 0;
}

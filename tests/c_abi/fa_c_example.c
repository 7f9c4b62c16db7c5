/*
 * A plain C consumer of the library: it uses include/fa.h and the HIP runtime
 * only (no Python, no torch). Two calls of the C ABI on a stream of its own:
 *
 *   prefill:  fa_fwd over bf16 Q, K, V [B, N, H, D] (causal), O in fp32
 *   decode:   fa_fwd_splitkv over a paged bf16 cache, then fa_splitkv_combine
 *
 * Inputs are raw little-endian files (bf16 bit patterns, int32 block table);
 * outputs are raw fp32 files. The device memory is the program's own: the
 * library allocates nothing. Usage:
 *
 *   fa_c_example prefill B H N D q.bin k.bin v.bin o.bin lse.bin
 *   fa_c_example decode  B H Nk D page_size num_pages max_pages splits
 *                        q.bin kc.bin vc.bin table.bin o.bin lse.bin
 *
 * Exit status 0 on success; every library or HIP error is printed with its
 * status text and ends the program with status 1.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

static void die(const char* what, const char* detail) {
  fprintf(stderr, "fa_c_example: %s: %s\n", what, detail);
  exit(1);
}

static void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

static void fa_check(int status, const char* what) {
  if (status != FA_OK) die(what, fa_status_string(status));
}

static void* read_file(const char* path, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) die("cannot open", path);
  void* p = malloc(bytes ? bytes : 1);
  if (!p) die("out of host memory", path);
  if (fread(p, 1, bytes, f) != bytes) die("short read", path);
  fclose(f);
  return p;
}

static void write_file(const char* path, const void* p, size_t bytes) {
  FILE* f = fopen(path, "wb");
  if (!f) die("cannot create", path);
  if (fwrite(p, 1, bytes, f) != bytes) die("short write", path);
  fclose(f);
}

/* Copy a host file to new device memory. */
static void* to_device(const char* path, size_t bytes) {
  void* h = read_file(path, bytes);
  void* d = NULL;
  hip_check(hipMalloc(&d, bytes), "hipMalloc");
  hip_check(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
  free(h);
  return d;
}

static void from_device(const char* path, const void* d, size_t bytes) {
  void* h = malloc(bytes);
  if (!h) die("out of host memory", path);
  hip_check(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
  write_file(path, h, bytes);
  free(h);
}

int main(int argc, char** argv) {
  if (argc < 2) die("usage", "fa_c_example prefill|decode ...");
  hipStream_t stream;
  hip_check(hipStreamCreate(&stream), "hipStreamCreate");

  /* A bad argument is reported before any device work. */
  if (fa_fwd(NULL, NULL, NULL, FA_BF16, NULL, FA_FP32, NULL, 1, 1, 1, 1, 128, 0.1f, 1, -1, -1,
             NULL, 0.0f, stream) != FA_ERR_NULL)
    die("fa_fwd", "NULL pointers were not rejected");

  if (strcmp(argv[1], "prefill") == 0 && argc == 11) {
    const int B = atoi(argv[2]), H = atoi(argv[3]), N = atoi(argv[4]), D = atoi(argv[5]);
    const size_t elems = (size_t)B * N * H * D;
    void* q = to_device(argv[6], elems * 2);
    void* k = to_device(argv[7], elems * 2);
    void* v = to_device(argv[8], elems * 2);
    void *o = NULL, *lse = NULL;
    hip_check(hipMalloc(&o, elems * 4), "hipMalloc");
    hip_check(hipMalloc(&lse, (size_t)B * H * N * 4), "hipMalloc");
    fa_check(fa_fwd(q, k, v, FA_BF16, o, FA_FP32, (float*)lse, B, H, N, N, D,
                    1.0f / sqrtf((float)D), 1, -1, -1, NULL, 0.0f, stream),
             "fa_fwd");
    hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");
    from_device(argv[9], o, elems * 4);
    from_device(argv[10], lse, (size_t)B * H * N * 4);
    hipFree(q); hipFree(k); hipFree(v); hipFree(o); hipFree(lse);
  } else if (strcmp(argv[1], "decode") == 0 && argc == 16) {
    const int B = atoi(argv[2]), H = atoi(argv[3]), Nk = atoi(argv[4]), D = atoi(argv[5]);
    const int ps = atoi(argv[6]), pages = atoi(argv[7]), max_pages = atoi(argv[8]);
    const int S = atoi(argv[9]);
    const size_t pool = (size_t)pages * ps * H * D;
    void* q = to_device(argv[10], (size_t)B * H * D * 2);
    void* kc = to_device(argv[11], pool * 2);
    void* vc = to_device(argv[12], pool * 2);
    void* table = to_device(argv[13], (size_t)B * max_pages * 4);
    void *op = NULL, *lp = NULL, *o = NULL, *lse = NULL;
    hip_check(hipMalloc(&op, (size_t)S * B * H * D * 4), "hipMalloc");
    hip_check(hipMalloc(&lp, (size_t)S * B * H * 4), "hipMalloc");
    hip_check(hipMalloc(&o, (size_t)B * H * D * 4), "hipMalloc");
    hip_check(hipMalloc(&lse, (size_t)B * H * 4), "hipMalloc");
    fa_check(fa_fwd_splitkv(q, kc, vc, FA_BF16, (const int*)table, max_pages, ps, (float*)op,
                            (float*)lp, S, B, H, 1, Nk, D, 1.0f / sqrtf((float)D), 1, -1, -1,
                            NULL, 0.0f, stream),
             "fa_fwd_splitkv");
    fa_check(fa_splitkv_combine((const float*)op, (const float*)lp, S, B, H, 1, D, o, FA_FP32,
                                (float*)lse, stream),
             "fa_splitkv_combine");
    hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");
    from_device(argv[14], o, (size_t)B * H * D * 4);
    from_device(argv[15], lse, (size_t)B * H * 4);
    hipFree(q); hipFree(kc); hipFree(vc); hipFree(table);
    hipFree(op); hipFree(lp); hipFree(o); hipFree(lse);
  } else {
    die("usage", "see the comment at the top of fa_c_example.c");
  }
  hip_check(hipStreamDestroy(stream), "hipStreamDestroy");
  return 0;
}

/*
 * One decode through the C ABI alone (no Python): reads q, kv and the
 * lengths from raw files, runs gqa_decode (include/gqa_decode.h) on device 0
 * with HIP runtime calls only, and writes out. Before it, the same decode
 * runs through the allocation-free entry point (gqa_decode_ex_noalloc, while
 * the library has allocated nothing in this process); its output must match
 * gqa_decode's byte for byte.
 *
 *   decode_from_c Q_FILE KV_FILE LENS_FILE OUT_FILE batch capacity q_scale
 *       q: fp16 [batch, 32, 128]; kv: fp16 [batch, 2, 8, capacity, 128];
 *       lens: int32 [batch]; out: fp16 [batch, 32, 128] (written).
 *   decode_from_c --bad-shape
 *       calls gqa_decode with batch 0 and prints the status it reports
 *       (needs no device: argument errors come before any device work).
 *
 * Exit status: 0 success, 1 a gqa_decode error (status and message on
 * stderr), 2 usage or file errors, 3 a HIP runtime error, 4 the two entry
 * points' outputs differ.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gqa_decode.h"

static int read_file(const char* path, void* buf, size_t n) {
  FILE* f = fopen(path, "rb");
  if (!f) return -1;
  const size_t got = fread(buf, 1, n, f);
  fclose(f);
  return got == n ? 0 : -1;
}

static int write_file(const char* path, const void* buf, size_t n) {
  FILE* f = fopen(path, "wb");
  if (!f) return -1;
  const size_t put = fwrite(buf, 1, n, f);
  return fclose(f) == 0 && put == n ? 0 : -1;
}

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));              \
      return 3;                                                               \
    }                                                                         \
  } while (0)

int main(int argc, char** argv) {
  if (argc == 2 && argv[1][0] == '-') {
    const int st = gqa_decode((void*)16, (void*)16, (const int32_t*)16, (void*)4096, 1.0f, 0,
                              64, NULL);
    printf("status %d: %s: %s\n", st, gqa_decode_status_string(st), gqa_decode_last_error());
    return st == GQA_ERR_BAD_SHAPE ? 0 : 1;
  }
  if (argc != 8) {
    fprintf(stderr, "usage: %s Q KV LENS OUT batch capacity q_scale\n", argv[0]);
    return 2;
  }
  const int batch = atoi(argv[5]), capacity = atoi(argv[6]);
  const float q_scale = strtof(argv[7], NULL);
  if (batch <= 0 || capacity <= 0) {
    fprintf(stderr, "batch and capacity must be positive\n");
    return 2;
  }
  const size_t q_bytes = (size_t)batch * GQA_NUM_Q_HEADS * GQA_HEAD_DIM * 2;
  const size_t kv_bytes = (size_t)batch * 2 * GQA_NUM_KV_HEADS * (size_t)capacity * GQA_HEAD_DIM * 2;
  const size_t lens_bytes = (size_t)batch * 4;
  void* hq = malloc(q_bytes);
  void* hkv = malloc(kv_bytes);
  void* hlens = malloc(lens_bytes);
  void* hout = malloc(q_bytes);
  void* hout2 = malloc(q_bytes);
  if (!hq || !hkv || !hlens || !hout || !hout2) return 2;
  if (read_file(argv[1], hq, q_bytes) || read_file(argv[2], hkv, kv_bytes) ||
      read_file(argv[3], hlens, lens_bytes)) {
    fprintf(stderr, "could not read the input files\n");
    return 2;
  }
  void *dq, *dkv, *dlens, *dout, *dout2;
  hipStream_t stream;
  HIP_OK(hipSetDevice(0));
  HIP_OK(hipMalloc(&dq, q_bytes));
  HIP_OK(hipMalloc(&dkv, kv_bytes));
  HIP_OK(hipMalloc(&dlens, lens_bytes));
  HIP_OK(hipMalloc(&dout, q_bytes));
  HIP_OK(hipMalloc(&dout2, q_bytes));
  HIP_OK(hipStreamCreate(&stream));
  HIP_OK(hipMemcpy(dq, hq, q_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dkv, hkv, kv_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, hlens, lens_bytes, hipMemcpyHostToDevice));
  int st = gqa_decode_ex_noalloc(dq, dkv, (const int32_t*)dlens, dout2, GQA_DTYPE_F16, NULL,
                                 q_scale, 1.0f, 1.0f, batch, capacity, 0, stream);
  if (st != GQA_OK) {
    fprintf(stderr, "gqa_decode_ex_noalloc: status %d (%s): %s\n", st,
            gqa_decode_status_string(st), gqa_decode_last_error());
    return 1;
  }
  st = gqa_decode(dq, dkv, (const int32_t*)dlens, dout, q_scale, batch, capacity, stream);
  if (st != GQA_OK) {
    fprintf(stderr, "gqa_decode: status %d (%s): %s\n", st, gqa_decode_status_string(st),
            gqa_decode_last_error());
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(hout, dout, q_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hout2, dout2, q_bytes, hipMemcpyDeviceToHost));
  gqa_decode_release_workspace();
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dkv));
  HIP_OK(hipFree(dlens));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dout2));
  if (write_file(argv[4], hout, q_bytes)) {
    fprintf(stderr, "could not write %s\n", argv[4]);
    return 2;
  }
  const int same = memcmp(hout, hout2, q_bytes) == 0;
  free(hq);
  free(hkv);
  free(hlens);
  free(hout);
  free(hout2);
  if (!same) {
    fprintf(stderr, "gqa_decode_ex_noalloc and gqa_decode wrote different bytes\n");
    return 4;
  }
  printf("gqa_decode_ex_noalloc output identical to gqa_decode\n");
  return 0;
}

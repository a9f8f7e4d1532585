/*
 * One decode through the C ABI alone (no Python): reads q, kv and the
 * lengths from raw files, runs gqa_decode (include/gqa_decode.h) on device 0
 * with HIP runtime calls only, and writes out.
 *
 *   decode_from_c Q_FILE KV_FILE LENS_FILE OUT_FILE batch capacity q_scale
 *       q: fp16 [batch, 32, 128]; kv: fp16 [batch, 2, 8, capacity, 128];
 *       lens: int32 [batch]; out: fp16 [batch, 32, 128] (written).
 *   decode_from_c --bad-shape
 *       calls gqa_decode with batch 0 and prints the status it reports
 *       (needs no device: argument errors come before any device work).
 *
 * Exit status: 0 success, 1 a gqa_decode error (status and message on
 * stderr), 2 usage or file errors, 3 a HIP runtime error.
 */
#include <stdio.h>
#include <stdlib.h>

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
  if (!hq || !hkv || !hlens || !hout) return 2;
  if (read_file(argv[1], hq, q_bytes) || read_file(argv[2], hkv, kv_bytes) ||
      read_file(argv[3], hlens, lens_bytes)) {
    fprintf(stderr, "could not read the input files\n");
    return 2;
  }
  void *dq, *dkv, *dlens, *dout;
  hipStream_t stream;
  HIP_OK(hipSetDevice(0));
  HIP_OK(hipMalloc(&dq, q_bytes));
  HIP_OK(hipMalloc(&dkv, kv_bytes));
  HIP_OK(hipMalloc(&dlens, lens_bytes));
  HIP_OK(hipMalloc(&dout, q_bytes));
  HIP_OK(hipStreamCreate(&stream));
  HIP_OK(hipMemcpy(dq, hq, q_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dkv, hkv, kv_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, hlens, lens_bytes, hipMemcpyHostToDevice));
  const int st = gqa_decode(dq, dkv, (const int32_t*)dlens, dout, q_scale, batch, capacity, stream);
  if (st != GQA_OK) {
    fprintf(stderr, "gqa_decode: status %d (%s): %s\n", st, gqa_decode_status_string(st),
            gqa_decode_last_error());
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(hout, dout, q_bytes, hipMemcpyDeviceToHost));
  gqa_decode_release_workspace();
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dkv));
  HIP_OK(hipFree(dlens));
  HIP_OK(hipFree(dout));
  if (write_file(argv[4], hout, q_bytes)) {
    fprintf(stderr, "could not write %s\n", argv[4]);
    return 2;
  }
  free(hq);
  free(hkv);
  free(hlens);
  free(hout);
  return 0;
}

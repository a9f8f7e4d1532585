// Drives the C ABI's argument checking under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; built with g++ against the
// C-ABI layer and kernels_stub.cpp). Every call must return its documented
// status; with no device visible a valid call returns GQA_ERR_NO_DEVICE.
// Prints one line per case and exits 0 when all match.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gqa_decode.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  printf("%-48s %4d %s\n", what, got, got == want ? "ok" : "MISMATCH");
  if (got != want) ++failures;
}

static gqa_layout contiguous(int C) {
  gqa_layout L;
  memset(&L, 0, sizeof(L));
  L.q_stride_batch = 32 * 128;
  L.q_stride_head = 128;
  L.kv_stride_row = 128;
  L.kv_stride_head = (int64_t)C * 128;
  L.kv_stride_kind = 8LL * C * 128;
  L.kv_stride_batch = 2 * L.kv_stride_kind;
  return L;
}

int main(void) {
  void* q = (void*)0x10000;
  void* kv = (void*)0x20000000;
  const int32_t* lens = (const int32_t*)0x30000;
  void* out = (void*)0x40000;
  const int nodev = GQA_ERR_NO_DEVICE;
  expect("null q", gqa_decode(NULL, kv, lens, out, 1.f, 2, 64, NULL), GQA_ERR_NULL);
  expect("batch 0", gqa_decode(q, kv, lens, out, 1.f, 0, 64, NULL), GQA_ERR_BAD_SHAPE);
  expect("capacity too large", gqa_decode(q, kv, lens, out, 1.f, 1, (1 << 22) + 1, NULL),
         GQA_ERR_BAD_SHAPE);
  expect("misaligned q", gqa_decode((char*)q + 2, kv, lens, out, 1.f, 2, 64, NULL),
         GQA_ERR_MISALIGNED);
  expect("out over q", gqa_decode(q, kv, lens, (char*)q + 256, 1.f, 2, 64, NULL), GQA_ERR_ALIAS);
  expect("negative chunk", gqa_decode_chunked(q, kv, lens, out, 1.f, 2, 64, -1, NULL),
         GQA_ERR_BAD_ARG);
  expect("unknown dtype", gqa_decode_typed(q, kv, lens, out, 7, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         GQA_ERR_BAD_ARG);
  expect("fp4 dtype via typed", gqa_decode_typed(q, kv, lens, out, GQA_DTYPE_FP4_KV, 1.f, 1.f,
                                                 1.f, 2, 64, 0, NULL), GQA_ERR_BAD_ARG);
  expect("valid call, no device", gqa_decode(q, kv, lens, out, 1.f, 2, 64, NULL), nodev);
  gqa_layout L = contiguous(64);
  expect("layout valid", gqa_decode_ex(q, kv, lens, out, 0, &L, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         nodev);
  L.kv_stride_row = 132;
  expect("kv rows not 16-byte aligned",
         gqa_decode_ex(q, kv, lens, out, 0, &L, 1.f, 1.f, 1.f, 2, 64, 0, NULL), GQA_ERR_BAD_ARG);
  L = contiguous(64);
  L.kv_stride_row = 1LL << 40;
  expect("huge stride", gqa_decode_ex(q, kv, lens, out, 0, &L, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         GQA_ERR_BAD_ARG);
  L = contiguous(64);
  L.num_q_heads = 72;
  L.num_kv_heads = 8;
  expect("9 heads per KV head", gqa_decode_ex(q, kv, lens, out, 0, &L, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         GQA_ERR_BAD_ARG);
  L = contiguous(64);
  L.num_q_heads = 1024;
  L.num_kv_heads = 1024;
  L.q_stride_batch = 1024 * 128;
  expect("batch x KV heads over 2^27",
         gqa_decode_ex(q, kv, lens, out, 0, &L, 1.f, 1.f, 1.f, 1 << 20, 64, 0, NULL),
         GQA_ERR_BAD_SHAPE);
  L = contiguous(64);
  L.block_table = (const int32_t*)0x50000;
  L.max_pages = 4;
  L.page_size = 24;
  L.num_pages = 9;
  expect("page size 24", gqa_decode_ex(q, kv, lens, out, 0, &L, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         GQA_ERR_BAD_ARG);
  L.page_size = 16;
  expect("paged valid", gqa_decode_ex(q, kv, lens, out, 0, &L, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         nodev);
  gqa_layout F;
  memset(&F, 0, sizeof(F));
  F.q_stride_batch = 32 * 128;
  F.q_stride_head = 128;
  F.kv_stride_row = 64;
  F.kv_stride_head = 64 * 64;
  F.kv_stride_kind = 8 * 64 * 64;
  F.kv_stride_batch = 2 * F.kv_stride_kind;
  gqa_block_scales S;
  memset(&S, 0, sizeof(S));
  S.scales = (const void*)0x60000;
  expect("fp4 valid", gqa_decode_fp4(q, kv, &S, lens, out, &F, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         nodev);
  expect("fp4 null scales", gqa_decode_fp4(q, kv, NULL, lens, out, &F, 1.f, 1.f, 1.f, 2, 64, 0, NULL),
         GQA_ERR_NULL);
  S.stride_row = 6;
  S.stride_head = 64 * 6;
  S.stride_kind = 8 * 64 * 6;
  S.stride_batch = 2 * S.stride_kind;
  expect("fp4 scale stride 6", gqa_decode_fp4(q, kv, &S, lens, out, &F, 1.f, 1.f, 1.f, 2, 64, 0,
                                              NULL), GQA_ERR_BAD_ARG);
  expect("launch form 3", gqa_decode_set_launch_form(3), GQA_ERR_BAD_ARG);
  expect("launch form auto", gqa_decode_set_launch_form(GQA_LAUNCH_AUTO), GQA_OK);
  expect("workspace bytes, no device", (int)gqa_decode_workspace_bytes(2, 64), 0);
  gqa_decode_release_workspace();
  for (int st = -12; st <= 0; ++st)
    if (!gqa_decode_status_string(st)) ++failures;
  printf("%d mismatches\n", failures);
  return failures ? 1 : 0;
}

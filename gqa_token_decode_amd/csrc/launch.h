// Internal interface between the C-ABI layer (gqa_decode_api.cpp) and the
// gfx950 kernels (gqa_decode_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace gqa {

// Element types: q, kv and out all fp16 or all bf16; or fp16 q and out with
// OCP FP8 E4M3 kv, or with block-scaled FP4 kv (E2M1 codes and E4M3 scales).
enum class ElemType { kF16, kBf16, kE4m3Kv, kFp4Kv };

// Addressing of q and kv, in bytes (see the kernel's Params). A non-null
// block_table selects the paged kernels: kv_sb is then the page stride, and
// pages hold 2^page_shift positions (page_shift >= 4).
struct Layout {
  long long q_sb, q_sh, kv_sb, kv_sk, kv_sh, kv_sr;
  const int32_t* block_table;
  int max_pages, page_shift, num_pages;
  int q_heads, kv_heads;   // q_heads a multiple of kv_heads, at most 8 times it
  // FP4 kv: the block scales (8 bytes per K or V row), addressed like kv
  // (kv_scales + b*sc_sb + kind*sc_sk + g*sc_sh + i*sc_sr; paged: page*sc_sb).
  const void* kv_scales;
  long long sc_sb, sc_sk, sc_sh, sc_sr;
};

// How the device-side planner cuts the valid rows into pieces.
struct SplitConfig {
  int pieces;         // automatic split: number of pieces (one workgroup each)
  int pieces_first;   // automatic split: the first pieces_first pieces are the longer ones
  int second_share;   // automatic split: length of the others, in 1/64ths of the first (64: equal)
  int min_piece;      // automatic split: lower bound on the piece length (rows)
  int forced_piece;   // > 0: fixed piece length; the grid then covers batch*capacity rows
  int seg_cost;       // automatic split: fixed cost units per (sequence, KV head) segment
  int row_align;      // 1, or 16 for paged caches (pieces and segments 16-row aligned)
  int combine_max_grid;   // combine kernel: workgroups at most (each takes segments in turns)
};

// Workgroups of the pieces kernel that fit on one CU at once (the fewest
// over its instantiations; 0 on error).
int resident_workgroups_per_cu();

// Number of workgroups launched for this shape and split (forced pieces must
// already be a multiple of cfg.row_align).
long long grid_for(int batch, int capacity, int kv_heads, const SplitConfig& cfg);

// Bytes of fp32 partial-result storage for a grid (two slots per workgroup,
// `group` query heads each).
size_t partial_bytes_for_grid(long long grid, int group);

// Bytes of per-segment descriptors for a batch (rounded to 256).
size_t segment_bytes_for_batch(int batch, int kv_heads);

// Fixed device scratch of the allocation-free entry point (one copy per
// device, held until the process ends): the single launch's tickets in the
// first kScratchTicketBytes (zero when the code object loads; every call
// leaves them zero), then the segment descriptors and partial results.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr size_t kScratchTicketBytes = (size_t)1 << 20;

// Device address of the scratch on device `dev`, which must be current
// (looked up once per device, then cached; the caller serialises calls).
hipError_t scratch_area(int dev, void** ptr);

// Enqueue the decode. `partials` must hold segment_bytes_for_batch(batch,
// kv_heads) + partial_bytes_for_grid(grid, group) bytes. With `tickets`
// (kv_heads * batch ints, zero before the call and left zero by it) one
// launch does everything: the last piece of each cut segment merges its
// partials. Without, two kernels run
// (pieces, then combine). `events` (may be null) points at four events:
// start and stop of the pieces kernel, then start and stop of the combine
// kernel (the last two are not recorded in the single-launch form).
hipError_t launch_decode(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                         ElemType elem, const Layout& layout, float score_scale_log2,
                         float out_scale, int batch, int capacity,
                         const SplitConfig& cfg, long long grid, void* partials, int* tickets,
                         hipStream_t stream, hipEvent_t* events);

}  // namespace gqa

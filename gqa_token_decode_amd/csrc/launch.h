// Internal interface between the C-ABI layer (gqa_decode_api.cpp) and the
// gfx950 kernels (gqa_decode_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace gqa {

// How the device-side planner splits the batch into work items.
struct SplitConfig {
  int target_items;   // automatic split: aim for about this many (b, kv head, chunk) items
  int min_chunk;      // automatic split: never cut chunks shorter than this many positions
  int forced_chunk;   // > 0: fixed cap on chunk length (automatic rules ignored)
};

// Upper bound on the number of work items the planner can produce for any
// seq_lens (each clamped to [0, capacity]). Returns -1 if it exceeds int.
long long max_work_items(int batch, int capacity, const SplitConfig& cfg);

// Bytes of fp32 workspace needed for `items` work items.
size_t workspace_bytes_for_items(long long items);

// Enqueue the split-KV partial kernel and the log-sum-exp combine kernel.
// `events` (may be null) points at three events recorded before the partial
// kernel, between the two kernels and after the combine kernel.
hipError_t launch_decode(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                         float score_scale_log2, int batch, int capacity,
                         const SplitConfig& cfg, long long grid_items, void* workspace,
                         hipStream_t stream, hipEvent_t* events);

}  // namespace gqa

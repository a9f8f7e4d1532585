// Split-KV FP16 GQA single-token decode for gfx950 (MI355X, CDNA4, wave64).
//
// Operation (FlashInfer PR #5052 analysis page, "SM110 FP16 GQA decode":
// section 1 docstring, section 2 specialisation, section 3 SDPA comparator):
// for batch entry b and query head h, with g = h / 4 and L = clamp(len, 0, C),
//   out[b,h] = softmax_i(scale * q[b,h] . K[b,g,i]) . V[b,g,i],  i < L.
//
// Two kernels on one stream:
//   1. split_partial: one 256-thread workgroup per work item (b, g, chunk).
//      The four query heads of KV head g share every K/V row the workgroup
//      loads, so each row of the cache crosses HBM exactly once. A sequence
//      with a single chunk writes its fp16 output directly; otherwise the
//      workgroup writes an fp32 partial (running max, softmax denominator,
//      unnormalised weighted sum of V) for each of its four heads.
//   2. split_combine: one workgroup per (b, h) merges the partials of a
//      multi-chunk sequence with a log-sum-exp rescale, and writes zeros
//      for empty sequences.
// Both kernels derive the same split from seq_lens on the device (the host
// never reads the lengths): chunk target T from the total valid length,
// n_b = ceil(L_b / T) near-equal chunks per sequence, items numbered
// b-major, then KV head, then chunk.
//
// Register layout inside the partial kernel (per wave of 64 lanes):
//   lane = 16 * r + j: row slot r in 0..3, column block j in 0..15.
//   One 16-byte load per lane moves 4 consecutive 256-byte rows (1 KiB,
//   fully coalesced); lane (r, j) holds elements 8j..8j+7 of row r.
//   q for the four heads is held the same way (8 fp16 per head per lane).
//   QK: 4 packed fp16 dot products (fp32 accumulate) per head, then a
//   16-lane DPP butterfly leaves the full score in every lane of the row.
//   Each row slot keeps its own online-softmax state (m, l) and its own
//   fp32 accumulators acc[head][8]; the 16 row states of the workgroup
//   (4 waves x 4 slots) are merged through LDS at the end.
// Rows at or beyond the chunk end are never loaded: their scores are set to
// -inf and their weights to 0 by selects, so no garbage or NaN stored beyond
// a sequence's length can reach the arithmetic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace gqa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kQHeads = 32;
constexpr int kKvHeads = 8;
constexpr int kGroup = kQHeads / kKvHeads;   // 4 query heads per KV head
constexpr int kDim = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowSlots = 4;                 // rows covered by one wave-wide 16-byte load
constexpr int kUnroll = 4;                   // K (and V) loads per lane per iteration
constexpr int kWaveRows = kRowSlots * kUnroll;    // 16 positions per wave per iteration
constexpr int kBlockRows = kWaves * kWaveRows;    // 64 positions per workgroup per iteration
constexpr int kStates = kWaves * kRowSlots;       // 16 softmax states per workgroup

struct PlanParams {
  const int32_t* seq_lens;
  int batch;
  int capacity;
  int target_items;
  int min_chunk;
  int forced_chunk;
};

__device__ __forceinline__ int clamp_len(int v, int cap) { return v < 0 ? 0 : (v > cap ? cap : v); }

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane receives the same value
// (each step adds a pair of equal operands in either order).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_f32<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_f32<0x141>(x);   // row_half_mirror: lane i <- 7 - i within 8
  x += dpp_f32<0x140>(x);   // row_mirror: lane i <- 15 - i within 16
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- planning
// Workgroup-wide helpers; every thread of the workgroup must call them.

__device__ long long block_sum_ll(long long v, long long* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  return t;
}

// Inclusive prefix sum over the workgroup's 256 threads; also returns the total.
__device__ int block_incl_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  __syncthreads();
  if (lane == 63) red[wv] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    before += (i < wv) ? red[i] : 0;
    all += red[i];
  }
  *total = all;
  return v + before;
}

// Chunk-length cap T for this call, from the total valid length.
__device__ int chunk_cap(const PlanParams& p, long long* red) {
  long long part = 0;
  for (int b = threadIdx.x; b < p.batch; b += kThreads) part += clamp_len(p.seq_lens[b], p.capacity);
  const long long total = block_sum_ll(part, red);
  if (p.forced_chunk > 0) return p.forced_chunk;
  long long t = (8 * total + p.target_items - 1) / p.target_items;
  if (t < p.min_chunk) t = p.min_chunk;
  if (t > p.capacity) t = p.capacity;
  return (int)(t < 1 ? 1 : t);
}

__device__ __forceinline__ int num_chunks(int len, int cap) {
  return len == 0 ? 0 : (int)(((long long)len + cap - 1) / cap);
}

struct Item {
  int b, g, c, n, len;
};

// Locate work item w. Returns false (uniformly) if w is past the last item.
__device__ bool find_item(int w, const PlanParams& p, int cap, Item* out, int* scan_red,
                          int* found) {
  if (threadIdx.x == 0) found[0] = -1;
  long long before = 0;   // chunks of all sequences before this block of b
  for (int b0 = 0; b0 < p.batch; b0 += kThreads) {
    const int b = b0 + threadIdx.x;
    const int len = b < p.batch ? clamp_len(p.seq_lens[b], p.capacity) : 0;
    const int n = num_chunks(len, cap);
    int total;
    const int incl = block_incl_scan(n, scan_red, &total);
    const long long lo = 8 * (before + incl - n), hi = 8 * (before + incl);
    if (n > 0 && w >= lo && w < hi) {
      found[0] = b;
      found[1] = (int)(w - lo);
      found[2] = n;
      found[3] = len;
    }
    before += total;
    __syncthreads();
    if (found[0] >= 0) break;
  }
  if (found[0] < 0) return false;
  out->b = found[0];
  out->n = found[2];
  out->len = found[3];
  out->g = found[1] / out->n;
  out->c = found[1] - out->g * out->n;
  return true;
}

// ---------------------------------------------------------------- kernel 1
__global__ __launch_bounds__(kThreads) void split_partial(
    const _Float16* __restrict__ q, const _Float16* __restrict__ kv, _Float16* __restrict__ out,
    float2* __restrict__ ws_ml, float* __restrict__ ws_acc, PlanParams pp, float scale_log2) {
  __shared__ long long red_ll[kWaves];
  __shared__ int red_i[kWaves];
  __shared__ int found[4];
  __shared__ float st_m[kStates][kGroup];
  __shared__ float st_l[kStates][kGroup];
  __shared__ float st_acc[kStates][kGroup][kDim];

  const int cap = chunk_cap(pp, red_ll);
  Item it;
  if (!find_item(blockIdx.x, pp, cap, &it, red_i, found)) return;

  // Near-equal chunks: every chunk is non-empty because (n-1)*cs < len.
  const int cs = (int)(((long long)it.len + it.n - 1) / it.n);
  const int start = it.c * cs;
  const int end = min(start + cs, it.len);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane >> 4, j = lane & 15;

  const size_t C = (size_t)pp.capacity;
  const _Float16* kbase = kv + ((size_t)(it.b * 2 + 0) * kKvHeads + it.g) * C * kDim + 8 * j;
  const _Float16* vbase = kv + ((size_t)(it.b * 2 + 1) * kKvHeads + it.g) * C * kDim + 8 * j;

  half2_t qf[kGroup][4];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(
        q + ((size_t)it.b * kQHeads + it.g * kGroup + h) * kDim + 8 * j);
    qf[h][0] = __builtin_bit_cast(half2_t, v.x);
    qf[h][1] = __builtin_bit_cast(half2_t, v.y);
    qf[h][2] = __builtin_bit_cast(half2_t, v.z);
    qf[h][3] = __builtin_bit_cast(half2_t, v.w);
  }

  const float kNegInf = -__builtin_inff();
  float m[kGroup], l[kGroup], acc[kGroup][8];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  for (int base = start + wv * kWaveRows; base < end; base += kBlockRows) {
    uint4 kr[kUnroll], vr[kUnroll];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int pos = base + kRowSlots * u + r;
      valid[u] = pos < end;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (valid[u]) {
        kr[u] = *reinterpret_cast<const uint4*>(kbase + (size_t)pos * kDim);
        vr[u] = *reinterpret_cast<const uint4*>(vbase + (size_t)pos * kDim);
      }
    }

    float s[kUnroll][kGroup];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const half2_t k0 = __builtin_bit_cast(half2_t, kr[u].x);
      const half2_t k1 = __builtin_bit_cast(half2_t, kr[u].y);
      const half2_t k2 = __builtin_bit_cast(half2_t, kr[u].z);
      const half2_t k3 = __builtin_bit_cast(half2_t, kr[u].w);
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        float a = __builtin_amdgcn_fdot2(qf[h][0], k0, 0.f, false);
        a = __builtin_amdgcn_fdot2(qf[h][1], k1, a, false);
        a = __builtin_amdgcn_fdot2(qf[h][2], k2, a, false);
        a = __builtin_amdgcn_fdot2(qf[h][3], k3, a, false);
        s[u][h] = row16_sum(a);
      }
    }

#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float mx = m[h];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        s[u][h] = valid[u] ? s[u][h] * scale_log2 : kNegInf;
        mx = fmaxf(mx, s[u][h]);
      }
      // mx == -inf only while this row slot has seen no valid position.
      const float alpha = (mx == kNegInf) ? 1.f : exp2_fast(m[h] - mx);
      m[h] = mx;
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        s[u][h] = valid[u] ? exp2_fast(s[u][h] - mx) : 0.f;
        psum += s[u][h];
      }
      l[h] = l[h] * alpha + psum;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
    }

#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const half2_t v0 = __builtin_bit_cast(half2_t, vr[u].x);
      const half2_t v1 = __builtin_bit_cast(half2_t, vr[u].y);
      const half2_t v2 = __builtin_bit_cast(half2_t, vr[u].z);
      const half2_t v3 = __builtin_bit_cast(half2_t, vr[u].w);
      const float vf[8] = {(float)v0.x, (float)v0.y, (float)v1.x, (float)v1.y,
                           (float)v2.x, (float)v2.y, (float)v3.x, (float)v3.y};
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(s[u][h], vf[e], acc[h][e]);
      }
    }
  }

  // Merge the 16 row-slot states of the workgroup.
  const int k = wv * kRowSlots + r;
  if (j == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      st_m[k][h] = m[h];
      st_l[k][h] = l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    float4* dst = reinterpret_cast<float4*>(&st_acc[k][h][8 * j]);
    dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
  }
  __syncthreads();

  const int hh = tid >> 6;          // head within the group
  const int d = (tid & 63) * 2;     // two output elements per thread
  float M = kNegInf;
#pragma unroll
  for (int s2 = 0; s2 < kStates; ++s2) M = fmaxf(M, st_m[s2][hh]);
  float den = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < kStates; ++s2) {
    const float ms = st_m[s2][hh];
    const float w = (ms == kNegInf) ? 0.f : exp2_fast(ms - M);
    den += w * st_l[s2][hh];
    n0 += w * st_acc[s2][hh][d];
    n1 += w * st_acc[s2][hh][d + 1];
  }

  const int head = it.g * kGroup + hh;
  if (it.n == 1) {
    half2_t o;
    o.x = (_Float16)(n0 / den);
    o.y = (_Float16)(n1 / den);
    *reinterpret_cast<half2_t*>(out + ((size_t)it.b * kQHeads + head) * kDim + d) = o;
  } else {
    const size_t slot = (size_t)blockIdx.x * kGroup + hh;
    *reinterpret_cast<float2*>(ws_acc + slot * kDim + d) = make_float2(n0, n1);
    if (d == 0) ws_ml[slot] = make_float2(M, den);
  }
}

// ---------------------------------------------------------------- kernel 2
constexpr int kCombineSubsets = kThreads / 64;   // chunk subsets reduced in parallel

__global__ __launch_bounds__(kThreads) void split_combine(
    _Float16* __restrict__ out, const float2* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    PlanParams pp) {
  __shared__ long long red_ll[kWaves];
  __shared__ float red_f[kWaves];
  __shared__ float part[kCombineSubsets][3][64];

  const int b = blockIdx.x / kQHeads;
  const int head = blockIdx.x - b * kQHeads;
  const int g = head / kGroup, hh = head - g * kGroup;
  const int tid = threadIdx.x;

  const int cap = chunk_cap(pp, red_ll);
  long long before = 0;
  for (int b2 = tid; b2 < b; b2 += kThreads)
    before += num_chunks(clamp_len(pp.seq_lens[b2], pp.capacity), cap);
  before = block_sum_ll(before, red_ll);
  const int len = clamp_len(pp.seq_lens[b], pp.capacity);
  const int n = num_chunks(len, cap);

  _Float16* dst = out + ((size_t)b * kQHeads + head) * kDim;
  if (n == 1) return;                       // written by the partial kernel
  if (n == 0) {                             // empty prefix: zero row
    if (tid < kDim / 2) {
      half2_t z;
      z.x = (_Float16)0.f;
      z.y = (_Float16)0.f;
      reinterpret_cast<half2_t*>(dst)[tid] = z;
    }
    return;
  }

  const long long item0 = 8 * before + (long long)g * n;
  float M = -__builtin_inff();
  for (int c = tid; c < n; c += kThreads) M = fmaxf(M, ws_ml[(item0 + c) * kGroup + hh].x);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) red_f[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));

  const int sub = tid >> 6, dp = tid & 63;
  float den = 0.f, n0 = 0.f, n1 = 0.f;
  for (int c = sub; c < n; c += kCombineSubsets) {
    const size_t slot = (size_t)(item0 + c) * kGroup + hh;
    const float2 ml = ws_ml[slot];
    const float2 a = *reinterpret_cast<const float2*>(ws_acc + slot * kDim + 2 * dp);
    const float w = exp2_fast(ml.x - M);
    den += w * ml.y;
    n0 += w * a.x;
    n1 += w * a.y;
  }
  part[sub][0][dp] = den;
  part[sub][1][dp] = n0;
  part[sub][2][dp] = n1;
  __syncthreads();
  if (sub == 0) {
    den = part[0][0][dp] + part[1][0][dp] + part[2][0][dp] + part[3][0][dp];
    n0 = part[0][1][dp] + part[1][1][dp] + part[2][1][dp] + part[3][1][dp];
    n1 = part[0][2][dp] + part[1][2][dp] + part[2][2][dp] + part[3][2][dp];
    half2_t o;
    o.x = (_Float16)(n0 / den);
    o.y = (_Float16)(n1 / den);
    reinterpret_cast<half2_t*>(dst)[dp] = o;
  }
}

}  // namespace

long long max_work_items(int batch, int capacity, const SplitConfig& cfg) {
  const long long per_seq_cap =
      cfg.forced_chunk > 0 ? ((long long)capacity + cfg.forced_chunk - 1) / cfg.forced_chunk
                           : ((long long)capacity + cfg.min_chunk - 1) / cfg.min_chunk;
  long long items = 8LL * batch * per_seq_cap;
  if (cfg.forced_chunk <= 0) {
    const long long bound = (long long)cfg.target_items + 8LL * batch;
    if (bound < items) items = bound;
  }
  return items > 0x7fffffffLL ? -1 : items;
}

size_t workspace_bytes_for_items(long long items) {
  return (size_t)items * kGroup * (sizeof(float2) + kDim * sizeof(float));
}

hipError_t launch_decode(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                         float score_scale_log2, int batch, int capacity,
                         const SplitConfig& cfg, long long grid_items, void* workspace,
                         hipStream_t stream, hipEvent_t* events) {
  PlanParams pp;
  pp.seq_lens = seq_lens;
  pp.batch = batch;
  pp.capacity = capacity;
  pp.target_items = cfg.target_items;
  pp.min_chunk = cfg.min_chunk;
  pp.forced_chunk = cfg.forced_chunk;

  float2* ws_ml = reinterpret_cast<float2*>(workspace);
  float* ws_acc = reinterpret_cast<float*>(ws_ml + (size_t)grid_items * kGroup);

  hipError_t err = hipSuccess;
  if (events && (err = hipEventRecord(events[0], stream)) != hipSuccess) return err;
  split_partial<<<dim3((unsigned)grid_items), dim3(kThreads), 0, stream>>>(
      static_cast<const _Float16*>(q), static_cast<const _Float16*>(kv),
      static_cast<_Float16*>(out), ws_ml, ws_acc, pp, score_scale_log2);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (events && (err = hipEventRecord(events[1], stream)) != hipSuccess) return err;
  split_combine<<<dim3((unsigned)(batch * kQHeads)), dim3(kThreads), 0, stream>>>(
      static_cast<_Float16*>(out), ws_ml, ws_acc, pp);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (events && (err = hipEventRecord(events[2], stream)) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace gqa

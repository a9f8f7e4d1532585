// FP16 GQA single-token decode for gfx950 (MI355X, CDNA4, wave64).
//
// Operation (FlashInfer PR #5052 analysis page, "SM110 FP16 GQA decode":
// section 1 docstring, section 2 specialisation, section 3 SDPA comparator):
// for batch entry b and query head h, with g = h / 4 and L = clamp(len, 0, C),
//   out[b,h] = softmax_i(q_scale / sqrt(128) * q[b,h] . K[b,g,i]) . V[b,g,i],  i < L.
//
// Work split (decided on the device from seq_lens; the host never reads them)
//   The valid rows of all (b, g) pairs are laid end to end, b-major then g:
//   segment (b, g) covers flat rows [8*P_b + g*L_b, +L_b), P_b = L_0 + ... +
//   L_{b-1}. That flat range of 8*sum(L) rows is cut into equal pieces of Q
//   rows, one per workgroup, so every workgroup streams the same number of
//   K/V bytes and all finish together. A piece covers the tail of one
//   segment, any number of whole segments and the head of another.
//   A segment inside one piece is finished by that workgroup (normalised
//   fp16 output). A segment cut by piece boundaries gets one fp32 partial
//   (running max, softmax denominator, unnormalised weighted V sum) per
//   piece, and a second kernel (one workgroup per sequence and query head)
//   merges them with a log-sum-exp rescale. The kernel boundary makes the partials visible
//   across XCDs; merging inside the first kernel would need device-scope
//   release fences (an L2 write-back per workgroup), which cost far more.
//
// Per-wave compute on the matrix cores (v_mfma_f32_16x16x32_f16, fp32
// accumulate), 32 rows per iteration; the 4 waves of a workgroup take
// interleaved 32-row tiles of their range:
//   QK: A = 16 K rows x 32 depth, loaded from HBM straight into registers
//       (lane (G, j) takes row j, depth 32kk + 8G .. +7, for kk = 0..3);
//       B = q^T with the group's 4 heads in columns 0..3 and zero columns
//       4..15. D gives lane (G, j) the scores of rows 4G..4G+3 for head j.
//   Online softmax in base 2 (scores carry log2(e)); rows at or beyond the
//   range end are never loaded and get score -inf and weight 0 by selects.
//   PV: A = weights (rows = heads, k = 32 rows), B = 32 V rows x 16 head-dim
//       columns. Two QK tiles' D layout already is one PV step's A layout
//       (lane (G, j) holds head j at rows 4G+r and 16+4G+r), so the weights
//       stay in their lanes; V takes the same row order through a per-wave
//       LDS tile read back transposed (ds_read_b64_tr_b16).
//   Weights are split into fp16 high and low parts (two MFMAs) so the sum
//   keeps fp32-level accuracy; the denominator sums the fp32 weights.
// Each K/V row crosses HBM once, for all 4 query heads of its group.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace gqa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef unsigned uint4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

constexpr int kQHeads = 32;
constexpr int kKvHeads = 8;
constexpr int kGroup = kQHeads / kKvHeads;   // 4 query heads per KV head
constexpr int kDim = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 32;                    // rows per wave per iteration
constexpr int kVStride = kDim + 8;           // LDS row stride of a V tile, in halves
constexpr int kSlotFloats = kGroup * (2 + kDim);   // one partial: 4 x (max, den) + 4 x 128 sums

struct Params {
  const _Float16* q;
  const _Float16* kv;
  const int32_t* seq_lens;
  _Float16* out;
  float2* ws_ml;       // [2 * grid][4] (max, denominator) per partial and head
  float* ws_acc;       // [2 * grid][4][128] unnormalised weighted V sums
  int2* seg_desc;      // [8 * batch] per segment: first piece, 2 * pieces + second-slot bit
  int batch;
  int capacity;
  int pieces;          // automatic split: number of equal pieces
  int min_piece;       // automatic split: lower bound on the piece length
  int forced_piece;    // > 0: fixed piece length
  float scale_log2;    // q_scale / sqrt(128) * log2(e)
};

__device__ __forceinline__ int clamp_len(int v, int cap) { return v < 0 ? 0 : (v > cap ? cap : v); }

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ long long uniform64(long long v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4_t load_nt(const _Float16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint4_t*>(p));
}

// ---------------------------------------------------------------- planning
// Workgroup-wide helpers; every thread of the workgroup must call them.

__device__ long long block_sum(long long v, long long* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  return t;
}

// Inclusive prefix sum over the workgroup; *total receives the sum of all.
__device__ long long block_scan(long long v, long long* red, long long* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  __syncthreads();
  if (lane == 63) red[wv] = v;
  __syncthreads();
  long long before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    before += (i < wv) ? red[i] : 0;
    all += red[i];
  }
  *total = all;
  return v + before;
}

// Batch entry b whose flat rows [8*P_b, 8*P_{b+1}) hold flat row p, and
// 8*P_b. p must be below 8 * sum(L).
__device__ void locate(long long p, const Params& P, long long* red, long long* found,
                       int* found_b) {
  if (threadIdx.x == 0) *found_b = -1;
  long long before = 0;
  for (int b0 = 0; b0 < P.batch; b0 += kThreads) {
    const int b = b0 + threadIdx.x;
    const long long len = b < P.batch ? clamp_len(P.seq_lens[b], P.capacity) : 0;
    long long total;
    const long long incl = block_scan(8 * len, red, &total);
    const long long lo = before + incl - 8 * len;
    if (len > 0 && p >= lo && p < lo + 8 * len) {
      *found_b = b;
      *found = lo;
    }
    before += total;
    __syncthreads();
    if (*found_b >= 0) break;
  }
}

// Small batches (<= 64): every wave finds the total and the batch entry of
// flat row p on its own (lane b holds sequence b), with no workgroup barrier.
// Returns the total valid rows; *found_b = -1 if p is past them.
__device__ long long wave_plan(const Params& P, long long (*piece_start)(const Params&, long long),
                               long long* p_out, long long* found, int* found_b) {
  const int lane = threadIdx.x & 63;
  const long long len = lane < P.batch ? clamp_len(P.seq_lens[lane], P.capacity) : 0;
  long long incl = 8 * len;
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  const long long total = __shfl(incl, 63);
  const long long p = piece_start(P, total);
  *p_out = p;
  const long long lo = incl - 8 * len;
  const unsigned long long hit = __ballot(len > 0 && p >= lo && p < incl);
  if (hit == 0) {
    *found_b = -1;
    return total;
  }
  const int b = __ffsll((long long)hit) - 1;
  *found_b = b;
  *found = __shfl(lo, b);
  return total;
}

struct Segment {
  int b, g, len;
  long long off;     // first flat row of the segment
};

// ---------------------------------------------------------------- compute
struct WaveAcc {
  float4_t O[8];     // PV accumulators (D layout): lane (0, j), reg r = head r, column 16*db + j
  float m;           // running max of head j (same in the 4 lane groups)
  float l;           // this lane group's share of head j's denominator
};

// Accumulate rows [lo, hi) of one (b, g) segment into the wave's state. The
// waves of the workgroup take interleaved 32-row tiles.
__device__ __forceinline__ void accumulate_rows(const _Float16* kbase, const _Float16* vbase,
                                                int lo, int hi, const half8_t qb[4],
                                                float scale_log2, _Float16* vt, WaveAcc& acc) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int G = lane >> 4, j = lane & 15;
  const float kNegInf = -__builtin_inff();
  const int tr_row = 4 * G + (j >> 2);
  const int tr_col = 4 * (j & 3);

  for (int t0 = lo + wv * kTile; t0 < hi; t0 += kWaves * kTile) {
    uint4_t kr[2][4], vr[8];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int pos = t0 + 16 * st + j;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        kr[st][kk] = (uint4_t){0u, 0u, 0u, 0u};
        if (pos < hi) kr[st][kk] = load_nt(kbase + (size_t)pos * kDim + 32 * kk + 8 * G);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pos = t0 + 4 * u + G;
      vr[u] = (uint4_t){0u, 0u, 0u, 0u};
      if (pos < hi) vr[u] = load_nt(vbase + (size_t)pos * kDim + 8 * j);
    }

    float4_t sc[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      sc[st] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sc[st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kr[st][kk]),
                                                        qb[kk], sc[st], 0, 0, 0);
    }

#pragma unroll
    for (int u = 0; u < 8; ++u)
      *reinterpret_cast<uint4_t*>(vt + (4 * u + G) * kVStride + 8 * j) = vr[u];

    float sv[8];
    float mx = kNegInf;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = t0 + 16 * st + 4 * G + r;
        const float x = pos < hi ? sc[st][r] * scale_log2 : kNegInf;
        sv[4 * st + r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Row t0 is below hi, so mx (and m_new) is finite; alpha is 0 on the
    // first tile, where acc.m is still -inf.
    const float m_new = fmaxf(acc.m, mx);
    const float alpha = exp2_hw(acc.m - m_new);
    acc.m = m_new;

    half8_t ph, pl;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = (sv[e] == kNegInf) ? 0.f : exp2_hw(sv[e] - m_new);
      psum += p;
      const _Float16 hi16 = (_Float16)p;
      ph[e] = hi16;
      pl[e] = (_Float16)(p - (float)hi16);
    }
    acc.l = acc.l * alpha + psum;

    // Row r of every PV tile is head r; lane h holds head h's alpha.
    const float a0 = __shfl(alpha, 0), a1 = __shfl(alpha, 1), a2 = __shfl(alpha, 2),
                a3 = __shfl(alpha, 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      acc.O[db][0] *= a0;
      acc.O[db][1] *= a1;
      acc.O[db][2] *= a2;
      acc.O[db][3] *= a3;
    }

#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const short4_t b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4_t*)(vt + tr_row * kVStride + 16 * db + tr_col));
      const short4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4_t*)(vt + (16 + tr_row) * kVStride + 16 * db + tr_col));
      half8_t vb;
      vb.lo = __builtin_bit_cast(half4_t, b0);
      vb.hi = __builtin_bit_cast(half4_t, b1);
      acc.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, vb, acc.O[db], 0, 0, 0);
      acc.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, vb, acc.O[db], 0, 0, 0);
    }
  }
}

struct MergeLds {
  float m[kWaves][kGroup];
  float l[kWaves][kGroup];
  float acc[kWaves][kGroup][kDim];
};

// Merge the 4 waves' states. Thread t ends with head hh = t / 64 and the
// columns d, d+1 (d = 2 * (t % 64)): max M, denominator den, sums n0, n1.
__device__ __forceinline__ void merge_waves(const WaveAcc& acc, MergeLds& sm, float& M,
                                            float& den, float& n0, float& n1) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = lane >> 4, j = lane & 15;
  const float kNegInf = -__builtin_inff();
  float l = acc.l + __shfl_xor(acc.l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();   // earlier readers of sm are done
  if (lane < kGroup) {
    sm.m[wv][lane] = acc.m;
    sm.l[wv][lane] = l;
  }
  if (G == 0) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.acc[wv][r][16 * db + j] = acc.O[db][r];
    }
  }
  __syncthreads();
  const int hh = tid >> 6, d = (tid & 63) * 2;
  M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.m[w][hh]);
  den = 0.f;
  n0 = 0.f;
  n1 = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float ms = sm.m[w][hh];
    const float wt = (ms == kNegInf) ? 0.f : exp2_hw(ms - M);   // waves without rows
    den += wt * sm.l[w][hh];
    n0 += wt * sm.acc[w][hh][d];
    n1 += wt * sm.acc[w][hh][d + 1];
  }
}

// Partial slot of a segment in piece w: 2w for the piece's first segment,
// 2w + 1 for a segment that starts strictly inside the piece (at most one of
// those is cut by the piece's end).
__device__ __forceinline__ long long slot_of(long long seg_off, long long piece_start, int w) {
  return 2LL * w + (seg_off > piece_start ? 1 : 0);
}

// Piece length Q for this call.
__device__ __forceinline__ long long piece_len(const Params& P, long long total) {
  if (P.forced_piece > 0) return P.forced_piece;
  long long Q = (total + P.pieces - 1) / P.pieces;
  return Q < P.min_piece ? P.min_piece : Q;
}

__device__ long long this_piece_start(const Params& P, long long total) {
  return (long long)blockIdx.x * piece_len(P, total);
}

// ---------------------------------------------------------------- kernel 1
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gqa_decode_pieces(Params P) {
  __shared__ long long red[kWaves];
  __shared__ long long sh_found;
  __shared__ int sh_found_b;
  __shared__ __attribute__((aligned(16))) _Float16 vtile[kWaves][kTile * kVStride];
  __shared__ __attribute__((aligned(16))) MergeLds sm;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = lane >> 4, j = lane & 15;
  const int w = blockIdx.x;

  // Empty sequences get zero rows and empty segment descriptors
  // (workgroup w takes b = w, w + grid, ...).
  for (int b = w; b < P.batch; b += gridDim.x) {
    if (clamp_len(P.seq_lens[b], P.capacity) == 0) {
      uint4_t* dst = reinterpret_cast<uint4_t*>(P.out + (size_t)b * kQHeads * kDim);
      dst[tid] = (uint4_t){0u, 0u, 0u, 0u};
      dst[tid + kThreads] = (uint4_t){0u, 0u, 0u, 0u};
      if (tid < kKvHeads) P.seg_desc[b * kKvHeads + tid] = make_int2(0, 0);
    }
  }

  long long total, p0, found;
  int found_b;
  if (P.batch <= 64) {
    total = wave_plan(P, this_piece_start, &p0, &found, &found_b);
  } else {
    long long part = 0;
    for (int b = tid; b < P.batch; b += kThreads) part += clamp_len(P.seq_lens[b], P.capacity);
    total = 8 * block_sum(part, red);
    p0 = this_piece_start(P, total);
    found_b = -1;
    if (p0 < total) {
      locate(p0, P, red, &sh_found, &sh_found_b);
      __syncthreads();
      found_b = sh_found_b;
      found = sh_found;
    }
  }
  total = uniform64(total);
  p0 = uniform64(p0);
  if (p0 >= total) return;                          // uniform: this piece is empty
  found = uniform64(found);
  found_b = __builtin_amdgcn_readfirstlane(found_b);
  const long long Q = piece_len(P, total);
  const long long p1 = p0 + Q < total ? p0 + Q : total;

  Segment s;
  s.b = found_b;
  s.len = clamp_len(P.seq_lens[s.b], P.capacity);
  s.g = (int)((p0 - found) / s.len);
  s.off = found + (long long)s.g * s.len;

  _Float16* vt = vtile[wv];
  const size_t C = (size_t)P.capacity;
  long long cur = p0;
  while (true) {
    const long long seg_end = s.off + s.len;
    const long long hi_flat = seg_end < p1 ? seg_end : p1;
    const int lo = (int)(cur - s.off), hi = (int)(hi_flat - s.off);

    // q^T as the B operand, one 32-deep slice per kk; columns >= 4 are zero.
    half8_t qb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4_t v = {0u, 0u, 0u, 0u};
      if (j < kGroup)
        v = *reinterpret_cast<const uint4_t*>(
            P.q + ((size_t)s.b * kQHeads + s.g * kGroup + j) * kDim + 32 * kk + 8 * G);
      qb[kk] = __builtin_bit_cast(half8_t, v);
    }
    const _Float16* kbase = P.kv + ((size_t)(s.b * 2 + 0) * kKvHeads + s.g) * C * kDim;
    const _Float16* vbase = P.kv + ((size_t)(s.b * 2 + 1) * kKvHeads + s.g) * C * kDim;

    WaveAcc acc;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc.O[db] = (float4_t){0.f, 0.f, 0.f, 0.f};
    acc.m = -__builtin_inff();
    acc.l = 0.f;
    accumulate_rows(kbase, vbase, lo, hi, qb, P.scale_log2, vt, acc);

    float M, den, n0, n1;
    merge_waves(acc, sm, M, den, n0, n1);
    const int hh = tid >> 6, d = (tid & 63) * 2;

    const long long first_w = s.off / Q, last_w = (seg_end - 1) / Q;
    if (first_w == w && tid == 0)                    // the segment starts in this piece
      P.seg_desc[s.b * kKvHeads + s.g] =
          make_int2(w, (int)(2 * (last_w - first_w + 1)) + (s.off > p0 ? 1 : 0));
    if (first_w == last_w) {                         // the segment lies in this piece
      half2_t o;
      o.x = (_Float16)(n0 / den);
      o.y = (_Float16)(n1 / den);
      *reinterpret_cast<half2_t*>(P.out + ((size_t)s.b * kQHeads + s.g * kGroup + hh) * kDim + d) = o;
    } else {
      const long long slot = slot_of(s.off, p0, w);
      *reinterpret_cast<float2*>(P.ws_acc + (slot * kGroup + hh) * kDim + d) = make_float2(n0, n1);
      if (d == 0) P.ws_ml[slot * kGroup + hh] = make_float2(M, den);
    }

    cur = hi_flat;
    if (cur >= p1) break;
    // Next segment: next KV head of b, else the next non-empty sequence
    // (one exists, because rows remain below p1 <= total).
    if (s.g + 1 < kKvHeads) {
      s.g += 1;
    } else {
      int nb = s.b + 1;
      int nl = clamp_len(P.seq_lens[nb], P.capacity);
      while (nl == 0) {
        ++nb;
        nl = clamp_len(P.seq_lens[nb], P.capacity);
      }
      s.b = nb;
      s.len = nl;
      s.g = 0;
    }
    s.off = seg_end;
  }
}

// ---------------------------------------------------------------- kernel 2
constexpr int kCombineSubsets = kThreads / 32;   // 8 subsets x 32 four-column groups

// One workgroup per (b, query head): if kernel 1 cut the segment (b, h / 4)
// into several pieces, merge their partials for head h and write the output
// row; otherwise exit. Each of 8 thread subsets merges every 8th partial
// with a running max (its loads do not depend on each other), then the
// subsets are merged through LDS.
__global__ __launch_bounds__(kThreads) void gqa_decode_combine(Params P) {
  __shared__ __attribute__((aligned(16))) float xs[kCombineSubsets][32][6];

  const int tid = threadIdx.x;
  const int b = blockIdx.x / kQHeads, head = blockIdx.x - b * kQHeads;
  const int g = head / kGroup, hh = head - g * kGroup;
  const int2 desc = P.seg_desc[b * kKvHeads + g];
  const int n = desc.y >> 1;
  if (n <= 1) return;                  // empty (zero row) or finished by kernel 1
  const int first_w = desc.x;
  // Partial i lives in piece first_w + i: the first piece may hold it in its
  // second slot, every later piece holds it as its first segment.
  const long long slot0 = 2LL * first_w + (desc.y & 1);

  const int sub = tid >> 5, c4 = (tid & 31) * 4;
  const float kNegInf = -__builtin_inff();
  float M = kNegInf, den = 0.f;
  float4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int i = sub; i < n; i += kCombineSubsets) {
    const long long sl = i == 0 ? slot0 : 2LL * (first_w + i);
    const float2 ml = P.ws_ml[sl * kGroup + hh];
    const float4_t a = *reinterpret_cast<const float4_t*>(P.ws_acc + (sl * kGroup + hh) * kDim + c4);
    const float Mn = fmaxf(M, ml.x);
    const float s_old = exp2_hw(M - Mn), s_new = exp2_hw(ml.x - Mn);
    den = den * s_old + ml.y * s_new;
    num = num * s_old + a * s_new;
    M = Mn;
  }
  float* x = xs[sub][tid & 31];
  x[0] = M;
  x[1] = den;
  x[2] = num[0];
  x[3] = num[1];
  x[4] = num[2];
  x[5] = num[3];
  __syncthreads();
  if (tid < 32) {
    float Mx = kNegInf;
#pragma unroll
    for (int k = 0; k < kCombineSubsets; ++k) Mx = fmaxf(Mx, xs[k][tid][0]);
    float d = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int k = 0; k < kCombineSubsets; ++k) {
      const float* y = xs[k][tid];
      const float wt = (y[0] == kNegInf) ? 0.f : exp2_hw(y[0] - Mx);   // subsets without partials
      d += wt * y[1];
      o0 += wt * y[2];
      o1 += wt * y[3];
      o2 += wt * y[4];
      o3 += wt * y[5];
    }
    half4_t o;
    o[0] = (_Float16)(o0 / d);
    o[1] = (_Float16)(o1 / d);
    o[2] = (_Float16)(o2 / d);
    o[3] = (_Float16)(o3 / d);
    *reinterpret_cast<half4_t*>(P.out + ((size_t)b * kQHeads + head) * kDim + 4 * tid) = o;
  }
}

}  // namespace

int resident_workgroups_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gqa_decode_pieces, kThreads, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

long long grid_for(int batch, int capacity, const SplitConfig& cfg) {
  if (cfg.forced_piece > 0) {
    const long long rows = 8LL * batch * capacity;
    return (rows + cfg.forced_piece - 1) / cfg.forced_piece;
  }
  return cfg.pieces;
}

size_t partial_bytes_for_grid(long long grid) {
  return (size_t)(2 * grid) * kSlotFloats * sizeof(float);
}

size_t segment_bytes_for_batch(int batch) {
  return ((size_t)batch * kKvHeads * sizeof(int2) + 255) & ~(size_t)255;
}

hipError_t launch_decode(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                         float score_scale_log2, int batch, int capacity, const SplitConfig& cfg,
                         long long grid, void* partials, hipStream_t stream, hipEvent_t* events) {
  Params P;
  P.q = static_cast<const _Float16*>(q);
  P.kv = static_cast<const _Float16*>(kv);
  P.seq_lens = seq_lens;
  P.out = static_cast<_Float16*>(out);
  P.seg_desc = reinterpret_cast<int2*>(partials);
  P.ws_ml = reinterpret_cast<float2*>(static_cast<char*>(partials) + segment_bytes_for_batch(batch));
  P.ws_acc = reinterpret_cast<float*>(P.ws_ml + (size_t)(2 * grid) * kGroup);
  P.batch = batch;
  P.capacity = capacity;
  P.pieces = (int)grid;
  P.min_piece = cfg.min_piece;
  P.forced_piece = cfg.forced_piece;
  P.scale_log2 = score_scale_log2;

  hipError_t err = hipSuccess;
  if (events && (err = hipEventRecord(events[0], stream)) != hipSuccess) return err;
  gqa_decode_pieces<<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (events && (err = hipEventRecord(events[1], stream)) != hipSuccess) return err;
  gqa_decode_combine<<<dim3((unsigned)(batch * kQHeads)), dim3(kThreads), 0, stream>>>(P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (events && (err = hipEventRecord(events[2], stream)) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace gqa

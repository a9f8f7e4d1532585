// FP16 GQA single-token decode for gfx950 (MI355X, CDNA4, wave64).
//
// Operation (FlashInfer PR #5052 analysis page, "SM110 FP16 GQA decode":
// section 1 docstring, section 2 specialisation, section 3 SDPA comparator):
// for batch entry b and query head h, with g = h / G (G = Hq / Hkv query
// heads per KV head; the page's case is Hq = 32, Hkv = 8, G = 4) and
// L = clamp(len, 0, C),
//   out[b,h] = softmax_i(q_scale / sqrt(128) * q[b,h] . K[b,g,i]) . V[b,g,i],  i < L.
//
// Work split (decided on the device from seq_lens; the host never reads them)
//   Every (b, g) pair with L_b > 0 is a segment of cost c0 + L_b: c0 units
//   stand for its fixed cost (q, merge, output) and come first, then one unit
//   per valid row. The segments are laid end to end, b-major then g, and that
//   cost line is cut into equal pieces of Q units, one per workgroup, so
//   workgroups get equal work and finish together, and tiny segments spread
//   over workgroups instead of queueing in one. A piece covers the tail of
//   one segment, any number of whole segments and the head of another; a
//   piece that holds only fixed-cost units of a segment skips it.
//   A segment inside one piece is finished by that workgroup (normalised
//   output). A segment cut by piece boundaries gets one fp32 partial
//   (running max, softmax denominator, unnormalised weighted V sum) per
//   piece, merged with a log-sum-exp rescale in a fixed order, either by a
//   second kernel (one workgroup per segment) or, in the single-launch form,
//   by the piece that completes the segment (per-segment atomic ticket).
//
// Per-wave compute on the matrix cores (fp32 accumulate), 16 rows per step;
// the 4 waves of a workgroup take interleaved 16-row tiles of each segment.
// Each wave streams its tiles through a two-stage LDS pipeline that runs
// across segment boundaries: while it computes tile i, the loads of tile
// i+1 (its next tile, in this segment or a later one) are in flight.
//   Buffer loads write K, V and the segment's q straight into LDS (no
//   register staging; 16-byte chunks of K/V rows XOR-swizzled by row). The
//   buffer resources are bounded by the segment's rows in this piece, so rows
//   past the range read as zeros, never as stored data.
//   QK (v_mfma_f32_16x16x32_f16): A = 16 K rows x 32 depth (lane (G4, j)
//   reads row j, depth 32kk + 8 G4 .. +7), B = q^T with the group's G <= 8
//   heads in columns 0..G-1 and zero columns G..15; D gives lane (G4, j) the
//   scores of rows 4 G4 .. 4 G4 + 3 for head j.
//   Online softmax in base 2 (scores carry log2(e)); rows at or beyond the
//   range end get score -inf and weight 0 by selects.
//   PV (v_mfma_f32_16x16x16_f16) computes O^T = V^T P^T: A = 16 V rows read
//   transposed from LDS (ds_read_b64_tr_b16: lane (G4, i) holds head-dim
//   column 16 db + i of rows 4 G4 .. +3), B = the weights, whose QK D layout
//   already is this B layout (lane (G4, j): head j, rows 4 G4 .. +3), so they
//   stay in their lanes. D gives lane (G4, j) head j's output columns
//   16 db + 4 G4 .. +3, so each lane rescales its accumulators by its own
//   head's factor. Weights are split into fp16 high and low parts (two MFMAs)
//   so the sum keeps fp32-level accuracy; the denominator sums the fp32
//   weights. fp16 weights are formed up to 2^15 instead of 1 (a reference
//   15 below the running maximum), so that their low parts stay normal fp16
//   numbers; the factor cancels between numerator and denominator.
//   LDS reads of a stage are issued from asm blocks with their own waits: the
//   compiler cannot tell the two stages apart and would otherwise wait for the
//   next tile's loads, which are in flight by design.
// Each K/V row crosses HBM once, for all G query heads of its group.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

// Scratch of the allocation-free entry point: the library's only device
// memory that is not allocated at run time. Host code never passes this
// name to a kernel or a copy (on the host it is a stand-in, not a device
// address); it uses the address that scratch_area() looks up per device.
static __device__ __align__(256) unsigned char scratch[gqa::kScratchBytes];

namespace gqa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t e16_t;      // 16-bit element storage: fp16 or bf16 bit patterns
typedef __attribute__((address_space(3))) void lds_void_t;
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef unsigned uint4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

constexpr int kMaxGroup = 8;                 // query heads per KV head, at most
constexpr int kDim = 128;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Kernels come in two forms: kG4 for exactly 4 query heads per KV head (the
// page's 32/8 case: group size, q loads and merge layout fixed at compile
// time) and a general form for any group of 1..8 heads.
template <bool kG4> constexpr int q_halves() { return (kG4 ? 4 : kMaxGroup) * kDim; }

// Element formats: q, K, V and out in fp16 or bf16 (16-row tiles of 256-byte
// rows), or fp16 q and out with OCP FP8 E4M3 K and V (32-row tiles of
// 128-byte rows; one stage holds the same 8 KiB), or fp16 q and out with
// block-scaled FP4 K and V (32-row tiles of 64-byte rows of E2M1 codes, plus
// 8 bytes of E4M3 block scales per row; a stage holds 4.5 KiB).
constexpr int kFmtF16 = 0, kFmtBf16 = 1, kFmtE4m3 = 2, kFmtFp4 = 3;
template <int F> constexpr int tile_rows() { return F == kFmtE4m3 || F == kFmtFp4 ? 32 : 16; }
template <int F> constexpr int row_bytes() {
  return F == kFmtFp4 ? kDim / 2 : F == kFmtE4m3 ? kDim : 2 * kDim;
}
constexpr int kFp4ScaleBytes = 8;            // E4M3 block scales per FP4 row (16 elements each)
// LDS pipeline stage of one wave: K rows, then V rows (kind_bytes each); FP4
// stages then hold the K and V block scales (32 rows x 8 B each).
template <int F> constexpr int kind_bytes() { return tile_rows<F>() * row_bytes<F>(); }
template <int F> constexpr int scale_offset() { return 2 * kind_bytes<F>(); }
template <int F> constexpr int stage_bytes() {
  return 2 * kind_bytes<F>() + (F == kFmtFp4 ? 2 * 32 * kFp4ScaleBytes : 0);
}
template <int F> constexpr int stage_halves() { return stage_bytes<F>() / 2; }
// Loads per tile and lane: 1 or 2 q loads (1 KiB each), then 4 x K and 4 x V
// (1 KiB each); FP4: 2 x K codes, 1 x K scales (256 B), 2 x V codes, 1 x V
// scales.
template <int F, bool kG4> constexpr int loads_per_tile() {
  return (kG4 ? 1 : 2) + (F == kFmtFp4 ? 6 : 8);
}
constexpr unsigned kBufferFlags = 0x00020000;     // raw buffer resource word 3 (gfx9 family)
constexpr int kNonTemporal = 2;              // buffer load cache policy: nt
constexpr int kHeadSlotFloats = 2 + kDim;   // one head of a partial: (max, den) + 128 sums
constexpr int kCombinePerHeadBelow = 256;   // segments: below, the combine may split heads

struct Params {
  const e16_t* q;
  const e16_t* kv;
  const uint8_t* kv_scales;   // FP4: E4M3 block scales, 8 per K or V row
  const int32_t* seq_lens;
  e16_t* out;
  float2* ws_ml;       // [2 * grid][G] (max, denominator) per partial and head
  float* ws_acc;       // [2 * grid][G][128] unnormalised weighted V sums
  int2* seg_desc;      // [Hkv * batch] per segment: first piece, 2 * pieces + second-slot bit
  int* tickets;        // [Hkv * batch] single launch: pieces of each segment done so far
                       // (zero between calls: the last piece resets its count)
  int fused;           // 1: the last piece of a cut segment merges its partials
  int batch;
  int capacity;
  int kv_heads;        // Hkv: segments per sequence
  int group;           // G = Hq / Hkv, 1 .. kMaxGroup
  int q_heads;         // Hq (rows of out per sequence)
  int wave_planner;    // 1: batch <= 64 and every cost total fits 32 bits
  int combine_per_head;   // combine kernel: one workgroup per (segment, head)
  int pieces;          // automatic split: number of pieces (one per workgroup)
  int pieces_first;    // automatic split: pieces 0 .. pieces_first - 1 are Qa units
                       // long, the others Qb (all equal when pieces_first == pieces)
  int second_share;    // Qb / Qa in 1/64ths (64: equal pieces)
  int min_piece;       // automatic split: lower bound on the piece length
  int forced_piece;    // > 0: fixed piece length
  int seg_cost;        // fixed cost units per segment (c0)
  float scale_log2;    // q_scale * k_scale / sqrt(128) * log2(e)
  float out_scale;     // v_scale: applied to the normalised output
  // Addressing, in bytes. q row (b, h) starts at q + b*q_sb + h*q_sh; K (kind
  // 0) or V (kind 1) row i of (b, g) at kv + b*kv_sb + kind*kv_sk + g*kv_sh +
  // i*kv_sr. Paged caches replace b*kv_sb by page*kv_sb, page =
  // block_table[b*max_pages + i/page_size], and i by i % page_size.
  long long q_sb, q_sh, kv_sb, kv_sk, kv_sh, kv_sr;
  long long sc_sb, sc_sk, sc_sh, sc_sr;   // FP4 block scales, addressed like kv
  const int32_t* block_table;   // paged: [batch][max_pages] page ids
  int max_pages, page_shift, num_pages;
  int row_align;                // 1, or 16 for paged caches: segments and pieces
                                // start at multiples of 16 rows
};

// Query heads per KV head: a compile-time 4 in the kG4 kernels.
template <bool kG4>
__device__ __forceinline__ int group_of(const Params& P) {
  return kG4 ? 4 : P.group;
}

__device__ __forceinline__ int clamp_len(int v, int cap) { return v < 0 ? 0 : (v > cap ? cap : v); }

// Rows a segment of length len occupies on the cost line: len rounded up to
// the row alignment (so that with alignment 16 every segment's rows, and
// every piece, start at a multiple of 16).
__device__ __forceinline__ long long cost_len(const Params& P, long long len) {
  return (len + P.row_align - 1) & ~(long long)(P.row_align - 1);
}

// Cost of sequence b on the cost line: Hkv segments of c0 + L units, or 0.
__device__ __forceinline__ long long seq_cost(const Params& P, long long len) {
  return len > 0 ? (long long)P.kv_heads * (cost_len(P, len) + P.seg_cost) : 0;
}

// Length of sequence b read through the scalar path (b must be uniform), so
// waiting for it does not wait for vector loads in flight.
__device__ __forceinline__ int seq_len_uniform(const int32_t* lens, int b, int cap) {
  const __attribute__((address_space(4))) int32_t* c = (const __attribute__((address_space(4))) int32_t*)lens;
  return clamp_len(c[b], cap);
}

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ long long uniform64(long long v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane steps on the VALU (no LDS round trip). The permlane swaps of
// gfx950 exchange 16-lane rows: called with the same value twice, each
// returns, per lane, the lane's own value and that of lane ^ 16 (resp.
// lane ^ 32) as its two results, so a symmetric op of the two results
// reduces over the pair.
__device__ __forceinline__ unsigned fbits(float x) { return __builtin_bit_cast(unsigned, x); }
__device__ __forceinline__ float bitsf(unsigned x) { return __builtin_bit_cast(float, x); }

// Max over the lanes j, j + 16, j + 32, j + 48 (j = lane % 16).
__device__ __forceinline__ float max_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  x = fmaxf(bitsf(a[0]), bitsf(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return fmaxf(bitsf(b[0]), bitsf(b[1]));
}

// Sum over the lanes j, j + 16, j + 32, j + 48 (j = lane % 16).
__device__ __forceinline__ float sum_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(x), false, false);
  x = bitsf(a[0]) + bitsf(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(x), false, false);
  return bitsf(b[0]) + bitsf(b[1]);
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

// Batch entry b whose cost range holds position p, and the start of that
// range. p must be below the total cost.
__device__ void locate(long long p, const Params& P, long long* red, long long* found,
                       int* found_b, int* found_len) {
  if (threadIdx.x == 0) *found_b = -1;
  long long before = 0;
  for (int b0 = 0; b0 < P.batch; b0 += kThreads) {
    const int b = b0 + threadIdx.x;
    const long long len = b < P.batch ? clamp_len(P.seq_lens[b], P.capacity) : 0;
    long long total;
    const long long cost = seq_cost(P, len);
    const long long incl = block_scan(cost, red, &total);
    const long long lo = before + incl - cost;
    if (cost > 0 && p >= lo && p < lo + cost) {
      *found_b = b;
      *found = lo;
      *found_len = (int)len;
    }
    before += total;
    __syncthreads();
    if (*found_b >= 0) break;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips): within each 16-lane row by shifts of
// 1, 2, 4 and 8, then row 0's total into rows 1 and 3 (row_bcast:15) and
// rows 0-1's total into rows 2 and 3 (row_bcast:31). Lanes whose source is
// outside the row, or disabled by the row mask, add 0.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// The cost line of a call is cut into P.pieces pieces, one per workgroup:
// pieces 0 .. G1 - 1 are Qa units long, the others Qb. With G1 == pieces (or
// a forced length) all are equal. Otherwise the workgroups that share a CU
// with an older one (ids >= G1, the second round of the dispatch) get the
// shorter pieces: on a CU the older workgroup's waves win instruction issue,
// which slows the younger ones by up to 1.6x in the compute-heavier kernels
// (FP4: 1.53 vs 0.94 us per tile, measured with per-wave clocks), and the
// CU's last stretch, with only the younger workgroup left, runs one wave
// per SIMD.
struct Pieces {
  long long Qa, Qb, G1;
};
constexpr long long kTwoRateMinUnits = 1024;   // cost units per piece, on average

__device__ __forceinline__ long long piece_start(const Pieces& pc, long long w) {
  return w < pc.G1 ? w * pc.Qa : pc.G1 * pc.Qa + (w - pc.G1) * pc.Qb;
}

__device__ __forceinline__ long long piece_length(const Pieces& pc, long long w) {
  return w < pc.G1 ? pc.Qa : pc.Qb;
}

// x / q for cost positions (both non-negative).
__device__ __forceinline__ long long div_cost(const Params& P, long long x, long long q) {
  return P.wave_planner ? (long long)((unsigned)x / (unsigned)q) : x / q;
}

// Index of the piece holding cost position x (below the total).
__device__ __forceinline__ long long piece_of(const Params& P, const Pieces& pc, long long x) {
  const long long a = pc.G1 * pc.Qa;
  return x < a ? div_cost(P, x, pc.Qa) : pc.G1 + div_cost(P, x - a, pc.Qb);
}

// Piece lengths for a cost total (32-bit arithmetic where the planner keeps
// every total below 2^32). Equal pieces: Q = ceil(total / pieces), at least
// min_piece, rounded up to the row alignment. Two lengths: Qb = ceil(Qa *
// share / 64) (at least min_piece, aligned) and Qa the smallest aligned
// length that covers the total, G1 Qa + (pieces - G1) Qb >= total (a double
// estimate, then exact upward steps).
__device__ __forceinline__ Pieces piece_lens(const Params& P, long long total) {
  Pieces pc;
  pc.G1 = P.pieces;
  if (P.forced_piece > 0) {
    pc.Qa = pc.Qb = P.forced_piece;
    return pc;
  }
  // Two lengths only for long pieces: on short ones (a few tiles per wave)
  // the call is latency-bound and the longer pieces would set its end.
  if (P.pieces_first >= P.pieces || total < (long long)P.pieces * kTwoRateMinUnits) {
    long long Q;
    if (P.wave_planner) {
      const unsigned t = (unsigned)total;
      Q = t / (unsigned)P.pieces + (t % (unsigned)P.pieces != 0);
    } else {
      Q = (total + P.pieces - 1) / P.pieces;
    }
    Q = Q < P.min_piece ? P.min_piece : Q;
    pc.Qa = pc.Qb = cost_len(P, Q);
    return pc;
  }
  const long long G1 = P.pieces_first, G2 = P.pieces - G1;
  auto qb_of = [&](long long qa) {
    long long qb = (qa * P.second_share + 63) / 64;
    qb = qb < P.min_piece ? P.min_piece : qb;
    return cost_len(P, qb);
  };
  const double den = (double)G1 + (double)G2 * (double)P.second_share * (1.0 / 64.0);
  long long qa = (long long)((double)total / den);
  qa = cost_len(P, qa < P.min_piece ? P.min_piece : qa);
  while (G1 * qa + G2 * qb_of(qa) < total) qa += P.row_align;
  const long long qb = qb_of(qa);
  pc.G1 = G1;
  pc.Qa = qa < qb ? qb : qa;
  pc.Qb = qb;
  return pc;
}

// Small batches (<= 64): raw_len is lane b's seq_lens[b] (loaded at kernel
// entry). Every wave finds the total and the batch entry of
// this workgroup's first cost position on its own (lane b holds sequence b),
// with no workgroup barrier and no LDS traffic. The total fits 32 bits: at
// most 64 * 8 * (2^22 + 16 + c0) units. Returns the total; *found_b = -1 if
// the piece starts past it. *lens_v keeps the clamped lengths (lane b holds
// sequence b's), so later segment steps read them with readlane instead of a
// dependent memory load.
__device__ long long wave_plan(const Params& P, int raw_len, long long* p_out, Pieces* pc_out,
                               long long* found, int* found_b, int* lens_v) {
  const int lane = threadIdx.x & 63;
  const long long len = lane < P.batch ? clamp_len(raw_len, P.capacity) : 0;
  *lens_v = (int)len;
  // 32-bit cost (the planner is only used when every total fits 32 bits)
  const unsigned cost =
      len > 0 ? (unsigned)P.kv_heads * (unsigned)(cost_len(P, len) + P.seg_cost) : 0u;
  const unsigned incl = wave_incl_scan(cost);
  const unsigned total = (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
  const Pieces pc = piece_lens(P, total);
  const long long p = piece_start(pc, blockIdx.x);
  *p_out = p;
  *pc_out = pc;
  const long long lo = (long long)(incl - cost);
  const unsigned long long hit = __ballot(cost > 0 && p >= lo && p < (long long)incl);
  if (hit == 0) {
    *found_b = -1;
    return total;
  }
  const int b = __ffsll((long long)hit) - 1;
  *found_b = b;
  *found = (unsigned)__builtin_amdgcn_readlane((int)(incl - cost), b);
  return total;
}

struct Segment {
  int b, g, len;
  long long off;     // first flat row of the segment
};

// ---------------------------------------------------------------- compute
// Position of 16-byte chunk c of row r inside an LDS V stage.
__device__ __forceinline__ int vchunk(int r, int c) { return c ^ (2 * (r & 7)); }

// Rows [lo, hi) of segment (b, g) that lie in this workgroup's piece; row i
// of the segment sits at cost position off + i (its fixed-cost units are
// [off - c0, off)). Wave-uniform. The byte offsets of the segment's blocks
// (set by seg_bases when the walk enters the segment) spare the tile loads
// their 64-bit products: kvo is K row 0 of (b, g) relative to P.kv (paged
// caches: the head's offset inside a page), sco the same for the FP4 block
// scales, qo the group's first q row relative to P.q.
struct Seg {
  int b, g, len, lo, hi;
  long long off;
  long long kvo, sco, qo;
  const __attribute__((address_space(4))) int32_t* btr;   // paged caches: b's block-table row
};

template <int F, bool kPaged>
__device__ __forceinline__ void seg_bases(const Params& P, Seg& s) {
  if constexpr (kPaged)
    s.btr = (const __attribute__((address_space(4))) int32_t*)P.block_table +
            (long long)s.b * P.max_pages;
  s.kvo = (kPaged ? 0 : (long long)s.b * P.kv_sb) + (long long)s.g * P.kv_sh;
  if constexpr (F == kFmtFp4)
    s.sco = (kPaged ? 0 : (long long)s.b * P.sc_sb) + (long long)s.g * P.sc_sh;
  s.qo = (long long)s.b * P.q_sb + (long long)(s.g * P.group) * P.q_sh;
}

__device__ __forceinline__ void seg_set_range(Seg& s, long long p_begin, long long p_end) {
  const long long b = p_begin - s.off, e = p_end - s.off;
  s.lo = (int)(b <= 0 ? 0 : (b < s.len ? b : s.len));
  s.hi = (int)(e <= 0 ? 0 : (e < s.len ? e : s.len));
}

// Whether the piece ending at p_end holds rows of a segment after s.
__device__ __forceinline__ bool more_segments(const Params& P, const Seg& s, long long p_end) {
  return s.off + cost_len(P, s.len) + P.seg_cost < p_end;
}

// Clamped length of sequence b (b uniform): from the wave's length register
// for batches <= 64 (lane b holds it), else through the scalar path.
__device__ __forceinline__ int seq_len_of(const Params& P, int lens_v, int b) {
  return P.wave_planner ? __builtin_amdgcn_readlane(lens_v, b)
                       : seq_len_uniform(P.seq_lens, b, P.capacity);
}

// Advance to the next segment (next KV head of b, else the next non-empty
// sequence). Only called while rows remain below p_end, so one exists.
// kBases: also set the block offsets (the tile walk; the segment walk of the
// merges needs only b and g).
template <int F, bool kPaged, bool kBases>
__device__ __forceinline__ void seg_next(const Params& P, Seg& s, long long p_end, int lens_v) {
  const long long end = s.off + cost_len(P, s.len) + P.seg_cost;
  if (s.g + 1 < P.kv_heads) {
    s.g += 1;
  } else {
    int nb = s.b + 1;
    int nl = seq_len_of(P, lens_v, nb);
    while (nl == 0) {
      ++nb;
      nl = seq_len_of(P, lens_v, nb);
    }
    s.b = nb;
    s.len = nl;
    s.g = 0;
  }
  s.off = end;
  seg_set_range(s, end, p_end);
  if constexpr (kBases) seg_bases<F, kPaged>(P, s);
}

// Move (s, t) to this wave's next tile in the piece: the next 16-row tile of
// the wave in s, else its first tile in a later segment. Returns false when
// the piece has no more tiles for this wave.
template <int F, bool kPaged>
__device__ __forceinline__ bool tile_next(const Params& P, Seg& s, int& t, long long p_end, int wv,
                                          int lens_v) {
  t += kWaves * tile_rows<F>();
  while (t >= s.hi) {
    if (!more_segments(P, s, p_end)) return false;
    seg_next<F, kPaged, true>(P, s, p_end, lens_v);
    t = s.lo + tile_rows<F>() * wv;
  }
  return true;
}

// First tile of this wave at or after (s, t) (t = s.lo + kRows * wv).
template <int F, bool kPaged>
__device__ __forceinline__ bool tile_first(const Params& P, Seg& s, int& t, long long p_end, int wv,
                                           int lens_v) {
  while (t >= s.hi) {
    if (!more_segments(P, s, p_end)) return false;
    seg_next<F, kPaged, true>(P, s, p_end, lens_v);
    t = s.lo + tile_rows<F>() * wv;
  }
  return true;
}

// 16-byte chunk c of row r of an E4M3 tile sits at chunk c ^ swz8(r) of the
// row in LDS, so the K reads (16 rows apart by 128 B) and the transposed V
// reads (rows r and r + 16 together) spread over the banks.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1) ^ (((r >> 4) & 1) << 2); }

// 16-byte chunk c of row r of an FP4 tile (64-byte rows) sits at chunk
// c ^ sw4(r): 8 consecutive rows read at one logical chunk (the K reads)
// then hit 8 different 16-byte bank groups of a 128-byte line.
__device__ __forceinline__ int sw4(int r) { return (r >> 1) & 3; }

// Buffer resource over rows [row0, row0 + nrows) of one K or V block that
// starts at `base` (row stride sr bytes); rows past nrows read as zeros.
// Offsets inside a block fit 31 bits (the host keeps row stride x capacity,
// or x page size, below 2^31), so they are formed in 32-bit arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const char* base, int row0, int nrows,
                                                            long long sr) {
  const int sr32 = (int)sr;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (unsigned)(row0 * sr32)), 0,
                                           nrows > 0 ? nrows * sr32 : 0, kBufferFlags);
}

// Page holding row i of the segment's sequence (paged caches; btr = that
// sequence's block-table row): the page id, or -1 if it is outside [0,
// num_pages) (its rows then read as zeros instead of faulting). Uniform:
// one scalar load.
__device__ __forceinline__ int page_id(const Params& P,
                                       const __attribute__((address_space(4))) int32_t* btr,
                                       int i) {
  const int page = btr[(unsigned)i >> P.page_shift];
  return (unsigned)page < (unsigned)P.num_pages ? page : -1;
}

// Byte offsets of the pages holding rows t and t + 16 of a tile of segment
// s (-1: no rows there, or an invalid page id), and for FP4 caches the
// offset of the scale page of row t (FP4 tiles lie in one page: pages and
// pieces are multiples of 32 rows). Unused for contiguous caches.
struct PageBases {
  long long p0 = -1, p1 = -1, s0 = -1;
};

template <int F>
__device__ __forceinline__ PageBases page_bases(const Params& P, const Seg& s, int t, bool live) {
  PageBases pb;
  const int nrows = live ? s.hi - t : 0;
  if (nrows > 0) {
    const int id = page_id(P, s.btr, t);
    if (id >= 0) {
      pb.p0 = (long long)id * P.kv_sb;
      if constexpr (F == kFmtFp4) pb.s0 = (long long)id * P.sc_sb;
    }
  }
  if constexpr (F == kFmtE4m3) {
    if (nrows > 16) {
      const int id = page_id(P, s.btr, t + 16);
      if (id >= 0) pb.p1 = (long long)id * P.kv_sb;
    }
  }
  return pb;
}

// Issue the loads of this wave's tile of segment s (rows [t, t + rows)) into
// an LDS stage (K, then V) and the segment's G query rows into the wave's q
// slot, in this order: q (1 load, or 2 in the general form), 4 x K, 4 x V
// (FP4: 2 x K codes, K scales, 2 x V codes, V scales).
// Rows at or past s.hi read as zeros. With live == false the buffers are
// empty: the same loads return zeros without touching memory, so every
// pipeline step has the same shape. The q load is live only for a wave's
// first tile of a segment (live_q); later tiles reuse the q registers, and
// their empty q load leaves zeros in the slot. Each K/V load moves 1 KiB:
// 4 rows of 256 B (16-bit formats), 8 rows of 128 B (E4M3) or 16 rows of
// 64 B (FP4 codes). In LDS the rows are dense whatever the strides.
// Paged caches (page size a multiple of 16): each 16-row half of a tile
// lies in one page, whose offset the caller passes in pb (FP4: the whole
// 32-row tile, pages and pieces being multiples of 32 rows).
template <int F, bool kPaged, bool kG4>
__device__ __forceinline__ void issue_tile(const Params& P, const Seg& s, int t, bool live,
                                           bool live_q, e16_t* stage, e16_t* qslot,
                                           const PageBases& pb) {
  constexpr int kRowBytes = row_bytes<F>();
  constexpr int kRows = tile_rows<F>();
  const int lane = threadIdx.x & 63;
  const int group = group_of<kG4>(P);
  const char* qg = reinterpret_cast<const char*>(P.q) + s.qo;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      (void*)qg, 0, live && live_q ? (int)((group - 1) * P.q_sh + 2 * kDim) : 0, kBufferFlags);
  // q: load u (one, or two in the general form) gives lane l 16 B of the
  // group's query row 4u + l/16, chunk l%16; rows at or past G lie beyond
  // the resource (or are masked when q rows overlap) and read as zeros.
#pragma unroll
  for (int u = 0; u < (kG4 ? 1 : 2); ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rq, (lds_void_t*)(reinterpret_cast<char*>(qslot) + 1024 * u), 16,
        (int)((4 * u + (lane >> 4)) * P.q_sh) + 16 * (lane & 15), 0, 0, 0);
  const int nrows = live ? s.hi - t : 0;          // rows of this tile below s.hi
  // DMA lane l writes 16 B at LDS offset 16*l of the 1 KiB block u: for
  // 16-bit formats row 4u + l/16, physical chunk l%16, which holds logical
  // chunk vchunk(row, l%16); for E4M3 row 8u + l/8, physical chunk l%8,
  // holding logical chunk (l%8) ^ swz8(row). Both swizzles are their own
  // inverse.
  char* st = reinterpret_cast<char*>(stage);
  if constexpr (F == kFmtFp4) {
    // Codes: load u gives lane l row 16u + l/4, physical 16-byte chunk l%4,
    // which holds logical chunk (l%4) ^ sw4(row). Scales: one 4-byte load
    // per lane, lane l taking bytes 4(l%2) .. +3 of row l/2, so the tile's
    // 32 x 8 scale bytes land densely, row by row.
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {
      __amdgpu_buffer_rsrc_t rc, rs;
      if constexpr (kPaged) {
        const int psz_mask = (1 << P.page_shift) - 1;
        const char* blk = reinterpret_cast<const char*>(P.kv) + kind * P.kv_sk + s.kvo;
        const char* sblk = reinterpret_cast<const char*>(P.kv_scales) + kind * P.sc_sk + s.sco;
        const int n = pb.p0 < 0 ? 0 : (nrows < 32 ? nrows : 32);   // the tile's rows, one page
        rc = rows_rsrc(blk + (pb.p0 < 0 ? 0 : pb.p0), t & psz_mask, n, P.kv_sr);
        rs = rows_rsrc(sblk + (pb.s0 < 0 ? 0 : pb.s0), t & psz_mask, n, P.sc_sr);
      } else {
        rc = rows_rsrc(reinterpret_cast<const char*>(P.kv) + s.kvo + kind * P.kv_sk, t, nrows,
                       P.kv_sr);
        rs = rows_rsrc(reinterpret_cast<const char*>(P.kv_scales) + s.sco + kind * P.sc_sk, t,
                       nrows, P.sc_sr);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = 16 * u + (lane >> 2);
        const int c = (lane & 3) ^ sw4(r);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rc, (lds_void_t*)(st + kind * kind_bytes<F>() + u * 1024), 16,
            (int)(r * P.kv_sr) + 16 * c, 0, 0, kNonTemporal);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void_t*)(st + scale_offset<F>() + kind * 32 * kFp4ScaleBytes), 4,
          (int)((lane >> 1) * P.sc_sr) + 4 * (lane & 1), 0, 0, kNonTemporal);
    }
    return;
  }
  // Paged: pb holds the byte offsets of the pages of rows t and t + 16.
  const long long pb0 = pb.p0, pb1 = pb.p1;
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {
    __amdgpu_buffer_rsrc_t r0, r1;   // rows [0, 16) and [16, 32) of the tile
    if constexpr (kPaged) {
      const char* blk = reinterpret_cast<const char*>(P.kv) + kind * P.kv_sk + s.kvo;
      const int psz_mask = (1 << P.page_shift) - 1;
      r0 = rows_rsrc(blk + (pb0 < 0 ? 0 : pb0), t & psz_mask, pb0 < 0 ? 0 : (nrows < 16 ? nrows : 16),
                     P.kv_sr);
      r1 = r0;
      if constexpr (kRows == 32)
        r1 = rows_rsrc(blk + (pb1 < 0 ? 0 : pb1), (t + 16) & psz_mask,
                       pb1 < 0 ? 0 : (nrows - 16 < 16 ? nrows - 16 : 16), P.kv_sr);
    } else {
      const char* blk = reinterpret_cast<const char*>(P.kv) + s.kvo + kind * P.kv_sk;
      r0 = rows_rsrc(blk, t, nrows, P.kv_sr);
      r1 = r0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int r, c;
      if constexpr (F == kFmtE4m3) {
        r = 8 * u + (lane >> 3);
        c = (lane & 7) ^ swz8(r);
      } else {
        r = 4 * u + (lane >> 4);
        c = vchunk(r, lane & 15);
      }
      // in paged mode the second half of an E4M3 tile has its own resource
      const bool second = kPaged && kRows == 32 && u >= 2;
      const int off = (int)((second ? r - 16 : r) * P.kv_sr) + 16 * c;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? r1 : r0,
                                               (lds_void_t*)(st + kind * 4096 + u * 1024), 16,
                                               off, 0, 0, kNonTemporal);
    }
  }
}

__device__ __forceinline__ unsigned lds_addr(const e16_t* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const e16_t*)p;
}

struct WaveAcc {
  float4_t O[8];     // O^T accumulators (D layout): lane (G4, j), reg r = head j,
                     // output column 16 db + 4 G4 + r
  float m;           // head j's weight reference (weight_ref: the running max,
                     // or 15 below it for fp16 weights; same in the 4 lane groups)
  float l;           // this lane group's share of head j's denominator
};

// q^T as the QK B operand, read from the wave's q slot: lane (G4, j) takes
// head j, depth 32kk + 8 G4 .. +7 (FP4 caches: depth 32 G4 + 8kk .. +7, the
// order in which a lane's FP4 K bytes hold the depth; a dot product does
// not depend on the order of its terms); columns j >= G are zero.
template <bool kG4, int F>
__device__ __forceinline__ void read_q(const e16_t* qslot, int group, uint4_t (&qb)[4]) {
  const int lane = threadIdx.x & 63, G = lane >> 4, j = lane & 15;
  int row = j & (kG4 ? 3 : 7);
  asm volatile("" : "+v"(row));
  constexpr bool kFp4 = F == kFmtFp4;
  const unsigned base = lds_addr(qslot) + 2 * (row * kDim + (kFp4 ? 32 : 8) * G);
  uint4_t x0, x1, x2, x3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:%5\n\t"
      "ds_read_b128 %2, %4 offset:%6\n\t"
      "ds_read_b128 %3, %4 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
      : "v"(base), "n"(kFp4 ? 16 : 64), "n"(kFp4 ? 32 : 128), "n"(kFp4 ? 48 : 192)
      : "memory");
  const uint4_t zero = {0u, 0u, 0u, 0u};
  qb[0] = j < group ? x0 : zero;
  qb[1] = j < group ? x1 : zero;
  qb[2] = j < group ? x2 : zero;
  qb[3] = j < group ? x3 : zero;
}

// LDS addresses of this lane's operand reads in stage 0 of its wave; stage 1
// lies stage_bytes<F>() higher (an immediate offset of the reads).
//   16-bit formats: k[kk] = row j, logical chunk 4kk + G (16 B); v[db] =
//   transposed read of row 4G + j/4, columns 16db + 4(j%4) .. +3.
//   E4M3: k[4h + kk] = row 16h + j, bytes 32kk + 8G .. +7; v[db] =
//   transposed read of row rowE(G, j/2), bytes 16db + 8(j%2) .. +7, where
//   rowE(G, e) = 4G + e for e < 4 and 16 + 4G + e - 4 for e >= 4.
//   FP4: k[h] = row 16h + j, logical chunk G (16 B: depth 32G .. 32G + 31);
//   k[2 + h] = the 2 scale bytes of that row for depth blocks 2G, 2G + 1;
//   v[rd] = transposed 4-bit read: lane (G, i) addresses row rowE(G, i % 8),
//   half i / 8 of logical chunk rd (columns 32rd + 16(i/8) .. +15);
//   v[4] = the V scales of rows 4G .. 4G + 3 (16 + 4G .. at +128).
struct LdsReads {
  unsigned k[8];
  unsigned v[8];
};

template <int F>
__device__ __forceinline__ LdsReads lds_reads(const e16_t* stage0) {
  const int lane = threadIdx.x & 63, G = lane >> 4, j = lane & 15;
  const unsigned kbase = lds_addr(stage0);
  const unsigned vbase = kbase + kind_bytes<F>();
  LdsReads r;
  if constexpr (F == kFmtFp4) {
    const unsigned sbase = kbase + scale_offset<F>();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 16 * h + j;
      r.k[h] = kbase + row * (kDim / 2) + 16 * (G ^ sw4(row));
      r.k[2 + h] = sbase + row * kFp4ScaleBytes + 2 * G;
    }
    // Transposed 4-bit reads (lane mapping measured on the hardware): within
    // each 16-lane group, output lane i receives, as its nibble e (e = 0..15,
    // low nibbles first), nibble i of the 8-byte chunk addressed by lane e.
    // Lanes e < 8 address row rowE(G, e), columns 32rd .. +15; lanes e >= 8
    // the same rows, columns 32rd + 16 .. +31. So lane (G, i) receives
    // column 32rd + i of rows rowE(G, 0..7) in its first dword and column
    // 32rd + 16 + i of the same rows in its second: the A operands (V^T) of
    // two K = 32 MFMAs.
    const int e = j & 7;
    const int row = e < 4 ? 4 * G + e : 16 + 4 * G + (e - 4);
#pragma unroll
    for (int rd = 0; rd < 4; ++rd)
      r.v[rd] = vbase + row * (kDim / 2) + 16 * (rd ^ sw4(row)) + 8 * (j >> 3);
    // V scales, converted once per wave (fp4_v_scales): lane (rp, dq) =
    // (lane / 4, lane % 4) reads the scale dword (blocks 4(dq / 2) .. +3) of
    // rows 2rp and 2rp + 1.
    r.v[4] = sbase + 32 * kFp4ScaleBytes + (lane >> 2) * 2 * kFp4ScaleBytes + 4 * ((lane & 3) >> 1);
#pragma unroll
    for (int i = 5; i < 8; ++i) r.v[i] = 0;
#pragma unroll
    for (int i = 4; i < 8; ++i) r.k[i] = 0;
  } else if constexpr (F == kFmtE4m3) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int row = 16 * h + j;
        r.k[4 * h + kk] = kbase + row * kDim + 16 * ((2 * kk + (G >> 1)) ^ swz8(row)) + 8 * (G & 1);
      }
    }
    // Transposed 8-bit reads (lane mapping measured on the hardware): within
    // each 16-lane group, output lane i receives byte i % 8 of the 8-byte
    // chunks addressed by lanes i/8 + 2e, e = 0..7. Lane (G, j) addresses
    // row rowE(G, j/2), columns 16db + 8(j%2) .. +7, so it receives column
    // 16db + j of rows rowE(G, 0..7): the B operand of a K = 32 MFMA.
    const int e = j >> 1;
    const int row = e < 4 ? 4 * G + e : 16 + 4 * G + (e - 4);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      r.v[db] = vbase + row * kDim + 16 * (db ^ swz8(row)) + 8 * (j & 1);
  } else {
    const int rr = 4 * G + (j >> 2);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) r.k[kk] = kbase + 2 * (j * kDim + 8 * vchunk(j, 4 * kk + G));
    // Transposed reads: lane (G, j) supplies the address of row 4G + j/4,
    // columns 16*db + 4*(j%4) .. +3 and receives column 16*db + j of rows
    // 4G .. 4G+3.
#pragma unroll
    for (int db = 0; db < 8; ++db)
      r.v[db] = vbase + 2 * (rr * kDim + 8 * vchunk(rr, 2 * db + ((j & 3) >> 1)) + 4 * (j & 1));
  }
  return r;
}

// Read the K and V operands of one stage (byte offset OFF from stage 0).
template <int OFF>
__device__ __forceinline__ void read_stage(const LdsReads& a, uint4_t (&k)[4], short4_t (&v)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12 offset:%24\n\t"
      "ds_read_b128 %1, %13 offset:%24\n\t"
      "ds_read_b128 %2, %14 offset:%24\n\t"
      "ds_read_b128 %3, %15 offset:%24\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %10, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %11, %23 offset:%24\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]),
        "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a.k[0]), "v"(a.k[1]), "v"(a.k[2]), "v"(a.k[3]), "v"(a.v[0]), "v"(a.v[1]),
        "v"(a.v[2]), "v"(a.v[3]), "v"(a.v[4]), "v"(a.v[5]), "v"(a.v[6]), "v"(a.v[7]), "n"(OFF)
      : "memory");
}

// Read the E4M3 K and V operands of one stage (byte offset OFF from stage 0).
template <int OFF>
__device__ __forceinline__ void read_stage8(const LdsReads& a, uint2 (&k)[8], uint2 (&v)[8]) {
  asm volatile(
      "ds_read_b64 %0, %16 offset:%32\n\t"
      "ds_read_b64 %1, %17 offset:%32\n\t"
      "ds_read_b64 %2, %18 offset:%32\n\t"
      "ds_read_b64 %3, %19 offset:%32\n\t"
      "ds_read_b64 %4, %20 offset:%32\n\t"
      "ds_read_b64 %5, %21 offset:%32\n\t"
      "ds_read_b64 %6, %22 offset:%32\n\t"
      "ds_read_b64 %7, %23 offset:%32\n\t"
      "ds_read_b64_tr_b8 %8, %24 offset:%32\n\t"
      "ds_read_b64_tr_b8 %9, %25 offset:%32\n\t"
      "ds_read_b64_tr_b8 %10, %26 offset:%32\n\t"
      "ds_read_b64_tr_b8 %11, %27 offset:%32\n\t"
      "ds_read_b64_tr_b8 %12, %28 offset:%32\n\t"
      "ds_read_b64_tr_b8 %13, %29 offset:%32\n\t"
      "ds_read_b64_tr_b8 %14, %30 offset:%32\n\t"
      "ds_read_b64_tr_b8 %15, %31 offset:%32\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
        "=&v"(k[6]), "=&v"(k[7]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
        "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a.k[0]), "v"(a.k[1]), "v"(a.k[2]), "v"(a.k[3]), "v"(a.k[4]), "v"(a.k[5]),
        "v"(a.k[6]), "v"(a.k[7]), "v"(a.v[0]), "v"(a.v[1]), "v"(a.v[2]), "v"(a.v[3]),
        "v"(a.v[4]), "v"(a.v[5]), "v"(a.v[6]), "v"(a.v[7]), "n"(OFF)
      : "memory");
}

// Eight E4M3 bytes (two dwords, byte 0 first) as eight fp16 values. Every
// E4M3 value is an fp16 value, so the conversion is exact; its results were
// checked on the hardware against the format's definition for all 256 codes.
__device__ __forceinline__ half8_t e4m3x8_to_f16(uint2 x) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.x, 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.x, 1.0f, true);
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.y, 1.0f, false);
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x.y, 1.0f, true);
  return (half8_t){a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Reference point of a tile's softmax weights (base 2): the weights are
// exp2(s - ref). The wave state, the wave merge and the partials carry this
// reference in place of the running maximum; any reference gives the same
// normalised result, since numerator and denominator share the factor
// exp2(max - ref). kBias (fp16 weight pairs): ref lies 15 below the running
// maximum, so weights reach 2^15 and their fp16 low parts stay normal down
// to 2^-18 of the largest (see split_weight). The bias is taken only while
// |mx| < 2^20, where the fp32 rounding of mx - 15 is at most 2^-4, so no
// weight exceeds 2^15.07 < 65504 (the fp16 maximum); beyond that the score
// magnitudes already carry fp32 rounding errors far above the split's.
// The reference never decreases (fmaxf), so rescale factors stay <= 1.
template <bool kBias>
__device__ __forceinline__ float weight_ref(float ref_old, float mx) {
  if constexpr (!kBias) return fmaxf(ref_old, mx);
  const float bias = __builtin_fabsf(mx) < 1048576.0f ? 15.0f : 0.0f;
  return fmaxf(ref_old, mx - bias);
}

// Element-type specific steps: MFMAs on fp16 or bf16 operands (raw 16-bit
// patterns in registers), the two-part rounding of the softmax weights, and
// the round-to-nearest-even output conversion.
template <bool kBf16>
__device__ __forceinline__ float4_t mfma_qk(uint4_t a, uint4_t b, float4_t c) {
  if constexpr (kBf16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

template <bool kBf16>
__device__ __forceinline__ float4_t mfma_pv(short4_t a, short4_t b, float4_t c) {
  if constexpr (kBf16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, a),
                                                 __builtin_bit_cast(half4_t, b), c, 0, 0, 0);
}

// p = hi + lo with hi = p rounded to the element type and lo = the rest,
// rounded again. bf16 (8 exponent bits): the pair carries 16 significant
// bits for any weight. fp16: hi carries 11 bits and lo 11 more while lo is a
// normal fp16 number, i.e. for p >= 2^-3; below that lo lies in fp16's
// subnormal range, whose fixed spacing 2^-24 bounds the pair's absolute
// error by 2^-25. fp16 weights are therefore formed up to 2^15 rather than
// up to 1 (weight_ref): the pair then has 22 bits for weights down to 2^-18
// of the largest, and an absolute error of at most 2^-40 of the largest
// below that.
template <bool kBf16>
__device__ __forceinline__ void split_weight(float p, short& hi, short& lo) {
  if constexpr (kBf16) {
    const __bf16 h = (__bf16)p;
    hi = __builtin_bit_cast(short, h);
    lo = __builtin_bit_cast(short, (__bf16)(p - (float)h));
  } else {
    const _Float16 h = (_Float16)p;
    hi = __builtin_bit_cast(short, h);
    lo = __builtin_bit_cast(short, (_Float16)(p - (float)h));
  }
}

// fp16 split of two weights at once: hi = (p0, p1) rounded to fp16, lo =
// (p - hi) rounded again, the same bits as split_weight<false> on each. p - hi
// is exact in fp32, so a fused multiply-add with mixed operands (hi as fp16,
// p as fp32) rounds it once: one instruction per lo half (v_fma_mixlo_f16 and
// v_fma_mixhi_f16 write the low and the high half) instead of a conversion
// back to fp32, a subtraction and a conversion.
__device__ __forceinline__ void split_weight_pair(float p0, float p1, unsigned& hi,
                                                  unsigned& lo) {
  const half2_t h = {(_Float16)p0, (_Float16)p1};
  hi = __builtin_bit_cast(unsigned, h);
  unsigned l;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(l)
      : "v"(hi), "v"(p0), "v"(p1));
  lo = l;
}

// Weights p[0..7] of an 8-row K = 32 operand as fp16 hi and lo parts.
__device__ __forceinline__ void split_weights8(const float (&p)[8], half8_t& ph, half8_t& pl) {
  unsigned h0, h1, h2, h3, l0, l1, l2, l3;
  split_weight_pair(p[0], p[1], h0, l0);
  split_weight_pair(p[2], p[3], h1, l1);
  split_weight_pair(p[4], p[5], h2, l2);
  split_weight_pair(p[6], p[7], h3, l3);
  ph = __builtin_bit_cast(half8_t, ((uint4_t){h0, h1, h2, h3}));
  pl = __builtin_bit_cast(half8_t, ((uint4_t){l0, l1, l2, l3}));
}

template <bool kBf16>
__device__ __forceinline__ e16_t to_elem(float x) {
  if constexpr (kBf16)
    return __builtin_bit_cast(e16_t, (__bf16)x);
  else
    return __builtin_bit_cast(e16_t, (_Float16)x);
}

// Read the FP4 operands of one stage (byte offset OFF from stage 0): K codes
// (2 x 16 B), K scales (2 x 2 B), V codes transposed (4 x 8 B) and one V
// scale dword of each of two rows (the lane's share of the conversion in
// fp4_v_scales).
template <int OFF>
__device__ __forceinline__ void read_stage_fp4(const LdsReads& a, uint4_t (&k)[2],
                                               unsigned (&ks)[2], uint2 (&v)[4], uint2& vs) {
  asm volatile(
      "ds_read_b128 %0, %10 offset:%17\n\t"
      "ds_read_b128 %1, %11 offset:%17\n\t"
      "ds_read_u16 %2, %12 offset:%17\n\t"
      "ds_read_u16 %3, %13 offset:%17\n\t"
      "ds_read_b64_tr_b4 %4, %14 offset:%17\n\t"
      "ds_read_b64_tr_b4 %5, %15 offset:%17\n\t"
      "ds_read_b64_tr_b4 %6, %16 offset:%17\n\t"
      "ds_read_b64_tr_b4 %7, %18 offset:%17\n\t"
      "ds_read_b32 %8, %19 offset:%17\n\t"
      "ds_read_b32 %9, %19 offset:%20\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(ks[0]), "=&v"(ks[1]), "=&v"(v[0]), "=&v"(v[1]),
        "=&v"(v[2]), "=&v"(v[3]), "=&v"(vs.x), "=&v"(vs.y)
      : "v"(a.k[0]), "v"(a.k[1]), "v"(a.k[2]), "v"(a.k[3]), "v"(a.v[0]), "v"(a.v[1]),
        "v"(a.v[2]), "n"(OFF), "v"(a.v[3]), "v"(a.v[4]), "n"(OFF + kFp4ScaleBytes)
      : "memory");
}

// Two E4M3 codes (bytes 0, 1 of the low or high half of x) as an fp16 pair,
// exactly (every E4M3 value is an fp16 value).
template <bool kHigh>
__device__ __forceinline__ half2_t e4m3x2_to_f16(unsigned x) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, kHigh);
}

// Eight FP4 E2M1 codes (one dword, element 2m in the low nibble of byte m) as
// fp16 values, elements 2m and 2m + 1 multiplied by the pair s[m]. The
// conversion runs at scale 1 (the conversion's own scale operand takes only
// a power of two: measured on the hardware); each product of an E2M1 value
// (at most 2 significant bits, |x| <= 6) and an E4M3 scale (at most 4 bits,
// 2^-9 <= |s| <= 448, or 0) is an fp16 value, so the multiply is exact.
__device__ __forceinline__ half8_t fp4x8_to_f16(unsigned x, half2_t s0, half2_t s1, half2_t s2,
                                                half2_t s3) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s0;
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s1;
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s2;
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s3;
  return (half8_t){a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// The V block scales of an FP4 tile as fp16 pairs, converted once per wave
// rather than by each of the 16 lanes that use them. Lane (rp, dq) = (lane /
// 4, lane % 4) holds, in vraw, the scale dword (blocks 4(dq / 2) .. +3) of
// rows 2rp (x) and 2rp + 1 (y); one byte permute pairs the two rows' scales
// of blocks 2dq and 2dq + 1, two conversions give (s[2rp][b], s[2rp + 1][b])
// for b = 2dq, 2dq + 1, stored as entry 4rp + dq = lane of the wave's
// 64-entry area. The PV operands pair exactly these rows.
__device__ __forceinline__ void fp4_v_scales(uint2 vraw, uint2* vsh) {
  const int lane = threadIdx.x & 63;
  const unsigned c = 2u * ((unsigned)lane & 1u);   // byte of block 2dq in its dword
  const unsigned sel = c | ((4u + c) << 8) | ((c + 1u) << 16) | ((5u + c) << 24);
  const unsigned w = __builtin_amdgcn_perm(vraw.y, vraw.x, sel);
  vsh[lane] = make_uint2(__builtin_bit_cast(unsigned, e4m3x2_to_f16<false>(w)),
                         __builtin_bit_cast(unsigned, e4m3x2_to_f16<true>(w)));
}

// Fold tile rows [t, t + 32) of an FP4 tile held in LDS stage `par` into
// acc. K: lane (G, j) holds depth 32G .. 32G + 31 of row 16h + j (q is read
// in the same depth order); each depth block of 16 has its own scale. QK
// runs as two 16-row halves, so lane (G, j) ends with the scores of rows
// rowE(G, 0..7) for head j, the B layout of a K = 32 PV MFMA. V: the
// transposed reads give lane (G, i) column c of rows rowE(G, 0..7); each of
// those rows has its own scale for c's block, applied per element pair.
__device__ __forceinline__ void compute_tile_fp4(const LdsReads& la, int par,
                                                 const uint4_t (&qb)[4], int t, int hi,
                                                 float scale_log2, uint2* vsh, WaveAcc& acc) {
  const int lane = threadIdx.x & 63, G = lane >> 4;
  const float kNegInf = -__builtin_inff();
  uint4_t kd[2];
  unsigned ks[2];
  uint2 vt[4];
  uint2 vraw;
  if (par)
    read_stage_fp4<stage_bytes<kFmtFp4>()>(la, kd, ks, vt, vraw);
  else
    read_stage_fp4<0>(la, kd, ks, vt, vraw);
  fp4_v_scales(vraw, vsh);

  float4_t sc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const half2_t s2 = e4m3x2_to_f16<false>(ks[h]);   // blocks 2G, 2G + 1 of row 16h + j
    const half2_t sa = {s2.x, s2.x}, sb = {s2.y, s2.y};
    sc[h] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const half2_t sp = kk < 2 ? sa : sb;
      sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fp4x8_to_f16(kd[h][kk], sp, sp, sp, sp),
                                                     __builtin_bit_cast(half8_t, qb[kk]), sc[h],
                                                     0, 0, 0);
    }
  }

  float sv[8];
  if (t + 32 <= hi) {                    // the whole tile is in range (wave-uniform)
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = sc[e >> 2][e & 3] * scale_log2;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = (e < 4 ? 0 : 16) + 4 * G + (e & 3);
      sv[e] = (t + row) < hi ? sc[e >> 2][e & 3] * scale_log2 : kNegInf;
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[e]);
  mx = max_over_row_groups(mx);
  // Row t is below hi, so mx (and m_new) is finite; alpha is 0 on the first
  // tile, where acc.m is still -inf. acc.m holds the weights' reference.
  const float m_new = weight_ref<true>(acc.m, mx);
  const float alpha = exp2_hw(acc.m - m_new);
  acc.m = m_new;

  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2_hw(sv[e] - m_new);               // 0 for rows out of range (score -inf)
    psum += p[e];
  }
  half8_t ph, pl;
  split_weights8(p, ph, pl);
  acc.l = acc.l * alpha + psum;

  // alpha is exactly 1 in every lane once no running maximum grows; the
  // rescale is then an identity and is skipped (a wave-uniform test).
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int db = 0; db < 8; ++db) acc.O[db] *= alpha;
  }
  // V scales as fp16 pairs (fp4_v_scales): entry 4rp + k holds those of
  // rows 2rp, 2rp + 1 for blocks 2k (x) and 2k + 1 (y); the lane's local rows
  // 2m, 2m + 1 are the row pair rp = 2G + m (m < 2) or 8 + 2G + (m - 2).
  uint2 sp[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int rp = (m < 2 ? 2 * G : 8 + 2 * G) + (m & 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) sp[m][k] = vsh[4 * rp + k];
  }
#pragma unroll
  for (int rd = 0; rd < 4; ++rd) {
    const int db = 2 * rd;
    half2_t p0[4], p1[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      p0[m] = __builtin_bit_cast(half2_t, sp[m][rd].x);
      p1[m] = __builtin_bit_cast(half2_t, sp[m][rd].y);
    }
    const half8_t va0 = fp4x8_to_f16(vt[rd].x, p0[0], p0[1], p0[2], p0[3]);
    const half8_t va1 = fp4x8_to_f16(vt[rd].y, p1[0], p1[1], p1[2], p1[3]);
    acc.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va0, ph, acc.O[db], 0, 0, 0);
    acc.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va0, pl, acc.O[db], 0, 0, 0);
    acc.O[db + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va1, ph, acc.O[db + 1], 0, 0, 0);
    acc.O[db + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va1, pl, acc.O[db + 1], 0, 0, 0);
  }
}

// Fold tile rows [t, t + 32) of an E4M3 tile held in LDS stage `par` into
// acc. QK runs as two 16-row halves on the fp16 MFMA (K converted exactly);
// lane (G, j) then holds the scores of rows 4G .. 4G+3 and 16 + 4G .. +3
// for head j: in the order rowE(G, 0..7), which is the A layout of a K = 32
// PV MFMA, matching the V operand read above.
__device__ __forceinline__ void compute_tile8(const LdsReads& la, int par, const uint4_t (&qb)[4],
                                              int t, int hi, float scale_log2, WaveAcc& acc) {
  const int lane = threadIdx.x & 63, G = lane >> 4;
  const float kNegInf = -__builtin_inff();
  uint2 kr[8], vr[8];
  if (par)
    read_stage8<stage_bytes<kFmtE4m3>()>(la, kr, vr);
  else
    read_stage8<0>(la, kr, vr);

  float4_t sc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    sc[h] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16(kr[4 * h + kk]),
                                                     __builtin_bit_cast(half8_t, qb[kk]), sc[h],
                                                     0, 0, 0);
  }

  float sv[8];
  if (t + 32 <= hi) {                    // the whole tile is in range (wave-uniform)
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = sc[e >> 2][e & 3] * scale_log2;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = (e < 4 ? 0 : 16) + 4 * G + (e & 3);
      sv[e] = (t + row) < hi ? sc[e >> 2][e & 3] * scale_log2 : kNegInf;
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[e]);
  mx = max_over_row_groups(mx);
  // Row t is below hi, so mx (and m_new) is finite; alpha is 0 on the first
  // tile, where acc.m is still -inf. acc.m holds the weights' reference.
  const float m_new = weight_ref<true>(acc.m, mx);
  const float alpha = exp2_hw(acc.m - m_new);
  acc.m = m_new;

  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2_hw(sv[e] - m_new);               // 0 for rows out of range (score -inf)
    psum += p[e];
  }
  half8_t ph, pl;
  split_weights8(p, ph, pl);
  acc.l = acc.l * alpha + psum;

  // O^T = V^T P^T: every accumulator of this lane belongs to head j.
  // alpha is exactly 1 in every lane once no running maximum grows; the
  // rescale is then an identity and is skipped (a wave-uniform test).
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int db = 0; db < 8; ++db) acc.O[db] *= alpha;
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const half8_t va = e4m3x8_to_f16(vr[db]);
    acc.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, acc.O[db], 0, 0, 0);
    acc.O[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl, acc.O[db], 0, 0, 0);
  }
}

// Fold tile rows [t, t + 16) held in LDS stage `par` into acc (fp16 or bf16).
template <bool kBf16>
__device__ __forceinline__ void compute_tile(const LdsReads& la, int par, const uint4_t (&qb)[4],
                                             int t, int hi, float scale_log2, WaveAcc& acc) {
  const int lane = threadIdx.x & 63, G = lane >> 4;
  const float kNegInf = -__builtin_inff();
  uint4_t kr[4];
  short4_t vr[8];
  if (par)
    read_stage<stage_bytes<kFmtF16>()>(la, kr, vr);
  else
    read_stage<0>(la, kr, vr);
  const uint4_t k0 = kr[0], k1 = kr[1], k2 = kr[2], k3 = kr[3];
  const short4_t v0 = vr[0], v1 = vr[1], v2 = vr[2], v3 = vr[3], v4 = vr[4], v5 = vr[5],
                 v6 = vr[6], v7 = vr[7];

  float4_t sc = {0.f, 0.f, 0.f, 0.f};
  sc = mfma_qk<kBf16>(k0, qb[0], sc);
  sc = mfma_qk<kBf16>(k1, qb[1], sc);
  sc = mfma_qk<kBf16>(k2, qb[2], sc);
  sc = mfma_qk<kBf16>(k3, qb[3], sc);

  float sv[4];
  if (t + 16 <= hi) {                    // the whole tile is in range (wave-uniform)
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = sc[r] * scale_log2;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = (t + 4 * G + r) < hi ? sc[r] * scale_log2 : kNegInf;
  }
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sv[r]);
  mx = max_over_row_groups(mx);
  // Row t is below hi, so mx (and m_new) is finite; alpha is 0 on the first
  // tile, where acc.m is still -inf. acc.m holds the weights' reference.
  const float m_new = weight_ref<!kBf16>(acc.m, mx);
  const float alpha = exp2_hw(acc.m - m_new);
  acc.m = m_new;

  float p[4];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = exp2_hw(sv[r] - m_new);               // 0 for rows out of range (score -inf)
    psum += p[r];
  }
  short4_t ph, pl;
  if constexpr (kBf16) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      short h, l;
      split_weight<true>(p[r], h, l);
      ph[r] = h;
      pl[r] = l;
    }
  } else {
    unsigned h0, h1, l0, l1;
    split_weight_pair(p[0], p[1], h0, l0);
    split_weight_pair(p[2], p[3], h1, l1);
    ph = __builtin_bit_cast(short4_t, make_uint2(h0, h1));
    pl = __builtin_bit_cast(short4_t, make_uint2(l0, l1));
  }
  acc.l = acc.l * alpha + psum;

  // O^T = V^T P^T: every accumulator of this lane belongs to head j.
  // alpha is exactly 1 in every lane once no running maximum grows; the
  // rescale is then an identity and is skipped (a wave-uniform test).
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
    for (int db = 0; db < 8; ++db) acc.O[db] *= alpha;
  }

  const short4_t vv[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    acc.O[db] = mfma_pv<kBf16>(vv[db], ph, acc.O[db]);
    acc.O[db] = mfma_pv<kBf16>(vv[db], pl, acc.O[db]);
  }
}

// One pipeline step for the tile held in `cur`: on the wave's first tile of
// a segment, take q from the q slot; issue the next tile (or an empty load
// group) into `nxt` and the q slot; wait for the current tile; fold it in.
// Loads complete in issue order, so "all but the newest N" waits are exact
// (vector stores issued in between only make them wait longer).
template <int F, bool kPaged, bool kG4>
__device__ __forceinline__ void tile_step(const Params& P, const LdsReads& la, int par,
                                          e16_t* nxt, e16_t* qslot, bool first,
                                          bool has_next, const Seg& nseg, int nt,
                                          bool next_new_seg, const PageBases& npb, int t, int hi,
                                          uint2* vsh, uint4_t (&qb)[4], WaveAcc& acc) {
  if (first) {
    // the q loads (the first 1 or 2 of the group) landed
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(loads_per_tile<F, kG4>() - (kG4 ? 1 : 2))
                 : "memory");
    read_q<kG4, F>(qslot, group_of<kG4>(P), qb);
  }
  issue_tile<F, kPaged, kG4>(P, nseg, nt, has_next, next_new_seg, nxt, qslot, npb);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(loads_per_tile<F, kG4>()) : "memory");   // K, V landed
  if constexpr (F == kFmtFp4)
    compute_tile_fp4(la, par, qb, t, hi, P.scale_log2, vsh, acc);
  else if constexpr (F == kFmtE4m3)
    compute_tile8(la, par, qb, t, hi, P.scale_log2, acc);
  else
    compute_tile<F == kFmtBf16>(la, par, qb, t, hi, P.scale_log2, acc);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its vector memory loads (the next tiles' loads stay in
// flight across it). __syncthreads() would also wait for all vector memory.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Softmax state of each wave for the wave merge. In the general form the
// waves' O^T rows go to each wave's free LDS stage (the stage no load is in
// flight into), so the merge needs no LDS of its own beyond these words; the
// kG4 form has a dedicated buffer for its 4 rows per wave (MergeRows4).
struct MergeLds {
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  int free_stage[kWaves];
};

constexpr int kMergeRow = kDim + 4;   // floats per head row in a merge buffer (bank spread)
static_assert(kWaves == 4, "merge_waves reads one row per wave in a 4-read asm block");

struct MergeRows4 {
  float acc[kWaves][4][kMergeRow];
};
struct NoRows {
  int unused;
};
template <bool kG4> struct MergeRowsOf { typedef NoRows type; };
template <> struct MergeRowsOf<true> { typedef MergeRows4 type; };

// Merge outputs per thread: heads t / 64 + 4k for k below this.
template <bool kG4> constexpr int heads_per_thread() { return kG4 ? 1 : kMaxGroup / kWaves; }

// Merge the 4 waves' states. Thread t ends with heads hh = t / 64 + 4k
// (k < heads_per_thread, for hh < G) and the columns d, d + 1
// (d = 2 * (t % 64)): max M[k], denominator den[k], sums n0[k], n1[k].
// General form: `par` is this wave's pipeline parity, and stage par ^ 1 of
// the wave is free; the last barrier orders every read of the free stages
// before the waves' next loads into them. kG4 form: rows4 is reused from
// segment to segment, so the first barrier orders the previous merge's
// reads before this merge's writes.
template <bool kG4, int kSH>
__device__ __forceinline__ void merge_waves(const WaveAcc& acc, int group, int par, MergeLds& sm,
                                            e16_t (*stages)[2][kSH], MergeRows4* rows4,
                                            float (&M)[heads_per_thread<kG4>()],
                                            float (&den)[heads_per_thread<kG4>()],
                                            float (&n0)[heads_per_thread<kG4>()],
                                            float (&n1)[heads_per_thread<kG4>()]) {
  constexpr int kHeads = heads_per_thread<kG4>();
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G4 = lane >> 4, j = lane & 15;
  const float kNegInf = -__builtin_inff();
  const float l = sum_over_row_groups(acc.l);
  if constexpr (kG4) lds_barrier();     // the previous merge's readers are done
  if (lane < group) {
    sm.m[wv][lane] = acc.m;
    sm.l[wv][lane] = l;
  }
  if constexpr (kG4) {
    if (j < 4) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<float4_t*>(&rows4->acc[wv][j][16 * db + 4 * G4]) = acc.O[db];
    }
  } else {
    if (lane == 0) sm.free_stage[wv] = par ^ 1;
    // The stage accesses are asm: the compiler would otherwise make them wait
    // for every load in flight (the next tile's loads also write LDS stages).
    if (j < group) {
      const unsigned base = lds_addr(stages[wv][par ^ 1]) + 4 * (j * kMergeRow + 4 * G4);
#pragma unroll
      for (int db = 0; db < 8; ++db)
        asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(base), "v"(acc.O[db]), "i"(64 * db)
                     : "memory");
    }
  }
  lds_barrier();
  const int d = (tid & 63) * 2;
  unsigned bufs[kWaves];
  if constexpr (!kG4) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) bufs[w] = lds_addr(stages[w][sm.free_stage[w]]);
  }
#pragma unroll
  for (int k = 0; k < kHeads; ++k) {
    const int hh = (tid >> 6) + kWaves * k;
    M[k] = kNegInf;
    den[k] = 0.f;
    n0[k] = 0.f;
    n1[k] = 0.f;
    if (hh >= group) continue;
    float2 x[kWaves];
    if constexpr (kG4) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        x[w] = *reinterpret_cast<const float2*>(&rows4->acc[w][hh][d]);
    } else {
      const unsigned off = 4 * (hh * kMergeRow + d);
      asm volatile(
          "ds_read_b64 %0, %4\n\t"
          "ds_read_b64 %1, %5\n\t"
          "ds_read_b64 %2, %6\n\t"
          "ds_read_b64 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
          : "v"(bufs[0] + off), "v"(bufs[1] + off), "v"(bufs[2] + off), "v"(bufs[3] + off)
          : "memory");
    }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M[k] = fmaxf(M[k], sm.m[w][hh]);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float ms = sm.m[w][hh];
      const float wt = (ms == kNegInf) ? 0.f : exp2_hw(ms - M[k]);   // waves without rows
      den[k] = __builtin_fmaf(wt, sm.l[w][hh], den[k]);
      n0[k] = __builtin_fmaf(wt, x[w].x, n0[k]);
      n1[k] = __builtin_fmaf(wt, x[w].y, n1[k]);
    }
  }
  if constexpr (!kG4) lds_barrier();
}

// Partial slot of a segment in piece w: 2w for the piece's first segment,
// 2w + 1 for a segment that starts strictly inside the piece (at most one of
// those is cut by the piece's end).
__device__ __forceinline__ long long slot_of(long long seg_off, long long piece_start, int w) {
  return 2LL * w + (seg_off > piece_start ? 1 : 0);
}

// Empty sequences get zero rows and empty segment descriptors (workgroup w
// takes b = w, w + grid, ...). Lengths come from the length register or
// scalar loads, so nothing here waits for vector loads in flight.
__device__ __forceinline__ void zero_empty_sequences(const Params& P, int lens_v, int w) {
  const int tid = threadIdx.x;
  for (int b = w; b < P.batch; b += gridDim.x) {
    if (seq_len_of(P, lens_v, b) == 0) {
      uint4_t* dst = reinterpret_cast<uint4_t*>(P.out + (size_t)b * P.q_heads * kDim);
      for (int i = tid; i < P.q_heads * (kDim / 8); i += kThreads) dst[i] = (uint4_t){0u, 0u, 0u, 0u};
      if (!P.fused)
        for (int g = tid; g < P.kv_heads; g += kThreads)
          P.seg_desc[(size_t)b * P.kv_heads + g] = make_int2(0, 0);
    }
  }
}

// ---------------------------------------------------------------- combine
// Partial results of the single-launch form are written and read as
// device-scope (agent) relaxed atomics: each access is then coherent across
// the XCDs' L2 caches by itself (the stores write through to memory, the
// loads do not hit stale L2 lines), so no L2 write-back or invalidate is
// needed around the ticket. Ordering: the writer waits for its stores to
// complete before its ticket is taken, and the merging workgroup issues its
// loads only after its ticket has returned.
__device__ __forceinline__ void store_partial(float2* p, float2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     __builtin_bit_cast(unsigned long long, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 load_partial(const float2* p) {
  return __builtin_bit_cast(
      float2, __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT));
}

struct CombineLds {
  float xs[kThreads][10];
};

// Merge the n partials of segment (b, g), which kernel 1 cut into pieces
// first_w .. first_w + n - 1, and write output rows of heads head0 ..
// head0 + nheads - 1 of the group (all G, or one). The 16 nheads (head,
// 8-column group) pairs are spread over the 256 threads: thread t takes pair
// t % 16 nheads (head head0 + pair / 16, columns 8 (pair % 16) .. +7) and,
// as subset t / (16 nheads) of S = 256 / (16 nheads) subsets (threads past
// S subsets idle), every S-th partial: a running max over batches of
// independent loads. The subsets are then merged through LDS, in a fixed
// order, so results do not depend on timing or on which workgroup runs the
// merge.
// Partial i lives in piece first_w + i: the first piece holds it in its
// second slot if the segment starts inside that piece (bit), every later
// piece holds it as its first segment.
// kCoherent: the partials were written in this launch (single-launch form)
// and are read with device-scope loads.
template <bool kBf16, bool kCoherent, bool kG4>
__device__ __forceinline__ void combine_segment(const Params& P, int b, int g, int first_w, int n,
                                                int bit, int head0, int nheads, CombineLds& lds) {
  const int tid = threadIdx.x;
  const int group = group_of<kG4>(P), npairs = 16 * nheads, nsub = kThreads / npairs;
  const long long slot0 = 2LL * first_w + bit;
  const int pair = tid % npairs, sub = tid / npairs;
  const int hh = head0 + (pair >> 4), c8 = (pair & 15) * 8;
  const float kNegInf = -__builtin_inff();
  float M = kNegInf, den = 0.f;
  float4_t na = {0.f, 0.f, 0.f, 0.f}, nb = {0.f, 0.f, 0.f, 0.f};
  // Partials sub, sub + S, ... in batches of kBatch: a batch's loads are all
  // issued before its first use, then merged one by one in index order.
  constexpr int kBatch = 4;
  const int first = sub < nsub ? sub : n;            // idle threads take no partials
  for (int i0 = first; i0 < n; i0 += kBatch * nsub) {
    float2 ml[kBatch];
    float4_t a0[kBatch], a1[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * nsub;
      if (i >= n) break;
      const long long sl = i == 0 ? slot0 : 2LL * (first_w + i);
      const float* src = P.ws_acc + (sl * group + hh) * kDim + c8;
      if constexpr (kCoherent) {
        ml[u] = load_partial(P.ws_ml + sl * group + hh);
        const float2* s2 = reinterpret_cast<const float2*>(src);
        const float2 x0 = load_partial(s2), x1 = load_partial(s2 + 1);
        const float2 x2 = load_partial(s2 + 2), x3 = load_partial(s2 + 3);
        a0[u] = (float4_t){x0.x, x0.y, x1.x, x1.y};
        a1[u] = (float4_t){x2.x, x2.y, x3.x, x3.y};
      } else {
        ml[u] = P.ws_ml[sl * group + hh];
        a0[u] = *reinterpret_cast<const float4_t*>(src);
        a1[u] = *reinterpret_cast<const float4_t*>(src + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (i0 + u * nsub >= n) break;
      // Explicit fused multiply-adds: the same operations wherever this
      // function is inlined (the two launch forms must agree bitwise).
      const float Mn = fmaxf(M, ml[u].x);
      const float s_old = exp2_hw(M - Mn), s_new = exp2_hw(ml[u].x - Mn);
      den = __builtin_fmaf(den, s_old, ml[u].y * s_new);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        na[k] = __builtin_fmaf(na[k], s_old, a0[u][k] * s_new);
        nb[k] = __builtin_fmaf(nb[k], s_old, a1[u][k] * s_new);
      }
      M = Mn;
    }
  }
  float* x = lds.xs[tid];
  x[0] = M;
  x[1] = den;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 + k] = na[k];
    x[6 + k] = nb[k];
  }
  __syncthreads();
  if (tid < npairs) {
    float Mx = kNegInf;
    for (int k = 0; k < nsub; ++k) Mx = fmaxf(Mx, lds.xs[k * npairs + pair][0]);
    float d = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < nsub; ++k) {
      const float* y = lds.xs[k * npairs + pair];
      const float wt = (y[0] == kNegInf) ? 0.f : exp2_hw(y[0] - Mx);   // subsets without partials
      d = __builtin_fmaf(wt, y[1], d);
#pragma unroll
      for (int c = 0; c < 8; ++c) o[c] = __builtin_fmaf(wt, y[2 + c], o[c]);
    }
    const float vs = P.out_scale;
    uint4_t r;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      r[c] = (unsigned)to_elem<kBf16>(o[2 * c] / d * vs) |
             ((unsigned)to_elem<kBf16>(o[2 * c + 1] / d * vs) << 16);
    *reinterpret_cast<uint4_t*>(P.out + ((size_t)b * P.q_heads + g * group + hh) * kDim + c8) = r;
  }
}

// ---------------------------------------------------------------- kernel 1
// The leading scalar arguments repeat fields of P so that they arrive
// preloaded in scalar registers (kernel-argument preloading, gfx950): the
// lengths load is issued before the rest of the arguments have been read.
template <int F, bool kPaged, bool kG4>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gqa_decode_pieces(const int32_t* seq_lens, int batch, int wave_planner, Params P) {
  int raw_len = 0;
  if (wave_planner) {
    const int ln = threadIdx.x & 63;
    raw_len = ln < batch ? seq_lens[ln] : 0;
  }
  constexpr bool kBf16 = F == kFmtBf16;
  constexpr int kRows = tile_rows<F>();
  __shared__ long long red[kWaves];
  __shared__ long long sh_found;
  __shared__ int sh_found_b, sh_found_len;
  __shared__ __attribute__((aligned(16))) e16_t stages[kWaves][2][stage_halves<F>()];
  __shared__ __attribute__((aligned(16))) e16_t qslots[kWaves][q_halves<kG4>()];
  __shared__ MergeLds sm;
  __shared__ __attribute__((aligned(16))) typename MergeRowsOf<kG4>::type rows4_lds;
  MergeRows4* rows4 = nullptr;
  if constexpr (kG4) rows4 = &rows4_lds;
  __shared__ int sh_last[2];
  __shared__ int sh_cut[2][3];   // single launch: (Hkv * b + g, first piece, n2) of cut segments
  // FP4: each wave's V block scales as fp16 pairs (fp4_v_scales)
  __shared__ __attribute__((aligned(16))) uint2 vscales[F == kFmtFp4 ? kWaves * 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
  const int G = lane >> 4, j = lane & 15;
  const int w = blockIdx.x;

  long long total, p0, found;
  Pieces pcw;
  int found_b, found_len = 0;
  int lens_v = 0;
  if (P.wave_planner) {
    total = wave_plan(P, raw_len, &p0, &pcw, &found, &found_b, &lens_v);
  } else {
    long long part = 0;
    for (int b = tid; b < P.batch; b += kThreads)
      part += seq_cost(P, clamp_len(P.seq_lens[b], P.capacity));
    total = block_sum(part, red);
    pcw = piece_lens(P, total);
    p0 = piece_start(pcw, w);
    found_b = -1;
    if (p0 < total) {
      locate(p0, P, red, &sh_found, &sh_found_b, &sh_found_len);
      __syncthreads();
      found_b = sh_found_b;
      found = sh_found;
      found_len = sh_found_len;
    }
  }
  total = uniform64(total);
  p0 = uniform64(p0);
  if (p0 >= total) {                                // uniform: this piece is empty
    zero_empty_sequences(P, lens_v, w);
    return;
  }
  found = uniform64(found);
  found_b = __builtin_amdgcn_readfirstlane(found_b);
  Pieces pc;
  pc.Qa = uniform64(pcw.Qa);
  pc.Qb = uniform64(pcw.Qb);
  pc.G1 = uniform64(pcw.G1);
  const long long len_w = piece_length(pc, w);
  const long long p1 = p0 + len_w < total ? p0 + len_w : total;

  Seg s;
  s.b = found_b;
  s.len = P.wave_planner ? __builtin_amdgcn_readlane(lens_v, s.b)
                         : __builtin_amdgcn_readfirstlane(found_len);
  const long long stride = cost_len(P, s.len) + P.seg_cost;
  // g = (p0 - found) / stride, which is below Hkv: a float estimate (off by
  // at most one), then exact integer corrections; no 64-bit division.
  const long long rel = p0 - found;
  s.g = (int)((float)rel * __builtin_amdgcn_rcpf((float)stride));
  s.g = s.g < 0 ? 0 : (s.g > P.kv_heads - 1 ? P.kv_heads - 1 : s.g);
  while (s.g > 0 && (long long)s.g * stride > rel) --s.g;
  while (s.g < P.kv_heads - 1 && (long long)(s.g + 1) * stride <= rel) ++s.g;
  s.off = found + (long long)s.g * stride + P.seg_cost;
  seg_set_range(s, p0, p1);
  seg_bases<F, kPaged>(P, s);
  if (s.hi <= s.lo) {                               // only fixed-cost units in this piece
    zero_empty_sequences(P, lens_v, w);
    return;
  }

  // Prime the pipeline with this wave's first tile.
  e16_t* st0 = stages[wv][0];
  e16_t* st1 = stages[wv][1];
  e16_t* qslot = qslots[wv];
  uint2* vsh = F == kFmtFp4 ? vscales + 64 * wv : vscales;
  const LdsReads la = lds_reads<F>(st0);
  Seg pf = s;
  int pt = s.lo + kRows * wv;
  const bool pf_ok = tile_first<F, kPaged>(P, pf, pt, p1, wv, lens_v);
  PageBases pbs;                                    // paged: pages of the issued tile
  if constexpr (kPaged) pbs = page_bases<F>(P, pf, pt, pf_ok);
  issue_tile<F, kPaged, kG4>(P, pf, pt, pf_ok, true, st0, qslot, pbs);
  zero_empty_sequences(P, lens_v, w);               // overlaps the first tile's loads
  int par = 0;
  // Single launch: the number of segments this piece cut (at most its first
  // and its last); sh_cut keeps them (in LDS, off the loop's registers).
  int ncut = 0;

  while (true) {
    WaveAcc acc;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc.O[db] = (float4_t){0.f, 0.f, 0.f, 0.f};
    acc.m = -__builtin_inff();
    acc.l = 0.f;
    // This wave's tiles of s; the prefetch cursor (pf, pt) is on the first.
    uint4_t qb[4];
    for (int t = s.lo + kRows * wv; t < s.hi; t += kWaves * kRows) {
      Seg nf = pf;
      int nt = pt;
      const bool n_ok = tile_next<F, kPaged>(P, nf, nt, p1, wv, lens_v);
      if constexpr (kPaged) pbs = page_bases<F>(P, nf, nt, n_ok);
      tile_step<F, kPaged, kG4>(P, la, par, par ? st0 : st1, qslot, t == s.lo + kRows * wv, n_ok, nf, nt,
                nf.off != s.off, pbs, t, s.hi, vsh, qb, acc);
      pf = nf;
      pt = nt;
      par ^= 1;
    }

    constexpr int kHeads = heads_per_thread<kG4>();
    const int group = group_of<kG4>(P);
    float M[kHeads], den[kHeads], n0[kHeads], n1[kHeads];
    merge_waves<kG4, stage_halves<F>()>(acc, group, par, sm, stages, rows4, M, den, n0, n1);
    const int d = (tid & 63) * 2;
    const int seg_id = s.b * P.kv_heads + s.g;

    // Pieces holding the segment's first and last rows: this one unless the
    // segment starts before p0 (ends after p1); only then a division, in 32
    // bits when every cost total fits them.
    const long long seg_end = s.off + s.len;
    const long long first_w = s.off >= p0 ? w : piece_of(P, pc, s.off);
    const long long last_w = seg_end <= p1 ? w : piece_of(P, pc, seg_end - 1);
    // 2 * (pieces holding rows of the segment) + (it starts inside its first
    // piece, whose second slot then holds its partial)
    const int n2 =
        (int)(2 * (last_w - first_w + 1)) + (s.off > piece_start(pc, first_w) ? 1 : 0);
    if (!P.fused && first_w == w && tid == 0)        // the segment starts in this piece
      P.seg_desc[seg_id] = make_int2(w, n2);
    if (first_w == last_w) {                         // the segment lies in this piece
      const float vs = P.out_scale;
#pragma unroll
      for (int k = 0; k < kHeads; ++k) {
        const int hh = (tid >> 6) + kWaves * k;
        if (hh >= group) continue;
        const unsigned o = (unsigned)to_elem<kBf16>(n0[k] / den[k] * vs) |
                           ((unsigned)to_elem<kBf16>(n1[k] / den[k] * vs) << 16);
        *reinterpret_cast<unsigned*>(
            P.out + ((size_t)s.b * P.q_heads + s.g * group + hh) * kDim + d) = o;
      }
    } else {
      const long long slot = slot_of(s.off, p0, w);
#pragma unroll
      for (int k = 0; k < kHeads; ++k) {
        const int hh = (tid >> 6) + kWaves * k;
        if (hh >= group) continue;
        float2* acc_dst = reinterpret_cast<float2*>(P.ws_acc + (slot * group + hh) * kDim + d);
        float2* ml_dst = P.ws_ml + slot * group + hh;
        if (P.fused) {
          store_partial(acc_dst, make_float2(n0[k], n1[k]));
          if (d == 0) store_partial(ml_dst, make_float2(M[k], den[k]));
        } else {
          *acc_dst = make_float2(n0[k], n1[k]);
          if (d == 0) *ml_dst = make_float2(M[k], den[k]);
        }
      }
      if (P.fused && tid == 0) {
        sh_cut[ncut][0] = seg_id;
        sh_cut[ncut][1] = (int)first_w;
        sh_cut[ncut][2] = n2;
      }
      ++ncut;
    }

    if (!more_segments(P, s, p1)) break;
    seg_next<F, kPaged, false>(P, s, p1, lens_v);
  }

  // Single launch: take a ticket for each cut segment; the piece that
  // completes a segment merges its partials (in the same fixed order as the
  // combine kernel, so both forms give the same bits). Tickets are taken
  // after all of this piece's segments, so the pipeline never waits on them.
  if (P.fused && ncut > 0) {
    // Every wave's partial stores (device-scope) complete before the
    // tickets are taken. This also drains the last (empty) tile loads into
    // LDS, so the stages are free for the merge below.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid < ncut) {
      const int seg = sh_cut[tid][0], n = sh_cut[tid][2] >> 1;
      const int done = __hip_atomic_fetch_add(P.tickets + seg, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      const bool last = done == n - 1;
      if (last) __hip_atomic_store(P.tickets + seg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh_last[tid] = last ? 1 : 0;
    }
    __syncthreads();
    bool merged = false;
    for (int i = 0; i < ncut; ++i) {
      if (sh_last[i] == 0) continue;               // uniform
      if (merged) __syncthreads();                 // the previous merge's LDS reads are done
      merged = true;
      const int seg = __builtin_amdgcn_readfirstlane(sh_cut[i][0]);
      const int fw = __builtin_amdgcn_readfirstlane(sh_cut[i][1]);
      const int n2 = __builtin_amdgcn_readfirstlane(sh_cut[i][2]);
      // the merge reads pieces fw .. fw + n - 1 only, all inside the grid
      const int nm = min(n2 >> 1, max(P.pieces - fw, 0));
      // the same subsets as the combine kernel: per head when it splits heads
      CombineLds& clds = *reinterpret_cast<CombineLds*>(&stages[0][0][0]);
      const int sb = seg / P.kv_heads, sg = seg % P.kv_heads;
      if (P.combine_per_head) {
        for (int h = 0; h < group_of<kG4>(P); ++h) {
          if (h > 0) __syncthreads();              // the previous head's LDS reads are done
          combine_segment<kBf16, true, kG4>(P, sb, sg, fw, nm, n2 & 1, h, 1, clds);
        }
      } else {
        combine_segment<kBf16, true, kG4>(P, sb, sg, fw, nm, n2 & 1, 0, group_of<kG4>(P), clds);
      }
    }
  }
}

// ---------------------------------------------------------------- kernel 2
// Two-launch form: one work unit per segment (b, g), or per (segment, query
// head) when segments are few (P.combine_per_head); if kernel 1 cut the
// segment into several pieces, merge their partials, else skip it. Per
// segment for many segments: G x fewer waves to dispatch, and most skip at
// once. Per head for few segments: G x more subsets share a segment's
// partials, so each thread folds G x fewer of them in sequence.
// Workgroup w takes units w, w + grid, ... (the grid is capped at
// kCombineMaxGrid workgroups, so any batch stays within one dispatch's
// 32-bit work-item count).
// The leading arguments repeat fields of P (preloaded, as for kernel 1).
template <int F, bool kG4>
__global__ __launch_bounds__(kThreads) void gqa_decode_combine(const int2* seg_desc, int per_head,
                                                               int group_arg, Params P) {
  __shared__ __attribute__((aligned(16))) CombineLds lds;
  const int group = kG4 ? 4 : group_arg;
  const long long units = (long long)P.batch * P.kv_heads * (per_head ? group : 1);
  bool merged = false;
  for (long long u = blockIdx.x; u < units; u += gridDim.x) {
    const int seg = (int)(per_head ? u / group : u);
    // A vector load (the index is hidden in a vector register): it is
    // issued at once, without waiting for the scalar loads of the other
    // arguments.
    int vseg = seg;
    asm volatile("" : "+v"(vseg));
    const int2 desc = seg_desc[vseg];
    const int b = seg / P.kv_heads, g = seg - b * P.kv_heads;
    // at most the pieces after the first (a descriptor is never beyond the grid)
    const int n = min(desc.y >> 1, max(P.pieces - desc.x, 0));
    if (n <= 1) continue;              // empty (zero rows) or finished by kernel 1
    if (merged) __syncthreads();       // the previous merge's LDS reads are done
    merged = true;
    if (per_head)
      combine_segment<F == kFmtBf16, false, kG4>(P, b, g, desc.x, n, desc.y & 1,
                                                 (int)(u - (long long)seg * group), 1, lds);
    else
      combine_segment<F == kFmtBf16, false, kG4>(P, b, g, desc.x, n, desc.y & 1, 0, group, lds);
  }
}

}  // namespace

namespace {
constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];   // per device: the scratch's device address
}  // namespace

hipError_t scratch_area(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int resident_workgroups_per_cu() {
  const void* kernels[16] = {
      (const void*)gqa_decode_pieces<kFmtF16, false, true>,
      (const void*)gqa_decode_pieces<kFmtBf16, false, true>,
      (const void*)gqa_decode_pieces<kFmtE4m3, false, true>,
      (const void*)gqa_decode_pieces<kFmtF16, true, true>,
      (const void*)gqa_decode_pieces<kFmtBf16, true, true>,
      (const void*)gqa_decode_pieces<kFmtE4m3, true, true>,
      (const void*)gqa_decode_pieces<kFmtF16, false, false>,
      (const void*)gqa_decode_pieces<kFmtBf16, false, false>,
      (const void*)gqa_decode_pieces<kFmtE4m3, false, false>,
      (const void*)gqa_decode_pieces<kFmtF16, true, false>,
      (const void*)gqa_decode_pieces<kFmtBf16, true, false>,
      (const void*)gqa_decode_pieces<kFmtE4m3, true, false>,
      (const void*)gqa_decode_pieces<kFmtFp4, false, true>,
      (const void*)gqa_decode_pieces<kFmtFp4, true, true>,
      (const void*)gqa_decode_pieces<kFmtFp4, false, false>,
      (const void*)gqa_decode_pieces<kFmtFp4, true, false>};
  int m = 1 << 30;
  for (const void* k : kernels) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, 0) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    m = n < m ? n : m;
  }
  return m;
}

long long grid_for(int batch, int capacity, int kv_heads, const SplitConfig& cfg) {
  if (cfg.forced_piece > 0) {
    const long long a = cfg.row_align > 1 ? cfg.row_align : 1;
    const long long rows = (long long)kv_heads * batch * ((capacity + a - 1) / a * a);
    return (rows + cfg.forced_piece - 1) / cfg.forced_piece;
  }
  return cfg.pieces;
}

size_t partial_bytes_for_grid(long long grid, int group) {
  return (size_t)(2 * grid) * group * kHeadSlotFloats * sizeof(float);
}

size_t segment_bytes_for_batch(int batch, int kv_heads) {
  return ((size_t)batch * kv_heads * sizeof(int2) + 255) & ~(size_t)255;
}

template <int F, bool kPaged, bool kG4>
hipError_t launch_kernels(const Params& P, long long grid, int batch, long long combine_cap,
                          hipStream_t stream, hipEvent_t* events) {
  // The combine only depends on the output type: fp16 for every format but bf16.
  constexpr int kCombineF = F == kFmtBf16 ? kFmtBf16 : kFmtF16;
  hipError_t err = hipSuccess;
  const long long units = (long long)batch * P.kv_heads * (P.combine_per_head ? P.group : 1);
  const dim3 pieces_grid((unsigned)grid),
      combine_grid((unsigned)(units < combine_cap ? units : combine_cap)), block(kThreads);
  if (events) {
    // Start/stop events attached to the dispatches: they time each kernel's
    // execution without extra packets between the kernels.
    hipExtLaunchKernelGGL(gqa_decode_pieces<F, kPaged, kG4>, pieces_grid, block, 0, stream, events[0],
                          events[1], 0, P.seq_lens, P.batch, P.wave_planner, P);
    if ((err = hipGetLastError()) != hipSuccess || P.fused) return err;
    hipExtLaunchKernelGGL(gqa_decode_combine<kCombineF, kG4>, combine_grid, block, 0, stream, events[2],
                          events[3], 0, P.seg_desc, P.combine_per_head, P.group, P);
    return hipGetLastError();
  }
  gqa_decode_pieces<F, kPaged, kG4>
      <<<pieces_grid, block, 0, stream>>>(P.seq_lens, P.batch, P.wave_planner, P);
  if ((err = hipGetLastError()) != hipSuccess || P.fused) return err;
  gqa_decode_combine<kCombineF, kG4>
      <<<combine_grid, block, 0, stream>>>(P.seg_desc, P.combine_per_head, P.group, P);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                         ElemType elem, const Layout& layout, float score_scale_log2,
                         float out_scale, int batch, int capacity, const SplitConfig& cfg,
                         long long grid, void* partials, int* tickets, hipStream_t stream,
                         hipEvent_t* events) {
  Params P;
  P.tickets = tickets;
  P.fused = tickets != nullptr ? 1 : 0;
  P.q = static_cast<const e16_t*>(q);
  P.kv = static_cast<const e16_t*>(kv);
  P.kv_scales = static_cast<const uint8_t*>(layout.kv_scales);
  P.sc_sb = layout.sc_sb;
  P.sc_sk = layout.sc_sk;
  P.sc_sh = layout.sc_sh;
  P.sc_sr = layout.sc_sr;
  P.seq_lens = seq_lens;
  P.out = static_cast<e16_t*>(out);
  const int group = layout.q_heads / layout.kv_heads;
  P.seg_desc = reinterpret_cast<int2*>(partials);
  P.ws_ml = reinterpret_cast<float2*>(static_cast<char*>(partials) +
                                      segment_bytes_for_batch(batch, layout.kv_heads));
  P.ws_acc = reinterpret_cast<float*>(P.ws_ml + (size_t)(2 * grid) * group);
  P.batch = batch;
  P.capacity = capacity;
  P.kv_heads = layout.kv_heads;
  P.q_heads = layout.q_heads;
  P.group = group;
  P.pieces = (int)grid;
  P.pieces_first = cfg.pieces_first > 0 && cfg.pieces_first < grid ? cfg.pieces_first : (int)grid;
  P.second_share = cfg.second_share > 0 && cfg.second_share <= 64 ? cfg.second_share : 64;
  if (P.second_share == 64) P.pieces_first = (int)grid;
  P.min_piece = cfg.min_piece;
  P.forced_piece = cfg.forced_piece;
  P.seg_cost = cfg.forced_piece > 0 ? 0 : cfg.seg_cost;
  P.scale_log2 = score_scale_log2;
  P.out_scale = out_scale;
  P.q_sb = layout.q_sb;
  P.q_sh = layout.q_sh;
  P.kv_sb = layout.kv_sb;
  P.kv_sk = layout.kv_sk;
  P.kv_sh = layout.kv_sh;
  P.kv_sr = layout.kv_sr;
  P.block_table = layout.block_table;
  P.max_pages = layout.max_pages;
  P.page_shift = layout.page_shift;
  P.num_pages = layout.num_pages;
  P.row_align = cfg.row_align > 1 ? cfg.row_align : 1;
  // The one-wave planner adds up to 64 sequence costs in 32 bits.
  {
    const long long a = P.row_align;
    const long long seg_max = (capacity + a - 1) / a * a + P.seg_cost;
    P.wave_planner = batch <= 64 && (long long)batch * layout.kv_heads * seg_max < (1LL << 32);
  }
  // One combine workgroup per head when segments are few and are cut into
  // more pieces than a whole-segment workgroup folds in one batch of loads
  // (4 per subset, 256 / 16G subsets). Pieces per segment, estimated from
  // the shape alone: the pieces shared by the segments, at most what one
  // segment of full capacity spans.
  {
    const long long segs = (long long)batch * layout.kv_heads;
    const long long piece_rows = cfg.forced_piece > 0 ? cfg.forced_piece : cfg.min_piece;
    const long long span = (capacity + P.seg_cost) / (piece_rows > 0 ? piece_rows : 1) + 1;
    const long long shared = cfg.forced_piece > 0 ? span : (grid + segs - 1) / segs;
    const long long n_est = shared < span ? shared : span;
    P.combine_per_head = segs < kCombinePerHeadBelow && n_est * group > 64 ? 1 : 0;
  }

  const bool paged = layout.block_table != nullptr;
  const bool g4 = group == 4;
#define GQA_LAUNCH(F)                                                              \
  (paged ? (g4 ? launch_kernels<F, true, true>(P, grid, batch, cfg.combine_max_grid, stream, events)      \
               : launch_kernels<F, true, false>(P, grid, batch, cfg.combine_max_grid, stream, events))    \
         : (g4 ? launch_kernels<F, false, true>(P, grid, batch, cfg.combine_max_grid, stream, events)     \
               : launch_kernels<F, false, false>(P, grid, batch, cfg.combine_max_grid, stream, events)))
  switch (elem) {
    case ElemType::kBf16:
      return GQA_LAUNCH(kFmtBf16);
    case ElemType::kE4m3Kv:
      return GQA_LAUNCH(kFmtE4m3);
    case ElemType::kFp4Kv:
      return GQA_LAUNCH(kFmtFp4);
    default:
      return GQA_LAUNCH(kFmtF16);
  }
#undef GQA_LAUNCH
}

}  // namespace gqa

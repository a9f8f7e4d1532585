/*
 * gqa_decode.h -- C ABI of the MI355X (gfx950) FP16 grouped-query-attention
 * single-token decode library (libgqa_decode.so).
 *
 * The operation is the one documented for `sm110_gqa_decode` on the
 * FlashInfer PR #5052 analysis page ("SM110 FP16 GQA decode"):
 *   - section 1 (docstring): q is a contiguous FP16 [batch, 32, 128] tensor,
 *     kv is a contiguous FP16 stacked cache [batch, 2, 8, capacity, 128],
 *     sequence lengths are a contiguous device int32 [batch] tensor, the
 *     output has q's shape and is owned by the caller, and the scores are
 *     multiplied by q_scale as well as by 1/sqrt(128);
 *   - section 2: 32 query heads, 8 KV heads, head dim 128, 4:1 grouping;
 *   - section 3 (benchmark): the result equals PyTorch SDPA with a boolean
 *     length mask, scale 1/sqrt(128) and enable_gqa=True.
 *
 * For every batch entry b and query head h (g = h / 4):
 *   L   = clamp(seq_lens[b], 0, capacity)
 *   s_i = (q_scale / sqrt(128)) * dot(q[b,h,:], kv[b,0,g,i,:])   for i < L
 *   out[b,h,:] = sum_i softmax(s)_i * kv[b,1,g,i,:]               (fp16, RNE)
 * Rows i >= L are never read. L == 0 yields a zero row.
 *
 * Arithmetic: fp16 inputs, fp32 accumulation for the dot products, the
 * softmax and the weighted sum, one round-to-nearest-even to fp16 at the end.
 *
 * Entry points: gqa_decode (the page's call); gqa_decode_chunked (a fixed
 * split length); gqa_decode_typed (bfloat16 tensors or an FP8 E4M3 cache,
 * with per-tensor K/V scales); gqa_decode_ex (the same with explicit
 * strides, other head counts and paged caches); gqa_decode_fp4 (a
 * block-scaled FP4 cache); and helpers for the workspace, the launch form,
 * kernel timing and error text. This library's extensions beyond the page
 * are marked as such where they are declared.
 *
 * All entry points are thread-safe. Compute entry points only enqueue work
 * on `stream` (no host synchronisation); a device-side fault surfaces at the
 * caller's next synchronisation. Every call reports its outcome as a
 * gqa_status; the thread-local text of the last failure is available from
 * gqa_decode_last_error().
 */
#ifndef GQA_DECODE_H_
#define GQA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_NUM_Q_HEADS 32
#define GQA_NUM_KV_HEADS 8
#define GQA_HEAD_DIM 128

/* Other head counts (gqa_decode_ex): at most GQA_MAX_GROUP query heads share
 * one KV head, at most GQA_MAX_KV_HEADS KV heads, and batch * num_kv_heads
 * stays at or below GQA_MAX_SEGMENTS. */
#define GQA_MAX_GROUP 8
#define GQA_MAX_KV_HEADS 1024
#define GQA_MAX_SEGMENTS (1 << 27)

/* Largest supported capacity (rows per (sequence, KV head)). The kernels
 * address one (sequence, KV head) block of K or V with 32-bit byte offsets,
 * so a block stays below 2 GiB: 2^22 rows x 256 B = 1 GiB. */
#define GQA_MAX_CAPACITY (1 << 22)

/* Status codes returned by the entry points (0 = success). */
typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_NULL = -1,             /* a required pointer is NULL                        */
  GQA_ERR_BAD_SHAPE = -2,        /* batch outside [1, 2^24] or capacity outside
                                    [1, GQA_MAX_CAPACITY]                              */
  GQA_ERR_MISALIGNED = -3,       /* q, kv or out not 16-byte aligned; seq_lens not 4   */
  GQA_ERR_ALIAS = -4,            /* out overlaps q, kv or seq_lens                     */
  GQA_ERR_NO_DEVICE = -5,        /* no HIP device visible                              */
  GQA_ERR_UNSUPPORTED_ARCH = -6, /* the device is not gfx950 (MI355X class)            */
  GQA_ERR_ALLOC = -7,            /* workspace allocation failed                        */
  GQA_ERR_LAUNCH = -8,           /* a kernel launch or runtime call failed             */
  GQA_ERR_BAD_ARG = -9,          /* an out-of-range scalar argument (e.g. chunk_len)   */
  GQA_ERR_DEVICE_MISMATCH = -10  /* a pointer is not device memory, or buffers live on
                                    different devices                                  */
} gqa_status;

/*
 * gqa_decode -- decode one token of FP16 GQA for every sequence in a batch.
 *
 * q        device, fp16 [batch, 32, 128], contiguous, 16-byte aligned (read).
 * kv       device, fp16 [batch, 2, 8, capacity, 128], contiguous, 16-byte
 *          aligned; kv[b,0] holds K and kv[b,1] holds V (read). Offsets are
 *          computed in 64 bits, so caches above 2^31 elements are supported.
 * seq_lens device, int32 [batch] (read on the device only; values are clamped
 *          to [0, capacity]; the host never reads them, so the call can be
 *          captured in a HIP graph once the workspace exists).
 * out      device, fp16 [batch, 32, 128], contiguous, 16-byte aligned,
 *          caller-allocated; must not overlap q, kv or seq_lens (written).
 * q_scale  extra score scale, applied together with 1/sqrt(128).
 * batch     1 .. 2^24.
 * capacity  1 .. GQA_MAX_CAPACITY.
 * stream   HIP stream to enqueue on (NULL = the device's null stream).
 *
 * All buffers must live on one device; the kernels run on that device and
 * the caller's current device is restored before returning. The split-KV
 * pieces kernel runs, followed by the log-sum-exp combine kernel, or (see
 * gqa_decode_set_launch_form) the pieces kernel alone, whose last workgroup
 * per cut segment does the combine. The library keeps a cached fp32
 * workspace per (device, stream) for the partial results of sequences split
 * across workgroups, and for the single launch an int array of 8 * batch
 * tickets, zeroed when allocated and left zero by every call. Both are
 * allocated on first need, so the first call on a new stream, or one needing
 * a larger workspace or batch, must not be under graph capture (such a call
 * returns GQA_ERR_ALLOC with nothing enqueued); later calls allocate nothing
 * and can be captured. Calls on one stream are ordered by the stream; calls
 * on different streams use different workspaces.
 * Graphs: a call captured into a graph keeps the workspace and tickets of
 * the stream it was captured on. A later, larger eager call on that stream
 * gets new buffers and leaves those in place (they are freed only by
 * gqa_decode_release_workspace), so the graph stays valid; replays must not
 * overlap calls that use the same buffers (other replays of graphs captured
 * on that stream, or eager calls on it of a size the captured buffers
 * serve). gqa_decode_release_workspace invalidates every graph captured
 * before it.
 *
 * Returns GQA_OK, or a negative gqa_status with nothing enqueued.
 */
int gqa_decode(const void* q, const void* kv, const int32_t* seq_lens, void* out,
               float q_scale, int batch, int capacity, hipStream_t stream);

/*
 * gqa_decode_chunked -- gqa_decode with an explicit split length.
 *
 * Same arguments and semantics as gqa_decode, plus:
 * chunk_len  0 selects the automatic split (identical to gqa_decode). A
 *            positive value fixes the piece length: the valid rows of all
 *            (sequence, KV head) pairs, laid end to end, are cut into pieces
 *            of chunk_len rows, one workgroup each; a pair cut into several
 *            pieces is merged by a log-sum-exp combine. Negative values
 *            return GQA_ERR_BAD_ARG; values so small that the partial results
 *            would exceed 4 GiB also return GQA_ERR_BAD_ARG.
 * Used to exercise specific split counts (1, 2, many) and to study the split.
 */
int gqa_decode_chunked(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                       float q_scale, int batch, int capacity, int chunk_len,
                       hipStream_t stream);

/* Element types accepted by gqa_decode_typed. */
typedef enum gqa_dtype {
  GQA_DTYPE_F16 = 0,     /* q, kv and out are IEEE binary16 (the page-4 operation)      */
  GQA_DTYPE_BF16 = 1,    /* q, kv and out are bfloat16 (8-bit exponent, 7-bit fraction)  */
  GQA_DTYPE_E4M3_KV = 2, /* q and out binary16; kv holds OCP FP8 E4M3 bytes (1 sign,
                            4 exponent bits with bias 7, 3 fraction bits; no
                            infinities; S.1111.111 is NaN), one byte per element  */
  GQA_DTYPE_FP4_KV = 3   /* q and out binary16; kv holds block-scaled FP4: only
                            through gqa_decode_fp4 (declared below)               */
} gqa_dtype;

/*
 * gqa_decode_typed -- gqa_decode_chunked for other element types, with
 * per-tensor K and V scales.
 *
 * Same layouts, alignment, ownership and error behaviour as gqa_decode, with
 * q, kv and out of element type `dtype` (a gqa_dtype: 2 bytes per element,
 * except E4M3 kv at 1 byte, so its kv is [batch, 2, 8, capacity, 128]
 * bytes). The stored K and V values stand for k_scale * K and v_scale * V
 * (for E4M3 this is the usual per-tensor dequantisation scale):
 *   s_i = (q_scale * k_scale / sqrt(128)) * dot(q[b,h,:], kv[b,0,g,i,:])
 *   out[b,h,:] = v_scale * sum_i softmax(s)_i * kv[b,1,g,i,:]
 * in fp32, rounded once to the output type (round to nearest even). With
 * dtype GQA_DTYPE_F16 and k_scale = v_scale = 1 this is gqa_decode_chunked.
 * The page-4 API is FP16 only (FlashInfer PR #5052 analysis page, section
 * 1); BF16, the scales and the E4M3 cache are this library's extension (the
 * E4M3 format and dequantisation in on-chip memory follow the FlashInfer
 * NVFP4 paged-context attention page, whose K/V pages are dequantised to
 * E4M3 in shared memory). E4M3 values inside [0, L) that are NaN are outside
 * the contract, as non-finite fp16 inputs are.
 * Range: the scores and the unnormalised sums (sum_i p_i v_i with every
 * p_i <= 1, plus sum_i p_i) are fp32, so the result is finite only while
 * scale * sum_d |q_d k_d| and L * max|v| stay below the fp32 maximum
 * (3.4e38), where scale includes q_scale and k_scale. fp16 and E4M3 inputs
 * meet this for any scales below about 1e25; bfloat16 values above about
 * 1e32 may not, and then the output may be infinite or NaN.
 * chunk_len  as for gqa_decode_chunked (0 = automatic split).
 * Returns GQA_ERR_BAD_ARG for an unknown dtype or a non-finite scale.
 */
int gqa_decode_typed(const void* q, const void* kv, const int32_t* seq_lens, void* out, int dtype,
                     float q_scale, float k_scale, float v_scale, int batch, int capacity,
                     int chunk_len, hipStream_t stream);

/*
 * Memory layout of q and kv for gqa_decode_ex. Strides count elements of the
 * tensor they describe (not bytes), must be non-negative, and must keep
 * every row 16-byte aligned (stride * element size a multiple of 16); each
 * 128-element head row is contiguous. The values for the contiguous layouts
 * of gqa_decode are given in brackets (C = capacity, Hq and Hkv the head
 * counts).
 *
 * Head counts: num_q_heads (Hq) query heads and num_kv_heads (Hkv) KV heads;
 * 0 for both selects the page's 32 and 8. Hq must be a multiple of Hkv with
 * at most GQA_MAX_GROUP query heads per KV head; query head h reads KV head
 * h / (Hq / Hkv) (contiguous groups, as SDPA's enable_gqa). q and out are
 * then [batch, Hq, 128] and kv [batch, 2, Hkv, capacity, 128]. Multi-head
 * (Hq = Hkv) and multi-query (Hkv = 1, Hq <= 8) attention are special cases.
 *
 * Paged cache (block_table != NULL): kv holds num_pages pages, each
 * [2][8][page_size][128] under the strides below (kv_stride_batch is then the
 * stride between pages); position i of sequence b is row i % page_size of
 * page block_table[b * max_pages + i / page_size]. This is the HND page
 * layout named on the FlashInfer NVFP4 paged-context attention page.
 * Positions at or beyond a sequence's length are never read, so their
 * table entries are never read either. A page id outside [0, num_pages)
 * for a position inside the length reads as zeros (no fault; the result
 * for that sequence is then meaningless).
 */
typedef struct gqa_layout {
  int64_t q_stride_batch;    /* q[b] -> q[b+1]                      [Hq*128]        */
  int64_t q_stride_head;     /* q[b,h] -> q[b,h+1]                  [128]           */
  int64_t kv_stride_batch;   /* kv[b] -> kv[b+1], or page -> page   [2*Hkv*C*128]   */
  int64_t kv_stride_kind;    /* K -> V                              [Hkv*C*128]     */
  int64_t kv_stride_head;    /* KV head g -> g+1                    [C*128]         */
  int64_t kv_stride_row;     /* position i -> i+1                   [128]           */
  const int32_t* block_table; /* NULL, or device int32 [batch][max_pages], 4-byte
                                 aligned, on the same device as kv                   */
  int max_pages;             /* paged: entries per block_table row                   */
  int page_size;             /* paged: positions per page, a power of two >= 16      */
  int num_pages;             /* paged: pages in kv                                   */
  int num_q_heads;           /* Hq, or 0 (with num_kv_heads 0) for 32                */
  int num_kv_heads;          /* Hkv, or 0 (with num_q_heads 0) for 8                 */
} gqa_layout;

/*
 * gqa_decode_ex -- gqa_decode_typed with explicit strides and an optional
 * page table.
 *
 * layout  NULL means the contiguous layouts with 32 and 8 heads (then
 *         identical to gqa_decode_typed). out stays a contiguous
 *         [batch, Hq, 128] tensor.
 * capacity  the largest position count of a sequence (lengths are clamped
 *         to it); for a paged cache at most max_pages * page_size.
 * chunk_len  as for gqa_decode_chunked; for a paged cache it is rounded up
 *         to a multiple of 16.
 * Limits (GQA_ERR_BAD_ARG): kv_stride_row must cover a row (256 B, or 128 B
 * for E4M3); kv_stride_row in bytes times capacity (paged: page_size) and
 * q_stride_head in bytes times 7 plus 256 must stay below 2^31 (32-bit
 * buffer offsets); head counts as above. The overlap check for out uses
 * each tensor's address range under its strides.
 * Use: strided views (e.g. q as a slice of a packed projection output, or
 * an NHD cache [batch, capacity, 2, 8, 128] seen as [batch, 2, 8, capacity,
 * 128]) and paged caches, without copies.
 */
int gqa_decode_ex(const void* q, const void* kv, const int32_t* seq_lens, void* out, int dtype,
                  const gqa_layout* layout, float q_scale, float k_scale, float v_scale,
                  int batch, int capacity, int chunk_len, hipStream_t stream);

/*
 * gqa_decode_ex_noalloc -- gqa_decode_ex that allocates no device memory,
 * for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops and harnesses that forbid allocation.
 *
 * Arguments, layouts, results and errors are those of gqa_decode_ex, and the
 * result is bitwise the same. Instead of the cached per-stream workspace, the
 * partial results, segment descriptors and single-launch tickets live in a
 * fixed 16 MiB device array compiled into the library: each device the
 * library runs on holds one copy, from the first call on that device until
 * the process ends. The first 1 MiB holds the tickets, which are zero when
 * the library is loaded and left zero by every call. The other 15 MiB take
 * the partials and descriptors: the automatic split needs about
 * 2 x (workgroups launched) x G x 520 B plus 8 B per (sequence, KV head);
 * on an MI355X (256 or 512 workgroups, by element type) that is at most
 * about 2.2 MB at the page's 32/8 heads plus 8 KiB per 128 sequences.
 * Limits: a call whose partials and descriptors exceed 15 MiB (large
 * batches, or small chunk_len), or that takes the single launch with more
 * than 2^18 (sequence, KV head) pairs, returns GQA_ERR_BAD_SHAPE with
 * nothing enqueued. Calls that overlap on one device share the array and
 * race: calls on one device must be ordered (one stream, or streams joined
 * by events), including replays of graphs that captured this call. No
 * timing events are recorded (gqa_decode_profile_begin does not apply).
 * dtype: as for gqa_decode_ex (FP4 caches: GQA_ERR_BAD_ARG).
 */
int gqa_decode_ex_noalloc(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                          int dtype, const gqa_layout* layout, float q_scale, float k_scale,
                          float v_scale, int batch, int capacity, int chunk_len,
                          hipStream_t stream);

/* E4M3 block scales per 128-element FP4 head row (one per 16 elements). */
#define GQA_FP4_SCALES_PER_ROW 8

/*
 * Block scales of an FP4 cache. Strides are in bytes (the scales are one
 * byte each) and follow kv's: scales + b*stride_batch + kind*stride_kind +
 * g*stride_head + i*stride_row is the first of the 8 scales of K (kind 0) or
 * V (kind 1) row i of KV head g of sequence b; for a paged cache b is the
 * page id and i the row within the page, and stride_batch the page stride.
 * All four strides 0 select the contiguous layout [blocks][2][Hkv][rows][8]
 * (blocks = batch and rows = capacity, or num_pages and page_size). Strides
 * must be multiples of 4, stride_row at least 8, and stride_row times
 * capacity (paged: page_size) below 2^31; scales must be 4-byte aligned
 * device memory on the decode's device.
 */
typedef struct gqa_block_scales {
  const void* scales;      /* device uint8 E4M3 codes                  */
  int64_t stride_batch;    /* [2*Hkv*C*8]                             */
  int64_t stride_kind;     /* [Hkv*C*8]                               */
  int64_t stride_head;     /* [C*8]                                   */
  int64_t stride_row;      /* [8]                                     */
} gqa_block_scales;

/*
 * gqa_decode_fp4 -- gqa_decode_ex for a block-scaled FP4 cache (the K/V page
 * format named on the FlashInfer NVFP4 paged-context attention page: E2M1
 * values with E4M3 block scales, dequantised in on-chip memory).
 *
 * kv holds, per K or V head row, 64 bytes of E2M1 codes: element 2m in the
 * low nibble of byte m, element 2m + 1 in the high nibble; a code is 1 sign
 * bit, 2 exponent bits with bias 1 and 1 fraction bit (magnitudes 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6). `scales` gives each row 8 E4M3 codes (format as for
 * GQA_DTYPE_E4M3_KV), code k scaling elements 16k .. 16k + 15. Element value
 * = E2M1 value x block scale; k_scale and v_scale are per-tensor scales on
 * top (as in gqa_decode_typed), q and out are binary16. The decode is then
 * that of gqa_decode_typed on the element values, in fp32 (each element
 * value is an fp16 value, so it enters the arithmetic exactly).
 * layout: as for gqa_decode_ex, with kv strides counted in bytes (the code
 * bytes are kv's elements): the contiguous layout is [batch, 2, Hkv,
 * capacity, 64] (kv_stride_row 64). Paged caches need page_size >= 32
 * (FP4 tiles are 32 rows); chunk_len is then rounded up to a multiple of
 * 32. Scales of rows inside [0, L) that are NaN are outside the contract;
 * rows at or beyond L (codes and scales) are never read.
 * Returns GQA_ERR_NULL if scales (or scales->scales) is NULL, and the
 * errors of gqa_decode_ex; gqa_decode_typed and gqa_decode_ex reject
 * GQA_DTYPE_FP4_KV with GQA_ERR_BAD_ARG.
 */
int gqa_decode_fp4(const void* q, const void* kv, const gqa_block_scales* scales,
                   const int32_t* seq_lens, void* out, const gqa_layout* layout, float q_scale,
                   float k_scale, float v_scale, int batch, int capacity, int chunk_len,
                   hipStream_t stream);

/*
 * gqa_decode_workspace_bytes -- size of the fp32 partial-result workspace
 * the automatic split of gqa_decode (fp16, 32 query and 8 KV heads) needs
 * for (batch, capacity) on the current device (a per-segment descriptor
 * table plus two partial slots per workgroup). Other head counts and
 * forced splits may need more; the library grows its cached workspace as
 * needed.
 * Returns 0 for invalid sizes or when no device is available.
 */
size_t gqa_decode_workspace_bytes(int batch, int capacity);

/*
 * Environment: GQA_DECODE_WORKSPACE_LIMIT=<bytes> caps the workspace the
 * library allocates; a call that would need a larger one on its (device,
 * stream) fails with GQA_ERR_ALLOC and enqueues nothing (workspaces already
 * large enough are reused). A workspace that grows is allocated at twice
 * its previous size or more (below the limit, if one is set).
 * GQA_DECODE_LAUNCH_FORM sets the initial launch form (see
 * gqa_decode_set_launch_form). GQA_DECODE_COMBINE_MAX_GRID=<n> (1 .. 65536,
 * default 1024) caps the workgroups of the combine kernel, which then
 * take the segments in turns; results do not depend on it (used to test
 * those turns at small sizes).
 */

/*
 * gqa_decode_release_workspace -- free every cached workspace and ticket
 * array (all devices and streams), including buffers kept alive for graphs
 * captured earlier: every graph that captured a decode call before this
 * call must not be replayed afterwards. Synchronises each device that held
 * one. Safe to call at any time no decode is in flight on another host
 * thread.
 */
void gqa_decode_release_workspace(void);

/* How a decode call runs its combine step. */
typedef enum gqa_launch_form {
  GQA_LAUNCH_AUTO = 0,    /* single launch when capacity <= GQA_SINGLE_LAUNCH_MAX_CAPACITY
                             and batch * KV heads * capacity <= GQA_SINGLE_LAUNCH_MAX_ROWS,
                             or capacity <= GQA_SINGLE_LAUNCH_MAX_CAPACITY_FEW_ROWS and
                             batch * KV heads * capacity <= GQA_SINGLE_LAUNCH_MAX_FEW_ROWS;
                             else two kernels (the default)                                  */
  GQA_LAUNCH_SINGLE = 1,  /* one kernel: the last workgroup to finish a cut (sequence, KV
                             head) segment merges its partial results, found through a
                             per-segment atomic ticket                                       */
  GQA_LAUNCH_TWO = 2      /* two kernels: split-KV pieces, then the log-sum-exp combine      */
} gqa_launch_form;

/* Bounds within which GQA_LAUNCH_AUTO picks the single launch (short
 * caches, where saving the second launch outweighs the ticket round trips;
 * with few rows in all, caches up to twice as long). */
#define GQA_SINGLE_LAUNCH_MAX_CAPACITY 512
#define GQA_SINGLE_LAUNCH_MAX_ROWS 131072
#define GQA_SINGLE_LAUNCH_MAX_CAPACITY_FEW_ROWS 1024
#define GQA_SINGLE_LAUNCH_MAX_FEW_ROWS 32768

/*
 * gqa_decode_set_launch_form -- select the launch form of later calls (all
 * threads, all devices). Both forms cut the work identically and merge
 * partial results in the same fixed order, so they return the same bits;
 * they differ only in speed. Returns GQA_OK, or GQA_ERR_BAD_ARG for a value
 * outside gqa_launch_form. The environment variable GQA_DECODE_LAUNCH_FORM
 * (0, 1 or 2) sets the initial value.
 */
int gqa_decode_set_launch_form(int form);

/* Static, human-readable text for a status code (never NULL). */
const char* gqa_decode_status_string(int status);

/* Text of the calling thread's last failure ("" if none). Valid until the
 * thread's next failing call. */
const char* gqa_decode_last_error(void);

/*
 * Kernel timing aid. gqa_decode_profile_begin() makes subsequent decode
 * calls (any thread) attach start and stop HIP events to the dispatch of
 * each of their two kernels on the call's stream, so the events time the
 * kernels' execution. gqa_decode_profile_end() waits for the recorded
 * events, returns the summed durations in milliseconds of the pieces kernel
 * and of the combine kernel (no time for single-launch calls, whose pieces
 * kernel includes the combine) and the number of calls recorded, then stops
 * recording. Any output pointer may be NULL. Calls made while their stream
 * is being captured into a graph are not timed (nor counted).
 */
int gqa_decode_profile_begin(void);
int gqa_decode_profile_end(double* pieces_ms, double* combine_ms, int* calls);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* GQA_DECODE_H_ */

// C-ABI layer of libgqa_decode.so: argument validation, per-device set-up,
// workspace cache, launch, error reporting. Declarations and the contract
// are in include/gqa_decode.h.
//
// Conventions taken from the binding launchers described on the FlashInfer
// PR #5563 analysis page (section 2, launcher changes): every buffer must be
// on one device, the launch is scoped to that device rather than requiring
// it to be current (the previous current device is restored), and bad
// arguments are reported as errors before anything is launched. The exact-
// architecture gate mirrors the "exact SM110" loading rule of the PR #5052
// page (section 2): here the kernels are built for gfx950 only.

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "gqa_decode.h"
#include "launch.h"

namespace {

constexpr int kPiecesPerSlotDefault = 1;   // one piece per resident workgroup
constexpr int kMinPieceDefault = 128;      // cost units: two 64-row steps of a workgroup
constexpr int kSegCostDefault = 128;       // fixed cost of a segment, in row units
constexpr int kCombineMaxGrid = 1 << 16;   // combine workgroups, at most
// Default cap on the combine kernel's workgroups: beyond it each workgroup
// takes several segments in turn. Dispatching one workgroup per segment
// costs more than the turns once segments run into the thousands (batch
// 4096 x 8 KV heads: combine 19.2 -> 12.2 us; caps of 2048-8192 in between,
// 512 slower again).
constexpr int kCombineGridDefault = 1024;
constexpr int kShortCapacity = 256;        // caches of at most this many rows count as short
// Forced chunk lengths may not make the workspace exceed this.
constexpr size_t kMaxForcedWorkspace = (size_t)4 << 30;

thread_local std::string t_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return code;
}

struct DeviceInfo {
  bool ready = false;
  int status = GQA_OK;
  int cus = 0;
  int resident = 0;   // decode workgroups per CU
  std::string arch;
};

// fp32 partial results, cached per (device, stream), and the single-launch
// form's per-segment tickets (zeroed once when allocated; every call leaves
// them zero). A buffer that a call under graph capture used may be read and
// written by every replay of that graph, so it is never freed before
// gqa_decode_release_workspace: when it is outgrown it moves to g_retired.
struct Workspace {
  int device;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
  int* tickets;
  size_t ticket_bytes;
  bool ptr_captured;       // a captured call holds ptr
  bool tickets_captured;   // a captured call holds tickets
};

struct Retired {
  int device;
  void* ptr;
};

struct ProfileRecord {
  hipEvent_t ev[4];   // pieces start, stop; combine start, stop
  bool two_kernels;   // the combine events were recorded (two-launch form)
};

std::mutex g_mu;
// gqa_launch_form of later calls (guarded by g_mu).
int g_launch_form = -1;   // -1: not yet read from the environment
std::vector<DeviceInfo> g_devices;
std::vector<Workspace> g_workspaces;
std::vector<Retired> g_retired;   // outgrown buffers that captured graphs may still use
bool g_profiling = false;
// Event triples reused across profiling sessions; the first g_profile_used
// belong to the current session.
std::vector<ProfileRecord> g_profile;
size_t g_profile_used = 0;

int env_int(const char* name, int fallback, int lo, int hi) {
  const char* s = getenv(name);
  if (!s || !*s) return fallback;
  char* end = nullptr;
  long v = strtol(s, &end, 10);
  if (*end || v < lo || v > hi) return fallback;
  return (int)v;
}

// Per-device facts, cached. Caller holds g_mu.
const DeviceInfo& device_info(int dev) {
  if ((int)g_devices.size() <= dev) g_devices.resize(dev + 1);
  DeviceInfo& di = g_devices[dev];
  if (di.ready) return di;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    di.status = GQA_ERR_LAUNCH;
    di.arch = "?";
  } else {
    di.arch = prop.gcnArchName;
    di.cus = prop.multiProcessorCount;
    // gcnArchName looks like "gfx950:sramecc+:xnack-".
    di.status = strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                        (prop.gcnArchName[6] == 0 || prop.gcnArchName[6] == ':')
                    ? GQA_OK
                    : GQA_ERR_UNSUPPORTED_ARCH;
    if (di.status == GQA_OK) {
      di.resident = gqa::resident_workgroups_per_cu();
      if (di.resident <= 0) di.resident = 1;
    }
  }
  di.ready = true;
  return di;
}

// One equal piece per workgroup launched (times an optional factor), all of
// them resident at once, so the whole decode runs in a single round.
// Workgroups per CU: as many as fit (two) where segments are short or the
// tiles' arithmetic is heavy, so that one workgroup's segment-end merges
// and tile compute overlap the other's loads; one elsewhere (fewer, longer
// streams per CU). Measured: 16-bit formats, one is 1-3% faster on every
// workload with caches of 384 rows or more, two are 4-24% faster on
// caches of at most 256 rows when (sequence, KV head) segments outnumber
// the CUs; FP4 cache, two (one is 18-30% slower); E4M3 cache, one for
// caches of more than 256 rows with no more segments than CUs (1-12%
// faster: each workgroup then holds at most about two segments), else two
// (5-33% faster on many short segments). With few segments of at most 256
// rows, the better choice depends on the lengths (full lengths: one
// workgroup holds whole segments, two cut each in two; random lengths:
// two spread the work wider), so both formats keep their earlier choice
// there. GQA_DECODE_WG_PER_CU overrides it.
// row_align (1, or 16 / 32 for paged caches) rounds the piece and cost sizes up.
gqa::SplitConfig split_config(const DeviceInfo& di, int forced_piece, int row_align, int dtype,
                              long long segments, int capacity) {
  gqa::SplitConfig cfg;
  const int per_slot = env_int("GQA_DECODE_PIECES_PER_SLOT", kPiecesPerSlotDefault, 1, 64);
  auto up = [row_align](int v) { return (v + row_align - 1) / row_align * row_align; };
  const int resident = di.resident > 0 ? di.resident : 1;
  const int cus = di.cus > 0 ? di.cus : 256;
  const bool wide = dtype == GQA_DTYPE_F16 || dtype == GQA_DTYPE_BF16;
  const bool short_cache = capacity <= kShortCapacity, few = segments <= cus;
  const bool one = (wide && !(short_cache && !few)) ||
                   (dtype == GQA_DTYPE_E4M3_KV && few && !short_cache);
  const int per_cu = env_int("GQA_DECODE_WG_PER_CU", one ? 1 : resident, 1, resident);
  cfg.pieces = cus * per_cu * per_slot;
  // With more than one workgroup per CU, the first `cus` of the grid (one per
  // CU, dispatched first) take longer pieces than the rest, which share their
  // CU with an older workgroup (see the kernel's piece_lens).
  cfg.pieces_first = per_cu >= 2 && per_slot == 1 ? cus : cfg.pieces;
  // FP4: the younger workgroups take 40/64 of the older ones' rows (3-8%
  // faster on the long workloads, measured; the kernel keeps equal pieces
  // when they are short). E4M3 measured no gain.
  cfg.second_share =
      env_int("GQA_DECODE_SECOND_SHARE", dtype == GQA_DTYPE_FP4_KV ? 40 : 64, 1, 64);
  cfg.min_piece = up(env_int("GQA_DECODE_MIN_PIECE", kMinPieceDefault, 1, 1 << 30));
  cfg.seg_cost = up(env_int("GQA_DECODE_SEG_COST", kSegCostDefault, 0, 1 << 20));
  cfg.forced_piece = forced_piece > 0 ? up(forced_piece) : 0;
  cfg.row_align = row_align;
  cfg.combine_max_grid =
      env_int("GQA_DECODE_COMBINE_MAX_GRID", kCombineGridDefault, 1, kCombineMaxGrid);
  return cfg;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Device that owns `p`, or -1 if `p` is not device-accessible memory.
int pointer_device(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return -1;
  return attr.device;
}

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
    (void)hipGetLastError();
    return true;   // unknown: treat as capturing (no allocation, no synchronisation)
  }
  return cap != hipStreamCaptureStatusNone;
}

// Drop an outgrown buffer of (dev, stream): kept until release if a captured
// call holds it, else freed once the stream's earlier calls are done with it.
bool drop_buffer(int dev, hipStream_t stream, void* p, bool captured) {
  if (!p) return true;
  if (captured) {
    g_retired.push_back(Retired{dev, p});
    return true;
  }
  const bool ok = hipStreamSynchronize(stream) == hipSuccess && hipFree(p) == hipSuccess;
  if (!ok) (void)hipGetLastError();
  return ok;
}

// Size to allocate when `need` bytes outgrow `have`: at least double, so that
// buffers retired under graph capture add up to less than the live one.
size_t grown_size(size_t have, size_t need, size_t cap) {
  size_t n = have * 2 > need ? have * 2 : need;
  if (cap > 0 && n > cap) n = need;
  return (n + 255) & ~(size_t)255;
}

size_t workspace_cap() {
  const char* e = getenv("GQA_DECODE_WORKSPACE_LIMIT");
  return e ? (size_t)strtoull(e, nullptr, 10) : 0;
}

// Workspace of at least `bytes` for (dev, stream). Caller holds g_mu and
// has made `dev` current. Sets *status on error. Growing is refused under
// graph capture (no allocation or synchronisation may be captured).
void* get_workspace(int dev, hipStream_t stream, size_t bytes, int* status) {
  Workspace* ws = nullptr;
  for (Workspace& w : g_workspaces)
    if (w.device == dev && w.stream == stream) ws = &w;
  const bool capturing = stream_capturing(stream);
  if (ws && ws->bytes >= bytes) {
    ws->ptr_captured = ws->ptr_captured || capturing;
    return ws->ptr;
  }
  // Optional cap on the library's device memory (bytes; unset or 0: none).
  const size_t cap = workspace_cap();
  if (cap > 0 && bytes > cap) {
    *status = fail(GQA_ERR_ALLOC,
                   "gqa_decode: a workspace of %zu bytes exceeds GQA_DECODE_WORKSPACE_LIMIT=%zu",
                   bytes, cap);
    return nullptr;
  }
  if (capturing) {
    *status = fail(GQA_ERR_ALLOC,
                   "gqa_decode: this call needs a larger workspace on its stream; make a call "
                   "of this size (or larger) on the stream outside graph capture first");
    return nullptr;
  }
  if (!ws) {
    g_workspaces.push_back(Workspace{dev, stream, nullptr, 0, nullptr, 0, false, false});
    ws = &g_workspaces.back();
  }
  const size_t n = grown_size(ws->bytes, bytes, cap);
  if (ws->ptr) {
    const bool ok = drop_buffer(dev, stream, ws->ptr, ws->ptr_captured);
    ws->ptr = nullptr;
    ws->bytes = 0;
    ws->ptr_captured = false;
    if (!ok) {
      *status = fail(GQA_ERR_LAUNCH, "gqa_decode: could not release the old workspace");
      return nullptr;
    }
  }
  if (hipMalloc(&ws->ptr, n) != hipSuccess) {
    (void)hipGetLastError();
    ws->ptr = nullptr;
    *status = fail(GQA_ERR_ALLOC, "gqa_decode: hipMalloc of %zu workspace bytes failed", n);
    return nullptr;
  }
  ws->bytes = n;
  return ws->ptr;
}

// Ticket array of at least `count` ints for (dev, stream), all zero. Only
// allocated and cleared outside graph capture (a captured memset node is not
// used here), so the first call on a stream must be eager. Caller holds g_mu
// and has made `dev` current; the workspace entry exists.
int* get_tickets(int dev, hipStream_t stream, size_t count, int* status) {
  Workspace* ws = nullptr;
  for (Workspace& w : g_workspaces)
    if (w.device == dev && w.stream == stream) ws = &w;
  const size_t bytes = (count * sizeof(int) + 255) & ~(size_t)255;
  const bool capturing = stream_capturing(stream);
  if (ws && ws->ticket_bytes >= bytes) {
    ws->tickets_captured = ws->tickets_captured || capturing;
    return ws->tickets;
  }
  if (!ws || capturing) {
    *status = fail(GQA_ERR_ALLOC,
                   "gqa_decode: the first call with this batch size on a stream must run "
                   "outside graph capture");
    return nullptr;
  }
  const size_t n = grown_size(ws->ticket_bytes, bytes, 0);
  if (ws->tickets) {
    const bool ok = drop_buffer(dev, stream, ws->tickets, ws->tickets_captured);
    ws->tickets = nullptr;
    ws->ticket_bytes = 0;
    ws->tickets_captured = false;
    if (!ok) {
      *status = fail(GQA_ERR_LAUNCH, "gqa_decode: could not release the old ticket array");
      return nullptr;
    }
  }
  void* p = nullptr;
  if (hipMalloc(&p, n) != hipSuccess) {
    (void)hipGetLastError();
    *status = fail(GQA_ERR_ALLOC, "gqa_decode: hipMalloc of %zu ticket bytes failed", n);
    return nullptr;
  }
  if (hipMemsetAsync(p, 0, n, stream) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p);
    *status = fail(GQA_ERR_LAUNCH, "gqa_decode: clearing the ticket array failed");
    return nullptr;
  }
  ws->tickets = static_cast<int*>(p);
  ws->ticket_bytes = n;
  return ws->tickets;
}

// Strides resolved to bytes, with the address range each of q, kv (and the
// FP4 block scales) spans.
struct Resolved {
  gqa::Layout lay{};          // value-initialised: kv_scales stays null unless set
  size_t q_extent = 0, kv_extent = 0, table_bytes = 0, scale_extent = 0;
  int row_align = 1;
};

// kv_eb: bytes per kv element (2, or 1 for E4M3 and the FP4 code bytes);
// fp4: kv rows are 64 code bytes (element pairs) instead of 128 elements.
int resolve_layout(const gqa_layout* in, int batch, int capacity, size_t kv_eb, bool fp4,
                   Resolved* r) {
  const long long C = capacity;
  const long long row_elems = fp4 ? GQA_HEAD_DIM / 2 : GQA_HEAD_DIM;
  gqa_layout L;
  if (in) {
    L = *in;
  } else {
    L = gqa_layout{};
    L.q_stride_batch = (long long)GQA_NUM_Q_HEADS * GQA_HEAD_DIM;
    L.q_stride_head = GQA_HEAD_DIM;
    L.kv_stride_row = row_elems;
    L.kv_stride_head = C * row_elems;
    L.kv_stride_kind = GQA_NUM_KV_HEADS * C * row_elems;
    L.kv_stride_batch = 2 * L.kv_stride_kind;
  }
  if (L.num_q_heads == 0 && L.num_kv_heads == 0) {
    L.num_q_heads = GQA_NUM_Q_HEADS;
    L.num_kv_heads = GQA_NUM_KV_HEADS;
  }
  const int Hq = L.num_q_heads, Hkv = L.num_kv_heads;
  if (Hq <= 0 || Hkv <= 0 || Hkv > GQA_MAX_KV_HEADS || Hq % Hkv != 0 || Hq / Hkv > GQA_MAX_GROUP)
    return fail(GQA_ERR_BAD_ARG,
                "gqa_decode: %d query heads over %d KV heads: need a positive multiple with at "
                "most %d query heads per KV head and at most %d KV heads",
                Hq, Hkv, GQA_MAX_GROUP, GQA_MAX_KV_HEADS);
  if ((long long)batch * Hkv > GQA_MAX_SEGMENTS)
    return fail(GQA_ERR_BAD_SHAPE, "gqa_decode: batch * num_kv_heads exceeds 2^27");
  const long long qs[2] = {L.q_stride_batch, L.q_stride_head};
  const long long ks[4] = {L.kv_stride_batch, L.kv_stride_kind, L.kv_stride_head, L.kv_stride_row};
  const long long kLimit = 1LL << 40;   // elements; keeps every product below 2^62
  for (long long v : qs)
    if (v < 0 || v > kLimit || (v * 2) % 16 != 0)
      return fail(GQA_ERR_BAD_ARG, "gqa_decode: q strides must be >= 0 and keep rows 16-byte aligned");
  for (long long v : ks)
    if (v < 0 || v > kLimit || (v * (long long)kv_eb) % 16 != 0)
      return fail(GQA_ERR_BAD_ARG, "gqa_decode: kv strides must be >= 0 and keep rows 16-byte aligned");
  const long long row_bytes = row_elems * (long long)kv_eb;
  const long long sr = L.kv_stride_row * (long long)kv_eb;
  if (sr < row_bytes)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode: kv_stride_row must cover a %lld-byte row", row_bytes);
  if ((GQA_MAX_GROUP - 1) * L.q_stride_head * 2 + 2 * GQA_HEAD_DIM >= (1LL << 31))
    return fail(GQA_ERR_BAD_ARG, "gqa_decode: q_stride_head is too large for 32-bit offsets");
  const bool paged = L.block_table != nullptr;
  long long rows_per_block = C;
  if (paged) {
    const int P = L.page_size;
    const int min_page = fp4 ? 32 : 16;
    if (P < min_page || (P & (P - 1)) != 0)
      return fail(GQA_ERR_BAD_ARG, "gqa_decode: page_size must be a power of two >= %d, got %d",
                  min_page, P);
    if (L.max_pages <= 0 || L.num_pages <= 0)
      return fail(GQA_ERR_BAD_ARG, "gqa_decode: max_pages and num_pages must be positive");
    if ((long long)L.max_pages * P < C)
      return fail(GQA_ERR_BAD_ARG, "gqa_decode: capacity %d exceeds max_pages * page_size", capacity);
    if ((uintptr_t)L.block_table & 3u)
      return fail(GQA_ERR_MISALIGNED, "gqa_decode: block_table must be 4-byte aligned");
    rows_per_block = P;
  }
  if (sr * rows_per_block >= (1LL << 31))
    return fail(GQA_ERR_BAD_ARG,
                "gqa_decode: kv_stride_row times %s is too large for 32-bit offsets",
                paged ? "page_size" : "capacity");
  const long long blocks = paged ? L.num_pages : batch;
  r->q_extent = (size_t)(((long long)(batch - 1) * L.q_stride_batch +
                          (long long)(Hq - 1) * L.q_stride_head + GQA_HEAD_DIM) * 2);
  r->kv_extent = (size_t)(((blocks - 1) * L.kv_stride_batch + L.kv_stride_kind +
                           (long long)(Hkv - 1) * L.kv_stride_head +
                           (rows_per_block - 1) * L.kv_stride_row + row_elems) * (long long)kv_eb);
  r->table_bytes = paged ? (size_t)batch * (size_t)L.max_pages * 4 : 0;
  r->lay.q_sb = L.q_stride_batch * 2;
  r->lay.q_sh = L.q_stride_head * 2;
  r->lay.kv_sb = L.kv_stride_batch * (long long)kv_eb;
  r->lay.kv_sk = L.kv_stride_kind * (long long)kv_eb;
  r->lay.kv_sh = L.kv_stride_head * (long long)kv_eb;
  r->lay.kv_sr = sr;
  r->lay.block_table = L.block_table;
  r->lay.max_pages = paged ? L.max_pages : 0;
  r->lay.num_pages = paged ? L.num_pages : 0;
  int shift = 0;
  while (paged && (1 << shift) < L.page_size) ++shift;
  r->lay.page_shift = shift;
  r->row_align = paged ? (fp4 ? 32 : 16) : 1;
  r->lay.q_heads = Hq;
  r->lay.kv_heads = Hkv;
  return GQA_OK;
}

// FP4 block scales: strides (bytes), 4-byte alignment for the 4-byte loads,
// 32-bit offsets, and the address range. All-zero strides select the
// contiguous [blocks][2][Hkv][rows][8] layout (blocks = batch, or pages).
int resolve_scales(const gqa_block_scales* sc, int batch, int capacity, Resolved* r) {
  if (!sc || !sc->scales)
    return fail(GQA_ERR_NULL, "gqa_decode_fp4: the block scales must be non-NULL");
  const bool paged = r->lay.block_table != nullptr;
  const long long rows = paged ? (1LL << r->lay.page_shift) : capacity;
  const long long Hkv = r->lay.kv_heads;
  long long sb = sc->stride_batch, sk = sc->stride_kind, sh = sc->stride_head,
            sr = sc->stride_row;
  if (sb == 0 && sk == 0 && sh == 0 && sr == 0) {
    sr = GQA_FP4_SCALES_PER_ROW;
    sh = rows * sr;
    sk = Hkv * sh;
    sb = 2 * sk;
  }
  const long long st[4] = {sb, sk, sh, sr};
  for (long long v : st)
    if (v < 0 || v > (1LL << 40) || v % 4 != 0)
      return fail(GQA_ERR_BAD_ARG,
                  "gqa_decode_fp4: block-scale strides must be >= 0 and multiples of 4 bytes");
  if (sr < GQA_FP4_SCALES_PER_ROW)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode_fp4: the block-scale row stride must cover 8 bytes");
  if (sr * rows >= (1LL << 31))
    return fail(GQA_ERR_BAD_ARG,
                "gqa_decode_fp4: block-scale row stride times %s is too large for 32-bit offsets",
                paged ? "page_size" : "capacity");
  if ((uintptr_t)sc->scales & 3u)
    return fail(GQA_ERR_MISALIGNED, "gqa_decode_fp4: the block scales must be 4-byte aligned");
  const long long blocks = paged ? r->lay.num_pages : batch;
  r->scale_extent = (size_t)((blocks - 1) * sb + sk + (Hkv - 1) * sh + (rows - 1) * sr +
                             GQA_FP4_SCALES_PER_ROW);
  r->lay.kv_scales = sc->scales;
  r->lay.sc_sb = sb;
  r->lay.sc_sk = sk;
  r->lay.sc_sh = sh;
  r->lay.sc_sr = sr;
  return GQA_OK;
}

int check_args(const void* q, const void* kv, const int32_t* seq_lens, const void* out, int batch,
               int capacity, int chunk_len) {
  if (!q || !kv || !seq_lens || !out)
    return fail(GQA_ERR_NULL, "gqa_decode: q, kv, seq_lens and out must be non-NULL");
  if (batch <= 0 || capacity <= 0)
    return fail(GQA_ERR_BAD_SHAPE, "gqa_decode: batch (%d) and capacity (%d) must be positive",
                batch, capacity);
  if (batch > (1 << 24))
    return fail(GQA_ERR_BAD_SHAPE, "gqa_decode: batch %d exceeds the supported 2^24", batch);
  if (capacity > GQA_MAX_CAPACITY)
    return fail(GQA_ERR_BAD_SHAPE, "gqa_decode: capacity %d exceeds the supported %d", capacity,
                GQA_MAX_CAPACITY);
  if (chunk_len < 0)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode: chunk_len must be >= 0, got %d", chunk_len);
  if (((uintptr_t)q | (uintptr_t)kv | (uintptr_t)out) & 15u)
    return fail(GQA_ERR_MISALIGNED, "gqa_decode: q, kv and out must be 16-byte aligned");
  if ((uintptr_t)seq_lens & 3u)
    return fail(GQA_ERR_MISALIGNED, "gqa_decode: seq_lens must be 4-byte aligned");
  return GQA_OK;
}

int check_alias(const void* q, const void* kv, const int32_t* seq_lens, const void* out,
                int batch, const Resolved& r) {
  const size_t ob = (size_t)batch * r.lay.q_heads * GQA_HEAD_DIM * 2;
  if (overlaps(out, ob, q, r.q_extent) || overlaps(out, ob, kv, r.kv_extent) ||
      overlaps(out, ob, seq_lens, (size_t)batch * 4) ||
      (r.table_bytes && overlaps(out, ob, r.lay.block_table, r.table_bytes)) ||
      (r.scale_extent && overlaps(out, ob, r.lay.kv_scales, r.scale_extent)))
    return fail(GQA_ERR_ALIAS,
                "gqa_decode: out must not overlap q, kv, seq_lens, block_table or the block scales");
  return GQA_OK;
}

// noalloc: take the fixed device scratch (gqa::scratch_area) instead of the
// cached per-stream workspace, and allocate nothing (no timing events
// either); shapes whose partials or tickets do not fit it are rejected.
int decode_impl(const void* q, const void* kv, const gqa_block_scales* scales,
                const int32_t* seq_lens, void* out, int dtype, const gqa_layout* layout,
                float q_scale, float k_scale, float v_scale, int batch, int capacity,
                int chunk_len, hipStream_t stream, bool noalloc = false) {
  int st = check_args(q, kv, seq_lens, out, batch, capacity, chunk_len);
  if (st != GQA_OK) return st;
  if (dtype != GQA_DTYPE_F16 && dtype != GQA_DTYPE_BF16 && dtype != GQA_DTYPE_E4M3_KV &&
      dtype != GQA_DTYPE_FP4_KV)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode: unknown dtype %d", dtype);
  const bool fp4 = dtype == GQA_DTYPE_FP4_KV;
  if (fp4 != (scales != nullptr))
    return fail(fp4 ? GQA_ERR_NULL : GQA_ERR_BAD_ARG,
                fp4 ? "gqa_decode_fp4: the block scales must be non-NULL"
                    : "gqa_decode: an FP4 cache goes through gqa_decode_fp4");
  Resolved res;
  st = resolve_layout(layout, batch, capacity, dtype == GQA_DTYPE_E4M3_KV || fp4 ? 1 : 2, fp4,
                      &res);
  if (st != GQA_OK) return st;
  if (fp4) {
    st = resolve_scales(scales, batch, capacity, &res);
    if (st != GQA_OK) return st;
  }
  st = check_alias(q, kv, seq_lens, out, batch, res);
  if (st != GQA_OK) return st;
  if (!std::isfinite(q_scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(GQA_ERR_BAD_ARG, "gqa_decode: q_scale, k_scale and v_scale must be finite");

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    (void)hipGetLastError();
    return fail(GQA_ERR_NO_DEVICE, "gqa_decode: no HIP device is visible");
  }
  const int dev = pointer_device(q);
  if (dev < 0) return fail(GQA_ERR_DEVICE_MISMATCH, "gqa_decode: q is not device memory");
  if (pointer_device(kv) != dev || pointer_device(out) != dev || pointer_device(seq_lens) != dev ||
      (res.lay.block_table && pointer_device(res.lay.block_table) != dev) ||
      (res.lay.kv_scales && pointer_device(res.lay.kv_scales) != dev))
    return fail(GQA_ERR_DEVICE_MISMATCH,
                "gqa_decode: q, kv, seq_lens, out (and block_table, block scales) must be device "
                "memory on one device");

  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) prev = -1;
  if (prev != dev && hipSetDevice(dev) != hipSuccess)
    return fail(GQA_ERR_LAUNCH, "gqa_decode: hipSetDevice(%d) failed", dev);

  st = GQA_OK;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    const DeviceInfo& di = device_info(dev);
    if (di.status != GQA_OK) {
      st = fail(di.status, "gqa_decode: device %d is %s; this library is built for gfx950", dev,
                di.arch.c_str());
    } else {
      const int Hkv = res.lay.kv_heads, group = res.lay.q_heads / res.lay.kv_heads;
      const gqa::SplitConfig cfg =
          split_config(di, chunk_len, res.row_align, dtype, (long long)batch * Hkv, capacity);
      const long long grid = gqa::grid_for(batch, capacity, Hkv, cfg);
      const size_t pbytes =
          grid > 0 ? gqa::segment_bytes_for_batch(batch, Hkv) +
                         gqa::partial_bytes_for_grid(grid, group)
                   : 0;
      if (grid <= 0 || grid >= (1LL << 24)) {
        // a dispatch holds below 2^32 work items: 2^24 workgroups of 256
        st = fail(GQA_ERR_BAD_ARG, "gqa_decode: the split needs 2^24 or more workgroups");
      } else if (chunk_len > 0 && pbytes > kMaxForcedWorkspace) {
        st = fail(GQA_ERR_BAD_ARG,
                  "gqa_decode: chunk_len %d is too small for batch %d and capacity %d "
                  "(partials would need %zu bytes)",
                  chunk_len, batch, capacity, pbytes);
      } else {
        if (g_launch_form < 0)
          g_launch_form = env_int("GQA_DECODE_LAUNCH_FORM", GQA_LAUNCH_AUTO, 0, 2);
        const long long rows = (long long)batch * Hkv * capacity;
        const bool single =
            g_launch_form == GQA_LAUNCH_SINGLE ||
            (g_launch_form == GQA_LAUNCH_AUTO &&
             ((capacity <= GQA_SINGLE_LAUNCH_MAX_CAPACITY && rows <= GQA_SINGLE_LAUNCH_MAX_ROWS) ||
              (capacity <= GQA_SINGLE_LAUNCH_MAX_CAPACITY_FEW_ROWS &&
               rows <= GQA_SINGLE_LAUNCH_MAX_FEW_ROWS)));
        void* ws = nullptr;
        int* tickets = nullptr;
        if (noalloc) {
          void* base = nullptr;
          const size_t ticket_need = (size_t)batch * Hkv * sizeof(int);
          const size_t room = gqa::kScratchBytes - gqa::kScratchTicketBytes;
          const hipError_t se = gqa::scratch_area(dev, &base);
          if (se != hipSuccess) {
            (void)hipGetLastError();
            st = fail(GQA_ERR_LAUNCH, "gqa_decode_ex_noalloc: the scratch address of device %d "
                      "could not be looked up: %s", dev, hipGetErrorString(se));
          } else if (pbytes > room) {
            st = fail(GQA_ERR_BAD_SHAPE,
                      "gqa_decode_ex_noalloc: this call needs %zu bytes of partial results and "
                      "segment descriptors; the fixed scratch holds %zu (use gqa_decode_ex)",
                      pbytes, room);
          } else if (single && ticket_need > gqa::kScratchTicketBytes) {
            st = fail(GQA_ERR_BAD_SHAPE,
                      "gqa_decode_ex_noalloc: the single launch needs %zu ticket bytes "
                      "(batch x KV heads x 4); the fixed scratch holds %zu (use the two-kernel "
                      "form or gqa_decode_ex)",
                      ticket_need, gqa::kScratchTicketBytes);
          } else {
            tickets = single ? static_cast<int*>(base) : nullptr;
            ws = static_cast<char*>(base) + gqa::kScratchTicketBytes;
          }
        } else {
          ws = get_workspace(dev, stream, pbytes, &st);
          if (ws && single) tickets = get_tickets(dev, stream, (size_t)batch * Hkv, &st);
        }
        if (ws && (tickets || !single)) {
          // Scores are formed as dot * q_scale * k_scale / sqrt(128) * log2(e),
          // so the kernel can use the hardware base-2 exponential.
          const double scale = (double)q_scale * (double)k_scale /
                               std::sqrt((double)GQA_HEAD_DIM) * 1.4426950408889634;
          hipEvent_t* ev = nullptr;
          hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
          if (!noalloc && g_profiling && hipStreamIsCapturing(stream, &cap) == hipSuccess &&
              cap == hipStreamCaptureStatusNone) {
            if (g_profile_used == g_profile.size()) {
              ProfileRecord rec;
              bool ok = true;
              for (int i = 0; i < 4; ++i) ok = ok && hipEventCreate(&rec.ev[i]) == hipSuccess;
              if (ok) g_profile.push_back(rec);
            }
            if (g_profile_used < g_profile.size()) {
              ProfileRecord& rec = g_profile[g_profile_used++];
              rec.two_kernels = !single;
              ev = rec.ev;
            }
          }
          const gqa::ElemType elem = dtype == GQA_DTYPE_BF16      ? gqa::ElemType::kBf16
                                     : dtype == GQA_DTYPE_E4M3_KV ? gqa::ElemType::kE4m3Kv
                                     : fp4                        ? gqa::ElemType::kFp4Kv
                                                                  : gqa::ElemType::kF16;
          const hipError_t e = gqa::launch_decode(q, kv, seq_lens, out, elem, res.lay,
                                                  (float)scale, v_scale, batch, capacity, cfg,
                                                  grid, ws, tickets, stream, ev);
          if (e != hipSuccess)
            st = fail(GQA_ERR_LAUNCH, "gqa_decode: kernel launch failed: %s", hipGetErrorString(e));
        }
      }
    }
  }
  if (prev >= 0 && prev != dev) (void)hipSetDevice(prev);
  return st;
}

}  // namespace

extern "C" {

int gqa_decode(const void* q, const void* kv, const int32_t* seq_lens, void* out, float q_scale,
               int batch, int capacity, hipStream_t stream) {
  return decode_impl(q, kv, nullptr, seq_lens, out, GQA_DTYPE_F16, nullptr, q_scale, 1.0f, 1.0f, batch,
                     capacity, 0, stream);
}

int gqa_decode_chunked(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                       float q_scale, int batch, int capacity, int chunk_len, hipStream_t stream) {
  return decode_impl(q, kv, nullptr, seq_lens, out, GQA_DTYPE_F16, nullptr, q_scale, 1.0f, 1.0f, batch,
                     capacity, chunk_len, stream);
}

int gqa_decode_typed(const void* q, const void* kv, const int32_t* seq_lens, void* out, int dtype,
                     float q_scale, float k_scale, float v_scale, int batch, int capacity,
                     int chunk_len, hipStream_t stream) {
  if (dtype == GQA_DTYPE_FP4_KV)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode_typed: an FP4 cache goes through gqa_decode_fp4");
  return decode_impl(q, kv, nullptr, seq_lens, out, dtype, nullptr, q_scale, k_scale, v_scale, batch,
                     capacity, chunk_len, stream);
}

int gqa_decode_ex(const void* q, const void* kv, const int32_t* seq_lens, void* out, int dtype,
                  const gqa_layout* layout, float q_scale, float k_scale, float v_scale,
                  int batch, int capacity, int chunk_len, hipStream_t stream) {
  if (dtype == GQA_DTYPE_FP4_KV)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode_ex: an FP4 cache goes through gqa_decode_fp4");
  return decode_impl(q, kv, nullptr, seq_lens, out, dtype, layout, q_scale, k_scale, v_scale,
                     batch, capacity, chunk_len, stream);
}

int gqa_decode_ex_noalloc(const void* q, const void* kv, const int32_t* seq_lens, void* out,
                          int dtype, const gqa_layout* layout, float q_scale, float k_scale,
                          float v_scale, int batch, int capacity, int chunk_len,
                          hipStream_t stream) {
  if (dtype == GQA_DTYPE_FP4_KV)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode_ex_noalloc: an FP4 cache goes through gqa_decode_fp4");
  return decode_impl(q, kv, nullptr, seq_lens, out, dtype, layout, q_scale, k_scale, v_scale,
                     batch, capacity, chunk_len, stream, true);
}

int gqa_decode_fp4(const void* q, const void* kv, const gqa_block_scales* scales,
                   const int32_t* seq_lens, void* out, const gqa_layout* layout, float q_scale,
                   float k_scale, float v_scale, int batch, int capacity, int chunk_len,
                   hipStream_t stream) {
  return decode_impl(q, kv, scales, seq_lens, out, GQA_DTYPE_FP4_KV, layout,
                     q_scale, k_scale, v_scale, batch, capacity, chunk_len, stream);
}

size_t gqa_decode_workspace_bytes(int batch, int capacity) {
  if (batch <= 0 || capacity <= 0 || batch > (1 << 24) || capacity > GQA_MAX_CAPACITY) return 0;
  int dev = 0, ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0 || hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  const DeviceInfo& di = device_info(dev);
  if (di.status != GQA_OK) return 0;
  const long long grid =
      gqa::grid_for(batch, capacity, GQA_NUM_KV_HEADS,
                    split_config(di, 0, 1, GQA_DTYPE_F16, (long long)batch * GQA_NUM_KV_HEADS,
                                 capacity));
  return gqa::segment_bytes_for_batch(batch, GQA_NUM_KV_HEADS) +
         gqa::partial_bytes_for_grid(grid, GQA_NUM_Q_HEADS / GQA_NUM_KV_HEADS);
}

void gqa_decode_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) prev = -1;
  for (Workspace& w : g_workspaces) {
    if (hipSetDevice(w.device) == hipSuccess) {
      (void)hipDeviceSynchronize();
      if (w.ptr) (void)hipFree(w.ptr);
      if (w.tickets) (void)hipFree(w.tickets);
    }
  }
  for (Retired& r : g_retired) {
    if (hipSetDevice(r.device) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(r.ptr);
    }
  }
  g_workspaces.clear();
  g_retired.clear();
  if (prev >= 0) (void)hipSetDevice(prev);
  (void)hipGetLastError();
}

int gqa_decode_set_launch_form(int form) {
  if (form < GQA_LAUNCH_AUTO || form > GQA_LAUNCH_TWO)
    return fail(GQA_ERR_BAD_ARG, "gqa_decode_set_launch_form: unknown form %d", form);
  std::lock_guard<std::mutex> lock(g_mu);
  g_launch_form = form;
  return GQA_OK;
}

const char* gqa_decode_status_string(int status) {
  switch (status) {
    case GQA_OK: return "success";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_BAD_SHAPE: return "invalid batch or capacity";
    case GQA_ERR_MISALIGNED: return "misaligned buffer";
    case GQA_ERR_ALIAS: return "output overlaps an input";
    case GQA_ERR_NO_DEVICE: return "no HIP device";
    case GQA_ERR_UNSUPPORTED_ARCH: return "device is not gfx950";
    case GQA_ERR_ALLOC: return "workspace allocation failed";
    case GQA_ERR_LAUNCH: return "kernel launch or HIP runtime call failed";
    case GQA_ERR_BAD_ARG: return "invalid scalar argument";
    case GQA_ERR_DEVICE_MISMATCH: return "buffer not device memory or on another device";
    default: return "unknown status";
  }
}

const char* gqa_decode_last_error(void) { return t_last_error.c_str(); }

int gqa_decode_profile_begin(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_profiling = true;
  g_profile_used = 0;
  return GQA_OK;
}

int gqa_decode_profile_end(double* pieces_ms, double* combine_ms, int* calls) {
  std::lock_guard<std::mutex> lock(g_mu);
  double tp = 0.0, tc = 0.0;
  int n = 0, st = GQA_OK;
  for (size_t i = 0; i < g_profile_used; ++i) {
    const ProfileRecord& r = g_profile[i];
    float a = 0.f, c = 0.f;
    if (hipEventSynchronize(r.ev[r.two_kernels ? 3 : 1]) != hipSuccess ||
        hipEventElapsedTime(&a, r.ev[0], r.ev[1]) != hipSuccess ||
        (r.two_kernels && hipEventElapsedTime(&c, r.ev[2], r.ev[3]) != hipSuccess)) {
      (void)hipGetLastError();
      st = fail(GQA_ERR_LAUNCH, "gqa_decode_profile_end: event query failed");
    } else {
      tp += a;
      tc += c;
      ++n;
    }
  }
  g_profile_used = 0;
  g_profiling = false;
  if (pieces_ms) *pieces_ms = tp;
  if (combine_ms) *combine_ms = tc;
  if (calls) *calls = n;
  return st;
}

}  // extern "C"

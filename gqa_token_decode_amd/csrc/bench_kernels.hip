// Measurement kernels for the benchmark (libgqa_bench.so), not part of the
// decode library or its ABI:
//   - a plain streaming read, the ceiling that HBM reads reach on this GPU
//     for a given byte count (the decode's roofline is the 8 TB/s peak; this
//     is what a kernel that does nothing but read achieves);
//   - a kernel that keeps every SIMD's vector ALU busy with independent fp32
//     FMAs, a known load for checking how the SQ utilisation counters are
//     normalised.
// Both are timed with start/stop events attached to their dispatches, so the
// times cover the kernels' execution only.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr unsigned kBufferFlags = 0x00020000;   // raw buffer resource word 3 (gfx9 family)
constexpr int kNonTemporal = 2;

// Workgroup w reads bytes [w * share, (w + 1) * share) of the buffer (share a
// multiple of 1 KiB; the last workgroups up to `bytes`, or nothing) with
// 16-byte buffer loads that write straight into LDS, the way the decode
// streams its K/V tiles: wave v takes 1 KiB chunks in groups of NF (chunks
// NF g .. NF g + NF - 1 for g = v, v + 4, ...), two groups in flight (a
// two-stage LDS pipeline: before issuing group g + 1 it waits for group g).
// Chunks past the share read as zeros without a memory access (buffer
// bounds). Of the probes tried on gfx950 (global loads, plain or
// nontemporal, 4 to 16 in flight per lane; this form with 4 or 8 KiB per
// group; two and four concurrent address streams per workgroup), this one
// read fastest. A word of LDS goes to sink only if it equals a value it
// practically never takes, so the loads are not removed.
template <int NF>
__global__ __launch_bounds__(kThreads) void stream_read(const char* __restrict__ buf,
                                                        long long bytes, long long share,
                                                        unsigned* sink) {
  __shared__ __attribute__((aligned(16))) char st[kThreads / 64][2][NF * 1024];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long lo = (long long)blockIdx.x * share;
  const long long hi = lo + share < bytes ? lo + share : bytes;
  const int n = hi > lo ? (int)(hi - lo) : 0;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(buf + (n > 0 ? lo : 0)), 0, n, kBufferFlags);
  const int chunks = (n + 1023) / 1024;
  int par = 0;
  for (int g = wv; g * NF < chunks; g += kThreads / 64) {
#pragma unroll
    for (int k = 0; k < NF; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(&st[wv][par][k * 1024]), 16,
                                               (g * NF + k) * 1024 + 16 * lane, 0, 0,
                                               kNonTemporal);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NF) : "memory");
    par ^= 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const unsigned x = *reinterpret_cast<volatile unsigned*>(&st[wv][0][lane * 4]);
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

// 8 independent FMA chains per lane, `iters` steps each: 8 * iters VALU FMAs
// per wave plus a few instructions of set-up and exit.
__global__ __launch_bounds__(kThreads) void valu_load(int iters, unsigned* sink) {
  float a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = (float)threadIdx.x * 1e-3f + (float)k;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = __builtin_fmaf(a[k], 0.999999f, 1e-7f);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += a[k];
  if (s == -1.0f) sink[blockIdx.x] = 1u;
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return n;
}

}  // namespace

extern "C" {

// Time `reps` streaming reads of `bytes` (a multiple of 16) on `stream`: read
// r covers [base + (r % copies) * stride, + bytes), so consecutive reads touch
// different copies (cold caches when the copies together exceed the caches).
// wgs_per_cu workgroups per compute unit share the bytes equally (in 1 KiB
// units); kib_in_flight (4 or 8) is the group size of each wave's two-stage
// pipeline. `sink` needs 4 bytes per workgroup (never written in practice).
// us_out[r] receives read r's duration in microseconds. Returns 0, or -1 on
// a bad argument or a HIP error (after which us_out is undefined).
// Synchronises the stream.
int gqa_bench_stream_read(const void* base, size_t bytes, size_t stride, int copies, int reps,
                          int wgs_per_cu, int kib_in_flight, void* sink, hipStream_t stream,
                          float* us_out) {
  if (!base || !sink || !us_out || bytes < 16 || (bytes & 15) || copies < 1 || reps < 1 ||
      wgs_per_cu < 1 || (kib_in_flight != 4 && kib_in_flight != 8))
    return -1;
  const int cus = cu_count();
  if (cus <= 0) return -1;
  const long long grid = (long long)cus * wgs_per_cu;
  const long long share = ((long long)((bytes + grid - 1) / grid) + 1023) / 1024 * 1024;
  if (share >= (1LL << 31)) return -1;   // 32-bit buffer offsets
  hipEvent_t ev[2];
  if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) return -1;
  int rc = 0;
  for (int r = 0; r < reps && rc == 0; ++r) {
    const char* p = static_cast<const char*>(base) + (size_t)(r % copies) * stride;
    if (kib_in_flight == 8)
      hipExtLaunchKernelGGL(stream_read<8>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                            ev[0], ev[1], 0, p, (long long)bytes, share,
                            static_cast<unsigned*>(sink));
    else
      hipExtLaunchKernelGGL(stream_read<4>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                            ev[0], ev[1], 0, p, (long long)bytes, share,
                            static_cast<unsigned*>(sink));
    float ms = 0.f;
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(ev[1]) != hipSuccess ||
        hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess)
      rc = -1;
    us_out[r] = ms * 1e3f;
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  return rc;
}

// Run the VALU load `reps` times (wgs_per_cu workgroups of 256 per compute
// unit, `iters` FMA steps of 8 chains per lane); us_out[r] receives each
// duration. Returns 0, or -1 on a HIP error. Synchronises the stream.
int gqa_bench_valu_load(int iters, int reps, int wgs_per_cu, void* sink, hipStream_t stream,
                        float* us_out) {
  if (!sink || !us_out || iters < 1 || reps < 1 || wgs_per_cu < 1) return -1;
  const int cus = cu_count();
  if (cus <= 0) return -1;
  hipEvent_t ev[2];
  if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) return -1;
  int rc = 0;
  for (int r = 0; r < reps && rc == 0; ++r) {
    hipExtLaunchKernelGGL(valu_load, dim3((unsigned)(cus * wgs_per_cu)), dim3(kThreads), 0, stream,
                          ev[0], ev[1], 0, iters, static_cast<unsigned*>(sink));
    float ms = 0.f;
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(ev[1]) != hipSuccess ||
        hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess)
      rc = -1;
    us_out[r] = ms * 1e3f;
  }
  (void)hipEventDestroy(ev[0]);
  (void)hipEventDestroy(ev[1]);
  return rc;
}

}  // extern "C"

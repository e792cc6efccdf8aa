// Measurement helper, not part of the drafting path: a pure-read stream over a
// device buffer, the achievable ceiling that the draft step's HBM roofline
// fraction is compared with.  Built into its own library (libdspark_probe.so).
//
// Variants (all read every byte once and fold it, so no load is removed):
//   kU          16-byte loads in flight per lane per iteration (4, 8 or 16);
//   kNT         nontemporal loads (no reuse expected in the caches);
//   kBlocked    workgroup b reads one contiguous slice of the buffer (as a
//               draft-step slab reads its own columns) instead of a grid-wide
//               interleave.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (kNT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ unsigned fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Chunks [lo, hi) of 16 bytes, lane offset `first`, step `step` between the
// kU loads of one iteration (the whole iteration advances kU * step).  Every
// index a load uses is below hi: the main loop runs only while the last of
// its kU indexes is, and the tail takes one chunk at a time.
template <int kU, bool kNT>
__device__ __forceinline__ unsigned fold_range(const u32x4* p, size_t first, size_t hi,
                                               size_t step) {
  unsigned acc = 0u;
  size_t i = first;
  for (; i + (kU - 1) * step < hi; i += kU * step) {
    u32x4 v[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) v[j] = load16<kNT>(p + i + j * step);
#pragma unroll
    for (int j = 0; j < kU; ++j) acc ^= fold(v[j]);
  }
  for (; i < hi; i += step) acc ^= fold(load16<kNT>(p + i));
  return acc;
}

// One word per workgroup is written only if the fold hits a fixed pattern,
// which keeps the result live without a store per workgroup.
template <int kU, bool kNT, bool kBlocked>
__global__ __launch_bounds__(kThreads) void read_stream(const u32x4* p, size_t n16,
                                                        unsigned* sink) {
  unsigned acc;
  if constexpr (kBlocked) {
    // slice of workgroup b: chunks [b * n16 / grid, (b + 1) * n16 / grid)
    const size_t lo = (size_t)blockIdx.x * n16 / gridDim.x;
    const size_t hi = (size_t)(blockIdx.x + 1) * n16 / gridDim.x;
    acc = fold_range<kU, kNT>(p, lo + threadIdx.x, hi, kThreads);
  } else {
    const size_t stride = (size_t)gridDim.x * kThreads;
    acc = fold_range<kU, kNT>(p, (size_t)blockIdx.x * kThreads + threadIdx.x, n16, stride);
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

template <int kU, bool kNT>
hipError_t launch_u(bool blocked, const u32x4* p, size_t n16, unsigned* sink, int grid,
                    hipStream_t st) {
  if (blocked)
    hipLaunchKernelGGL((read_stream<kU, kNT, true>), dim3(grid), dim3(kThreads), 0, st, p, n16,
                       sink);
  else
    hipLaunchKernelGGL((read_stream<kU, kNT, false>), dim3(grid), dim3(kThreads), 0, st, p, n16,
                       sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) from `buf` with `grid`
// workgroups of 256 threads on `stream`; `sink` holds at least `grid` words.
// `unroll` is 4, 8 or 16 loads in flight per lane, `nontemporal` and `blocked`
// are 0 or 1 (see the variants above).  Returns 0 on success, 1 on a bad
// argument, 2 on a launch error.
int dspark_probe_read_ex(const void* buf, size_t bytes, unsigned* sink, int grid, int unroll,
                         int nontemporal, int blocked, void* stream) {
  if (!buf || !sink || grid < 1 || (bytes & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (nontemporal & ~1) != 0 ||
      (blocked & ~1) != 0)
    return 1;
  const u32x4* p = reinterpret_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool bl = blocked != 0;
  hipError_t e;
  if (unroll == 4)
    e = nontemporal ? launch_u<4, true>(bl, p, n16, sink, grid, st)
                    : launch_u<4, false>(bl, p, n16, sink, grid, st);
  else if (unroll == 8)
    e = nontemporal ? launch_u<8, true>(bl, p, n16, sink, grid, st)
                    : launch_u<8, false>(bl, p, n16, sink, grid, st);
  else if (unroll == 16)
    e = nontemporal ? launch_u<16, true>(bl, p, n16, sink, grid, st)
                    : launch_u<16, false>(bl, p, n16, sink, grid, st);
  else
    return 1;
  return e == hipSuccess ? 0 : 2;
}

// The plain variant: four loads in flight, cached, grid-wide interleave.
int dspark_probe_read(const void* buf, size_t bytes, unsigned* sink, int grid, void* stream) {
  return dspark_probe_read_ex(buf, bytes, sink, grid, 4, 0, 0, stream);
}

}  // extern "C"

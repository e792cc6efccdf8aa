// Hardware-aware prefix scheduler [P1 "DSpark" §4.1 (eqs. B, tau, Theta; the
// global sort), §4.2 (early stop), §4.3 (the asynchronous variant); P3
// スケジューラ; P2 "按负载决定验证多少"].
//
// The global sort orders the N = R*gamma candidates by key (a descending, flat
// index ascending).  Its output position of candidate i is the number of
// candidates whose key comes first, and the prefix sum G at that position is
// the sum of q over the same candidates -- both are counts over all pairs, so
// no sort is run.  One launch:
//   1. Every workgroup (ceil(N / 4) of them, one candidate per wave) stages
//      the N keys (bits(a) << 13 | 8191 - i; larger = earlier) and
//      q_j = rint(a_j * 2^32) in LDS; lane s compares its wave's candidate
//      with keys s, s+64, ... and the 64 lanes add up rank_i and G_i.  q_j
//      are integers below 2^33 and every partial sum stays below 2^53, so G
//      is exact in fp64 whatever the order of the additions.  Candidate i
//      writes, at its position p = rank_i, G_p and its request i / gamma; the
//      last one also writes G_N.
//   2. The last workgroup to finish (two levels of device-scope counters,
//      reset by the workgroups that complete them) forms
//      Theta_fix(b) = (double)(R*2^32 + G_b) * sps[R + b] at every position;
//      b* = the first b with Theta_fix(b+1) <= Theta_fix(b) (N if none);
//      ell[r] = number of positions below b* that hold a candidate of r (a
//      prefix of r's block, because rows of a are non-increasing).
// The asynchronous variant ranks a_lag (with G) and a_cur (requests by
// position) in the same launch (blockIdx.y); the last workgroup takes K = the
// b in 0..N with the largest Theta_fix(b) (the smallest b on a tie) and
// admits the first K positions of a_cur's order.
//
// Results cross workgroups as device-scope atomic stores and loads, which the
// L2 of each XCD does not hold back, and each workgroup's stores have
// completed before it raises a counter; no cache-wide fence is needed.
#include "dspark_kernels.h"
#include "dspark_device.h"

namespace dspark {

namespace {

constexpr int kMaxN = 8192;         // 13 index bits in the key
constexpr int kRankThreads = 256;   // 4 waves, one candidate each
constexpr int kPerWg = 4;           // candidates per workgroup
constexpr int kChunk = 2048;        // keys staged in LDS at a time
constexpr int kGroups = 16;         // first-level finishing counters
constexpr int kCounterStride = 32;  // words: one 128-byte line per counter
constexpr size_t kCounterBytes = (size_t)(1 + kGroups) * kCounterStride * 4;

// Larger key = earlier in the sorted order: a descending, then flat index
// ascending.  Non-positive and NaN a sort as 0.  bits(a) < 2^31 for a >= 0, so
// the key fits 44 bits.
__device__ __forceinline__ unsigned long long sched_key(float f, int i) {
  const uint32_t bits = (f > 0.0f) ? __float_as_uint(f) : 0u;
  return ((unsigned long long)bits << 13) | (uint32_t)(kMaxN - 1 - i);
}

// q = round-half-even(a * 2^32) as an exact integer in fp64 (0 where the key
// treats a as 0).
__device__ __forceinline__ double q_of(float f) {
  return rint((double)((f > 0.0f) ? f : 0.0f) * 4294967296.0);
}

struct KeyQ {
  unsigned long long key;
  double q;
};

__device__ __forceinline__ void tally(const KeyQ& v, unsigned long long ki, int& cnt, double& G) {
  const bool ahead = v.key > ki;
  cnt += ahead ? 1 : 0;
  G += ahead ? v.q : 0.0;
}

// rank and G of candidate `ki` against all N candidates of `src`; the 64
// lanes of a wave share one candidate and return the totals in every lane.
__device__ __forceinline__ void count_ahead(const float* src, int N, unsigned long long ki,
                                            KeyQ* kq, int& cnt, double& G) {
  const int lane = threadIdx.x & 63;
  cnt = 0;
  G = 0.0;
  for (int c0 = 0; c0 < N; c0 += kChunk) {
    const int n = min(kChunk, N - c0);
    if (c0 > 0) __syncthreads();  // the previous chunk is consumed
    // all of a thread's loads in flight before any is used (indices clamped
    // into the chunk; the extra values are never stored)
    constexpr int kLoads = kChunk / kRankThreads;
    float f[kLoads];
#pragma unroll
    for (int s = 0; s < kLoads; ++s)
      f[s] = src[c0 + min((int)threadIdx.x + s * kRankThreads, n - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kLoads; ++s) {
      const int j = threadIdx.x + s * kRankThreads;
      if (j < n) kq[j] = KeyQ{sched_key(f[s], c0 + j), q_of(f[s])};
    }
    __syncthreads();
    // eight records read before any is used, then the remainder one by one
    constexpr int kBatch = 8;
    int j = lane;
    for (; j + 64 * (kBatch - 1) < n; j += 64 * kBatch) {
      KeyQ v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = kq[j + 64 * u];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) tally(v[u], ki, cnt, G);
    }
    for (; j < n; j += 64) tally(kq[j], ki, cnt, G);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off);
    G += __shfl_xor(G, off);
  }
}

// Device-scope (relaxed) accesses for what crosses workgroups.
__device__ __forceinline__ void store_agent(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     (unsigned long long)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_agent(const double* p) {
  return __longlong_as_double((long long)__hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void store_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this wave's stores have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Best (largest v, then smallest b) over the workgroup; every thread returns
// it.  rv, rb hold one entry per wave.
__device__ __forceinline__ void block_best(double& v, int& b, double* rv, int* rb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double ov = __shfl_xor(v, off);
    const int ob = __shfl_xor(b, off);
    if (ov > v || (ov == v && ob < b)) {
      v = ov;
      b = ob;
    }
  }
  if (lane == 0) {
    rv[wave] = v;
    rb[wave] = b;
  }
  __syncthreads();
  v = rv[0];
  b = rb[0];
#pragma unroll
  for (int w = 1; w < kRankThreads / 64; ++w)
    if (rv[w] > v || (rv[w] == v && rb[w] < b)) {
      v = rv[w];
      b = rb[w];
    }
}

// Raises the finishing counters for this workgroup (thread 0 only); true for
// the last workgroup of the launch.  Workgroup w counts on group w % kGroups,
// the last of a group on the top counter; each completed counter is reset to
// zero for the next call.  Same-address atomics serialise, hence two levels.
__device__ __forceinline__ bool count_finished(unsigned* done) {
  const unsigned total = gridDim.x * gridDim.y;
  const unsigned w = blockIdx.y * gridDim.x + blockIdx.x;
  const unsigned grp = w % kGroups;
  const unsigned ngroups = min(total, (unsigned)kGroups);
  const unsigned in_grp = (total - grp + kGroups - 1) / kGroups;
  unsigned* gc = done + (1 + grp) * kCounterStride;
  if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != in_grp - 1)
    return false;
  __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
      ngroups - 1)
    return false;
  __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The last workgroup: positions b = t + 256 s (s < kSlots) cover 0..N.
// Theta_fix(b) goes to LDS (th, kSlots * 256 doubles) so that a position
// meets its successor; ell is counted in LDS from the requests by position.
template <int kSlots>
__device__ __forceinline__ void finish_schedule(const SchedRankArgs& a, double* th, double* rv,
                                                int* rb, int* ell_s) {
  const int t = threadIdx.x;
  const int N = a.N, R = a.R;
  // R*2^32 + G_b is an integer below 2^53, so the fp64 sum is exact and equals
  // the int64 one.  Every load is issued before any is used (indices clamped
  // to the last position; slots beyond N are never read back).
  const double tau0 = (double)((long long)R << 32);
  double gb[kSlots], sb[kSlots];
  int rq[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int b = min(t + s * kRankThreads, N);
    gb[s] = load_agent(a.gpos + b);
    sb[s] = a.sps[R + b];
    rq[s] = load_agent(a.req + min(b, N - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int r = t; r < R; r += kRankThreads) ell_s[r] = 0;
  double thv[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    thv[s] = (tau0 + gb[s]) * sb[s];
    th[t + s * kRankThreads] = thv[s];
  }
  __syncthreads();
  double v;
  int bb;
  if (!a.async) {
    // the first position whose admission does not raise Theta (N if none)
    v = 0.0;
    bb = N;
#pragma unroll
    for (int s = kSlots - 1; s >= 0; --s) {
      const int b = t + s * kRankThreads;
      if (b < N && !(th[b + 1] > thv[s])) bb = b;
    }
  } else {
    // the largest Theta over b = 0..N, the smallest b on a tie
    v = -1.0;
    bb = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const int b = t + s * kRankThreads;
      if (b <= N && (thv[s] > v || (thv[s] == v && b < bb))) {
        v = thv[s];
        bb = b;
      }
    }
  }
  block_best(v, bb, rv, rb);
  if (bb > N) bb = 0;  // no position won (a NaN rate table): admit nothing
#pragma unroll
  for (int s = 0; s < kSlots; ++s)
    if (t + s * kRankThreads < bb && (unsigned)rq[s] < (unsigned)R) atomicAdd(&ell_s[rq[s]], 1);
  __syncthreads();
  for (int r = t; r < R; r += kRankThreads) a.ell[r] = ell_s[r];
  if (t == 0) {
    *a.budget = bb;
    if (a.theta != nullptr) *a.theta = th[bb] * 0x1p-32;
  }
}

// blockIdx.y = 0: a (sync) or a_lag (async), writing G by position (and, for
// the sync scheduler, the requests by position); blockIdx.y = 1 (async): a_cur,
// writing the requests by position.
template <int kSlots>
__global__ __launch_bounds__(kRankThreads) void sched_rank_kernel(SchedRankArgs a) {
  // the key stage of the count, then Theta by position in the last workgroup
  constexpr int kLdsBytes = kChunk * (int)sizeof(KeyQ) > kSlots * kRankThreads * 8
                                ? kChunk * (int)sizeof(KeyQ)
                                : kSlots * kRankThreads * 8;
  __shared__ __align__(16) unsigned char lds[kLdsBytes];
  __shared__ double rv[kRankThreads / 64];
  __shared__ int rb[kRankThreads / 64];
  __shared__ int ell_s[512];
  __shared__ int last_s;
  const bool cur = blockIdx.y == 1;
  const float* src = cur ? a.a_cur : a.a;
  const int N = a.N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x * kPerWg + wave;
  const bool valid = item < N;
  const int ic = valid ? item : N - 1;
  const float fi = src[ic];
  int rank;
  double G;
  count_ahead(src, N, sched_key(fi, ic), reinterpret_cast<KeyQ*>(lds), rank, G);
  if (valid && lane == 0) {
    if (cur || !a.async) store_agent(a.req + rank, item / a.gamma);
    if (!cur) {
      store_agent(a.gpos + rank, G);
      if (rank == N - 1) store_agent(a.gpos + N, G + q_of(fi));
    }
  }
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) last_s = count_finished(a.done);
  __syncthreads();
  if (!last_s) return;
  finish_schedule<kSlots>(a, reinterpret_cast<double*>(lds), rv, rb, ell_s);
}

template <int kSlots>
hipError_t launch_slots(const SchedRankArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(sched_rank_kernel<kSlots>, dim3(a.n_wgs, a.async ? 2 : 1),
                     dim3(kRankThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Workspace: the finishing counters (top, then kGroups groups, one 128-byte
// line each) | req[N] (int32) | gpos[N + 1] (fp64).
size_t sched_ws_bytes(int N) {
  return kCounterBytes + (((size_t)4 * N + 255) & ~(size_t)255) + (size_t)8 * (N + 1);
}

void sched_ws_layout(SchedRankArgs& a, void* ws) {
  unsigned char* p = reinterpret_cast<unsigned char*>(ws);
  a.n_wgs = (a.N + kPerWg - 1) / kPerWg;
  a.done = reinterpret_cast<unsigned*>(p);
  a.req = reinterpret_cast<int32_t*>(p + kCounterBytes);
  a.gpos = reinterpret_cast<double*>(p + kCounterBytes + (((size_t)4 * a.N + 255) & ~(size_t)255));
}

// The smallest instantiated slot count with positions 0..N in slots * 256.
hipError_t launch_schedule_ranked(const SchedRankArgs& a, hipStream_t stream) {
  const int need = a.N + 1;
  if (need <= 2 * kRankThreads) return launch_slots<2>(a, stream);
  if (need <= 4 * kRankThreads) return launch_slots<4>(a, stream);
  if (need <= 9 * kRankThreads) return launch_slots<9>(a, stream);
  if (need <= 17 * kRankThreads) return launch_slots<17>(a, stream);
  return launch_slots<(kMaxN + 1 + kRankThreads - 1) / kRankThreads>(a, stream);
}

}  // namespace dspark

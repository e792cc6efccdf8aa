// Hardware-aware prefix scheduler [P1 "DSpark" §4.1 (eqs. B, tau, Theta; the
// global sort), §4.2 (early stop); P3 スケジューラ; P2 "按负载决定验证多少"].
//
// One workgroup of 1024 threads:
//   1. keys (~bits(a) << 32 | flat index) for the N = R*gamma candidates,
//      padded to a power of two with all-ones keys, sorted ascending by a
//      bitonic network: a descending, ties by flat index ascending.  Each
//      thread keeps kPer consecutive keys in registers: compare-exchanges
//      inside a thread need nothing, those between threads of one wave go
//      through cross-lane shuffles, and only partners in different waves
//      (stride >= 64 * kPer) go through LDS with workgroup barriers.
//   2. q_i = rint(a_i * 2^32) as int64 (exact scaling, round half to even);
//      thread t owns a contiguous run of sorted positions, sums its q's, and a
//      fixed-order scan over the 1024 run totals gives every prefix G_b exactly
//      (integer sums do not depend on the order).
//   3. Theta_fix(b) = (double)(R*2^32 + G_b) * sps[R + b]; the budget b* is
//      the first b with Theta_fix(b+1) <= Theta_fix(b) (or N).
//   4. ell[r] = number of the first b* sorted candidates that belong to r --
//      always a prefix of r's block because rows of a are non-increasing.
#include "dspark_kernels.h"
#include "dspark_device.h"

namespace dspark {

namespace {

constexpr int kMaxN = 8192;
constexpr int kThreads = 1024;

__device__ __forceinline__ unsigned long long shfl_xor64(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// Bitonic network over n2 = kPer * kThreads * (1 or less) keys; thread t owns
// positions t * kPer .. t * kPer + kPer - 1 in `k` (n2 / kThreads of them are
// real when n2 < kPer * kThreads: the rest hold all-ones keys and stay last).
template <int kPer>
__device__ __forceinline__ void bitonic_sort(unsigned long long (&k)[kPer], unsigned long long* lds, int n2) {
  const int t = threadIdx.x;
  const int lane_bits = 6;  // 64 lanes
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < kPer) {  // partners inside the thread (constant register indices)
#pragma unroll
        for (int cs = kPer / 2; cs > 0; cs >>= 1) {
          if (cs != stride) continue;
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            if ((j & cs) != 0) continue;  // i & cs == j & cs since t * kPer is a multiple of kPer
            const int i = t * kPer + j;
            const bool asc = (i & size) == 0;
            const unsigned long long x = k[j], y = k[j + cs];
            const bool sw = (x > y) == asc;
            k[j] = sw ? y : x;
            k[j + cs] = sw ? x : y;
          }
        }
      } else if (stride < (kPer << lane_bits)) {  // partners in the same wave
        const int m = stride / kPer;  // lane distance
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int i = t * kPer + j;
          const unsigned long long o = shfl_xor64(k[j], m);
          const bool lower = (i & stride) == 0;
          const bool asc = (i & size) == 0;
          // the lower position keeps the smaller key when ascending
          const bool keep_min = lower == asc;
          k[j] = keep_min ? (o < k[j] ? o : k[j]) : (o > k[j] ? o : k[j]);
        }
      } else {  // partners in other waves: through LDS
#pragma unroll
        for (int j = 0; j < kPer; ++j) lds[t * kPer + j] = k[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int i = t * kPer + j;
          const unsigned long long o = lds[i ^ stride];
          const bool lower = (i & stride) == 0;
          const bool asc = (i & size) == 0;
          const bool keep_min = lower == asc;
          k[j] = keep_min ? (o < k[j] ? o : k[j]) : (o > k[j] ? o : k[j]);
        }
        __syncthreads();
      }
    }
  }
}

// The network on the first P of the kPer register keys.
template <int P, int kPer>
__device__ __forceinline__ void sort_prefix(unsigned long long (&k)[kPer], unsigned long long* lds,
                                            int n2) {
  unsigned long long kk[P];
#pragma unroll
  for (int j = 0; j < P; ++j) kk[j] = k[j];
  bitonic_sort<P>(kk, lds, n2);
#pragma unroll
  for (int j = 0; j < P; ++j) k[j] = kk[j];
}

// Sort the N = R * gamma candidates of `a` into `key` (ascending; see the
// file comment) and return the per-thread run [b0, b1) of sorted positions with
// the fixed-point prefix sum G at b0 (`base`) and the total over all N.
// Called by all kThreads threads; ends with the keys visible in LDS.
struct Runs {
  int b0, b1;
  long long base, total;
};

__device__ __forceinline__ long long q_of(unsigned long long key) {
  const float v = __uint_as_float(~(uint32_t)(key >> 32));
  return (long long)rint((double)v * 4294967296.0);
}

__device__ __forceinline__ Runs sort_and_scan(const float* a, int N, unsigned long long* key, long long* wsum) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int n2 = kThreads;  // at least one key per thread so every thread runs the network
  while (n2 < N) n2 <<= 1;
  constexpr int kPer = kMaxN / kThreads;
  const int per2 = n2 / kThreads;  // keys per thread actually in the network
  unsigned long long k[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = t * per2 + j;
    unsigned long long v = ~0ull;
    if (j < per2 && i < N) {
      const float f = a[i];
      const uint32_t bits = (f > 0.0f) ? __float_as_uint(f) : 0u;  // NaN / <= 0 sort as 0
      v = ((unsigned long long)(~bits) << 32) | (uint32_t)i;
    }
    k[j] = v;
  }
  switch (per2) {  // the network over n2 keys, per2 in registers per thread
    case 1: sort_prefix<1>(k, key, n2); break;
    case 2: sort_prefix<2>(k, key, n2); break;
    case 4: sort_prefix<4>(k, key, n2); break;
    default: bitonic_sort<kPer>(k, key, n2); break;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (j < per2) key[t * per2 + j] = k[j];
  __syncthreads();

  Runs u;
  const int per = (N + kThreads - 1) / kThreads;
  u.b0 = min(N, t * per);
  u.b1 = min(N, u.b0 + per);
  long long own = 0;
  for (int i = u.b0; i < u.b1; ++i) own += q_of(key[i]);
  // inclusive scan of the per-thread sums: within the wave, then over waves
  long long incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)incl, off), hi = __shfl_up((uint32_t)((unsigned long long)incl >> 32), off);
    const long long v = (long long)(((unsigned long long)hi << 32) | lo);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  long long before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  u.total = 0;
  for (int w = 0; w < kThreads / 64; ++w) u.total += wsum[w];
  u.base = before + incl - own;  // G at position b0
  __syncthreads();               // wsum and key may be reused after this
  return u;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(SchedArgs a) {
  __shared__ unsigned long long key[kMaxN];
  __shared__ long long wsum[kThreads / 64];
  __shared__ int ell_s[512];
  __shared__ int stop_s;
  __shared__ double theta_s;
  const int t = threadIdx.x;
  const int N = a.R * a.gamma;
  for (int i = t; i < a.R; i += kThreads) ell_s[i] = 0;
  if (t == 0) stop_s = N;
  const Runs u = sort_and_scan(a.a, N, key, wsum);
  const long long tau0 = (long long)a.R << 32;

  long long G = u.base;
  for (int i = u.b0; i < u.b1; ++i) {
    const long long Gn = G + q_of(key[i]);
    const double th = (double)(tau0 + G) * a.sps[a.R + i];
    const double thn = (double)(tau0 + Gn) * a.sps[a.R + i + 1];
    if (!(thn > th)) {
      atomicMin(&stop_s, i);
      break;
    }
    G = Gn;
  }
  __syncthreads();
  const int bstar = stop_s;

  G = u.base;
  for (int i = u.b0; i < u.b1; ++i) {
    if (i == bstar) theta_s = (double)(tau0 + G) * a.sps[a.R + i];
    if (i < bstar) {
      atomicAdd(&ell_s[(int)(key[i] & 0xFFFFFFFFu) / a.gamma], 1);
      G += q_of(key[i]);
    }
  }
  if (bstar == N && t == kThreads - 1) theta_s = (double)(tau0 + u.total) * a.sps[a.R + N];
  __syncthreads();
  for (int i = t; i < a.R; i += kThreads) a.ell[i] = ell_s[i];
  if (t == 0) {
    *a.budget = bstar;
    if (a.theta != nullptr) *a.theta = theta_s * 0x1p-32;
  }
}

// Asynchronous variant [P1 §4.3; P3 スケジューラの実運用適用]: the budget K is
// the b in 0..N with the largest Theta_fix(b) computed from the survival
// probabilities of two steps earlier (a_lag), over all b (no early stop; the
// smallest such b); then the K candidates with the largest current survival
// (a_cur, same key order) are admitted.
__global__ __launch_bounds__(kThreads) void schedule_async_kernel(SchedAsyncArgs a) {
  __shared__ unsigned long long key[kMaxN];
  __shared__ long long wsum[kThreads / 64];
  __shared__ int ell_s[512];
  __shared__ double red_v[kThreads / 64];
  __shared__ int red_b[kThreads / 64];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int N = a.R * a.gamma;
  for (int i = t; i < a.R; i += kThreads) ell_s[i] = 0;
  const long long tau0 = (long long)a.R << 32;

  // 1. K from the lagged survival: thread t scores b = i + 1 for i in its run
  //    (thread 0 also b = 0); the best (Theta, smallest b) wins.
  const Runs u = sort_and_scan(a.a_lag, N, key, wsum);
  double bv = -1.0;
  int bb = 0x7fffffff;
  if (t == 0) {
    bv = (double)tau0 * a.sps[a.R];
    bb = 0;
  }
  long long G = u.base;
  for (int i = u.b0; i < u.b1; ++i) {
    G += q_of(key[i]);
    const double th = (double)(tau0 + G) * a.sps[a.R + i + 1];
    if (th > bv) {  // positions rise within the run: strict '>' keeps the smallest b
      bv = th;
      bb = i + 1;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const double ov = __shfl_xor(bv, off);
    const int ob = __shfl_xor(bb, off);
    if (ov > bv || (ov == bv && ob < bb)) {
      bv = ov;
      bb = ob;
    }
  }
  if (lane == 0) {
    red_v[wave] = bv;
    red_b[wave] = bb;
  }
  __syncthreads();
  double kv = red_v[0];
  int K = red_b[0];
  for (int w = 1; w < kThreads / 64; ++w)
    if (red_v[w] > kv || (red_v[w] == kv && red_b[w] < K)) {
      kv = red_v[w];
      K = red_b[w];
    }
  __syncthreads();  // the key buffer is reused below

  // 2. top-K of the current survival
  const Runs c = sort_and_scan(a.a_cur, N, key, wsum);
  for (int i = c.b0; i < c.b1; ++i)
    if (i < K) atomicAdd(&ell_s[(int)(key[i] & 0xFFFFFFFFu) / a.gamma], 1);
  __syncthreads();
  for (int i = t; i < a.R; i += kThreads) a.ell[i] = ell_s[i];
  if (t == 0) {
    *a.budget = K;
    if (a.theta != nullptr) *a.theta = kv * 0x1p-32;
  }
}

}  // namespace

hipError_t launch_schedule(const SchedArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_schedule_async(const SchedAsyncArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_async_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dspark

// Hardware-aware prefix scheduler [P1 "DSpark" §4.1 (eqs. B, tau, Theta; the
// global sort), §4.2 (early stop); P3 スケジューラ; P2 "按负载决定验证多少"].
//
// One workgroup of 1024 threads:
//   1. keys (~bits(a) << 32 | flat index) for the N = R*gamma candidates,
//      sorted ascending by their high half (a descending) with a stable LDS
//      radix sort (four passes of 8-bit digits, ranks from wave ballots and a
//      workgroup scan of per-wave digit counts), so equal a keep flat index
//      order.
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

constexpr int kWavesS = kThreads / 64;
constexpr int kDigits = 256;
constexpr int kSlots = kMaxN / kThreads;  // items per lane at the largest N

// Exclusive prefix sum of one value per thread over the whole workgroup, in
// thread order; `tot` receives the sum over all threads.  Uses wsum[0..15].
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& tot) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < kWavesS; ++w) {
    const int x = wsum[w];
    before += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();  // wsum may be reused after this
  return before + incl - v;
}

// Stable LSD radix sort of the N 64-bit keys in `src` by their high 32 bits,
// four passes of 8-bit digits (ties keep their order, so keys that carry the
// flat index in the low bits end up ordered by it).  Wave w owns items
// w*C .. w*C + C - 1 (C = 64 * slots), lane l of slot j item w*C + 64 j + l,
// so inside a wave the items run slot-major.  Per slot, the lanes holding one
// digit find each other with eight ballots; their rank is the count of that
// digit already seen by the wave (an LDS counter per wave and digit, advanced
// by the lowest such lane) plus the matching lanes below.  A workgroup scan
// over the counters in digit-major, wave-minor order then gives every
// (wave, digit) its first output position.  The result ends in `src`.
__device__ __forceinline__ void radix_sort(unsigned long long* src, unsigned long long* dst,
                                           int* wcount, int* wsum, int N) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int slots = (N + kThreads - 1) / kThreads;
  const int C = 64 * slots;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 32 + 8 * pass;
    for (int i = t; i < kWavesS * kDigits; i += kThreads) wcount[i] = 0;
    __syncthreads();
    int* wc = wcount + wave * kDigits;
    unsigned long long v[kSlots];
    int rank[kSlots], dig[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      rank[j] = 0;
      dig[j] = 0;
      v[j] = 0ull;
      if (j < slots) {
        const int idx = wave * C + 64 * j + lane;
        const bool valid = idx < N;
        v[j] = valid ? src[idx] : 0ull;
        const int d = (int)((v[j] >> shift) & 0xFFu);
        // lanes of this slot holding digit d: agree with d on all 8 bits
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
          const unsigned long long b = (d >> bit) & 1;
          peers &= __ballot(b != 0) ^ (b - 1ull);  // the ballot itself, or its complement
        }
        dig[j] = d;
        if (valid) {
          const int seen = wc[d];
          const unsigned long long below = peers & lt;
          rank[j] = seen + __popcll(below);
          if (below == 0ull) wc[d] = seen + __popcll(peers);
        }
      }
    }
    __syncthreads();
    // first output position of every (wave, digit): thread t takes digit t/4
    // and waves 4(t%4) .. 4(t%4)+3
    {
      const int d = t >> 2, w0 = (t & 3) * 4;
      int c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = wcount[(w0 + i) * kDigits + d];
        sum += c[i];
      }
      int tot;
      int base = block_excl_scan(sum, wsum, tot);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wcount[(w0 + i) * kDigits + d] = base;
        base += c[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      if (j < slots) {
        const int idx = wave * C + 64 * j + lane;
        if (idx < N) {
          const int pos = wc[dig[j]] + rank[j];
          if (pos < N) dst[pos] = v[j];
        }
      }
    }
    __syncthreads();
    unsigned long long* tmp = src;
    src = dst;
    dst = tmp;
  }
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

// Length of thread t's run of sorted positions, [t * per, t * per + per)
// clipped to N (per = ceil(N / kThreads) <= kSlots).
__device__ __forceinline__ int run_length(int N) {
  const int per = (N + kThreads - 1) / kThreads;
  const int b0 = min(N, (int)threadIdx.x * per);
  return min(N, b0 + per) - b0;
}

__device__ __forceinline__ Runs sort_and_scan(const float* a, int N, unsigned long long* key,
                                              unsigned long long* tmp, int* wcount, int* wsum,
                                              long long* lsum) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  for (int i = t; i < N; i += kThreads) {
    const float f = a[i];
    const uint32_t bits = (f > 0.0f) ? __float_as_uint(f) : 0u;  // NaN / <= 0 sort as 0
    key[i] = ((unsigned long long)(~bits) << 32) | (uint32_t)i;
  }
  __syncthreads();
  radix_sort(key, tmp, wcount, wsum, N);

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
  if (lane == 63) lsum[wave] = incl;
  __syncthreads();
  long long before = 0;
  for (int w = 0; w < wave; ++w) before += lsum[w];
  u.total = 0;
  for (int w = 0; w < kThreads / 64; ++w) u.total += lsum[w];
  u.base = before + incl - own;  // G at position b0
  __syncthreads();               // lsum and key may be reused after this
  return u;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(SchedArgs a) {
  __shared__ unsigned long long key[kMaxN];
  __shared__ unsigned long long tmp[kMaxN];
  __shared__ int wcount[kWavesS * kDigits];
  __shared__ int wsum[kWavesS];
  __shared__ long long lsum[kWavesS];
  __shared__ int ell_s[512];
  __shared__ int stop_s;
  __shared__ double theta_s;
  const int t = threadIdx.x;
  const int N = a.R * a.gamma;
  for (int i = t; i < a.R; i += kThreads) ell_s[i] = 0;
  if (t == 0) stop_s = N;
  // this thread's SPS entries R + b0 .. R + b1 (b1 - b0 <= kSlots), loaded
  // before the sort so that their latency hides behind it
  double sp[kSlots + 1];
  const int nb = run_length(N);
  {
    const double* sps = a.sps + a.R + min(N, t * ((N + kThreads - 1) / kThreads));
#pragma unroll
    for (int j = 0; j <= kSlots; ++j) sp[j] = j <= nb ? sps[j] : 0.0;
  }
  const Runs u = sort_and_scan(a.a, N, key, tmp, wcount, wsum, lsum);
  const long long tau0 = (long long)a.R << 32;

  long long G = u.base;
  bool stopped = false;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    if (j < nb && !stopped) {
      const int i = u.b0 + j;
      const long long Gn = G + q_of(key[i]);
      const double th = (double)(tau0 + G) * sp[j];
      const double thn = (double)(tau0 + Gn) * sp[j + 1];
      if (!(thn > th)) {
        atomicMin(&stop_s, i);
        stopped = true;
      }
      G = Gn;
    }
  }
  __syncthreads();
  const int bstar = stop_s;

  G = u.base;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    if (j < nb) {
      const int i = u.b0 + j;
      if (i == bstar) theta_s = (double)(tau0 + G) * sp[j];
      if (i < bstar) {
        atomicAdd(&ell_s[(int)(key[i] & 0xFFFFFFFFu) / a.gamma], 1);
        G += q_of(key[i]);
      }
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
  __shared__ unsigned long long tmp[kMaxN];
  __shared__ int wcount[kWavesS * kDigits];
  __shared__ int wsum[kWavesS];
  __shared__ long long lsum[kWavesS];
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
  double sp[kSlots + 1];
  const int nb = run_length(N);
  {
    const double* sps = a.sps + a.R + min(N, t * ((N + kThreads - 1) / kThreads));
#pragma unroll
    for (int j = 0; j <= kSlots; ++j) sp[j] = j <= nb ? sps[j] : 0.0;
  }
  const Runs u = sort_and_scan(a.a_lag, N, key, tmp, wcount, wsum, lsum);
  double bv = -1.0;
  int bb = 0x7fffffff;
  if (t == 0) {
    bv = (double)tau0 * a.sps[a.R];
    bb = 0;
  }
  long long G = u.base;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    if (j < nb) {
      const int i = u.b0 + j;
      G += q_of(key[i]);
      const double th = (double)(tau0 + G) * sp[j + 1];
      if (th > bv) {  // positions rise within the run: strict '>' keeps the smallest b
        bv = th;
        bb = i + 1;
      }
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
  const Runs c = sort_and_scan(a.a_cur, N, key, tmp, wcount, wsum, lsum);
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

// Hardware-aware prefix scheduler [P1 "DSpark" §4.1 (eqs. B, tau, Theta; the
// global sort), §4.2 (early stop); P3 スケジューラ; P2 "按负载决定验证多少"].
//
// One workgroup of 1024 threads:
//   1. keys (~bits(a) << 32 | flat index) for the N = R*gamma candidates,
//      padded to a power of two with all-ones keys, sorted ascending in LDS by
//      a bitonic network: a descending, ties by flat index ascending.
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

__global__ __launch_bounds__(kThreads) void schedule_kernel(SchedArgs a) {
  __shared__ unsigned long long key[kMaxN];
  __shared__ long long tsum[kThreads];
  __shared__ int ell_s[512];
  __shared__ int stop_s;
  __shared__ double theta_s;
  const int t = threadIdx.x;
  const int N = a.R * a.gamma;
  int n2 = 1;
  while (n2 < N) n2 <<= 1;

  for (int i = t; i < n2; i += kThreads) {
    unsigned long long k = ~0ull;
    if (i < N) {
      const float v = a.a[i];
      const uint32_t bits = (v > 0.0f) ? __float_as_uint(v) : 0u;  // NaN / <= 0 sort as 0
      k = ((unsigned long long)(~bits) << 32) | (uint32_t)i;
    }
    key[i] = k;
  }
  for (int i = t; i < a.R; i += kThreads) ell_s[i] = 0;
  if (t == 0) stop_s = N;
  __syncthreads();

  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < (n2 >> 1); i += kThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const unsigned long long x = key[lo], y = key[hi];
        if ((x > y) == asc) {
          key[lo] = y;
          key[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  const int per = (N + kThreads - 1) / kThreads;
  const int b0 = t * per;
  const int b1 = min(N, b0 + per);
  auto q_at = [&](int i) -> long long {
    const float v = __uint_as_float(~(uint32_t)(key[i] >> 32));
    return (long long)rint((double)v * 4294967296.0);
  };
  long long own = 0;
  for (int i = b0; i < b1; ++i) own += q_at(i);
  tsum[t] = own;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const long long add = (t >= off) ? tsum[t - off] : 0;
    __syncthreads();
    tsum[t] += add;
    __syncthreads();
  }
  const long long base = tsum[t] - own;  // G at position b0
  const long long tau0 = (long long)a.R << 32;

  long long G = base;
  for (int i = b0; i < b1; ++i) {
    const long long Gn = G + q_at(i);
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

  G = base;
  for (int i = b0; i < b1; ++i) {
    if (i == bstar) theta_s = (double)(tau0 + G) * a.sps[a.R + i];
    if (i < bstar) {
      atomicAdd(&ell_s[(int)(key[i] & 0xFFFFFFFFu) / a.gamma], 1);
      G += q_at(i);
    }
  }
  if (bstar == N && t == kThreads - 1) theta_s = (double)(tau0 + tsum[kThreads - 1]) * a.sps[a.R + N];
  __syncthreads();
  for (int i = t; i < a.R; i += kThreads) a.ell[i] = ell_s[i];
  if (t == 0) {
    *a.budget = bstar;
    if (a.theta != nullptr) *a.theta = theta_s * 0x1p-32;
  }
}

}  // namespace

hipError_t launch_schedule(const SchedArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dspark

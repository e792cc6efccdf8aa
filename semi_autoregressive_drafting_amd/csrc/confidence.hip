// Batched confidence head and survival product for a drafted block
// [P1 "DSpark" §3.1 eq. c_k; §1.1 eq. a_j; §4.1 eq. tau]:
//   c[r][k-1] = sigma(w[0:d] . h[r][k-1] + w[d:] . W1[x[r][k-1]])
//   a[r][k-1] = a[r][k-2] * c[r][k-1]   (fp32, left to right, a[r][-1] = 1)
// One workgroup (4 waves) per request, positions in order; each dot product
// uses the same workgroup-level function as the draft step (conf_dot_wg), so
// both paths give bit-identical c and a.
#include "dspark_kernels.h"
#include "dspark_device.h"

namespace dspark {

namespace {

template <class W>
__global__ __launch_bounds__(256) void confidence_kernel(ConfArgs a) {
  using store_t = typename W::store_t;
  __shared__ float red[4];
  const int r = blockIdx.x;
  float run = 1.0f;
  for (int k = 1; k <= a.gamma; ++k) {
    const size_t o = (size_t)r * a.gamma + (k - 1);
    const int xp = checked_token(a.x[(size_t)r * (a.gamma + 1) + (k - 1)], a.V, a.err);
    const store_t* hrow = reinterpret_cast<const store_t*>(a.h) + o * a.d;
    const store_t* erow = reinterpret_cast<const store_t*>(a.W1) + (size_t)xp * a.rank;
    const float c = sigmoid_f32(conf_dot_wg<W>(hrow, erow, a.w, a.d, a.rank, red));
    run = __fmul_rn(run, c);
    if (threadIdx.x == 0) {
      a.c[o] = c;
      a.a[o] = run;
    }
  }
}

}  // namespace

hipError_t launch_confidence(const ConfArgs& a, hipStream_t stream) {
  const dim3 grid(a.R);
  if (a.bf16)
    hipLaunchKernelGGL((confidence_kernel<WBf16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((confidence_kernel<WF32>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dspark

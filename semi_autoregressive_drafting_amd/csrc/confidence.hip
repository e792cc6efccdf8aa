// Batched confidence head and survival product for a drafted block
// [P1 "DSpark" §3.1 eq. c_k; §1.1 eq. a_j; §4.1 eq. tau]:
//   c[r][k-1] = sigma(w[0:d] . h[r][k-1] + w[d:] . W1[x[r][k-1]])
//   a[r][k-1] = a[r][k-2] * c[r][k-1]   (fp32, left to right, a[r][-1] = 1)
// One workgroup per request; positions run in order inside the workgroup, each
// dot product with the same thread-strided partials and fixed tree as the
// fused draft-step combine, so both paths give bit-identical c and a.
#include "dspark_kernels.h"
#include "dspark_device.h"

namespace dspark {

namespace {

template <class W>
__global__ __launch_bounds__(256) void confidence_kernel(ConfArgs a) {
  using store_t = typename W::store_t;
  __shared__ float sbuf[256];
  const int r = blockIdx.x, t = threadIdx.x;
  float run = 1.0f;
  for (int k = 1; k <= a.gamma; ++k) {
    const size_t o = (size_t)r * a.gamma + (k - 1);
    int xp = a.x[(size_t)r * (a.gamma + 1) + (k - 1)];
    xp = xp < 0 ? 0 : (xp >= a.V ? a.V - 1 : xp);  // device ids are not validated
    const store_t* hrow = reinterpret_cast<const store_t*>(a.h) + o * a.d;
    const store_t* erow = reinterpret_cast<const store_t*>(a.W1) + (size_t)xp * a.rank;
    const float dot = block_sum256(conf_partial<W>(hrow, erow, a.w, a.d, a.rank, t), sbuf);
    if (t == 0) {
      const float c = sigmoid_f32(dot);
      run = __fmul_rn(run, c);
      a.c[o] = c;
      a.a[o] = run;
    }
  }
}

}  // namespace

hipError_t launch_confidence(const ConfArgs& a, hipStream_t stream) {
  if (a.bf16)
    hipLaunchKernelGGL((confidence_kernel<WBf16>), dim3(a.R), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((confidence_kernel<WF32>), dim3(a.R), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dspark

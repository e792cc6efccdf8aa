// Training gradients behind the logits [P1 "DSpark" §2.3 (Markov head
// B = W1[x_{k-1}] W2), §3.1 (confidence head), §5 (losses)].
//
// With dz = dL/dz [n_rows][V] from the logit pass (dL/dU is dz itself) and
// dl = dL/dl [n_rows] for the confidence logit l = w.[h; e], e = W1[x*_{k-1}]:
//
//   dE   = dz . W2t + dl w[d:]           [n_rows][rank]  (gradient of the gathered rows)
//   dW1  = scatter-add of the dE rows to their tokens x*_{k-1}
//   dW2t = dz^T . E                      [V][rank]
//   dh   = dl w[:d]                      [n_rows][d]
//   dw   = sum_rows dl [h; e]            [d + rank]
//
// The two contractions run on MFMA (v_mfma_f32_32x32x16_bf16): dz is rounded
// to bf16 as an operand (the weights are bf16 already), products accumulate
// in fp32.  Both MFMA operands must hold 8 consecutive K values per lane, and
// K is the vocabulary for dE and the row for dW2t, so the kernels first make
// a vocabulary-major copy of W2t and a row-major copy of E^T in the
// workspace.  Every sum runs in a fixed order: results are bit-reproducible.
//
//   G2 transpose_w2     W2t [V][rank] -> w2 [rank][vp] (zero past V)
//   G3 gather_et        E^T [rank][n_pad] from W1 and x* (zero past n_rows)
//   G4 grad_e_partial   per (128-row group, vocabulary slab) partial dz . W2t
//   G5 grad_e_reduce    slab partials in slab order + dl w[d:]  -> dE
//   G6 grad_w2t         per 32-entry vocabulary tile, dz^T . E over all rows
//   G7 zero_rows / scatter_dw1   dW1 = 0, then per token the sum of its dE
//      rows in row order (written by the token's first row)
//   G8 grad_conf        dh, and dw by one thread per column over the rows in
//      order (fp64)
#include "dspark_kernels.h"
#include "dspark_device.h"

namespace dspark {

namespace {

constexpr int kGThreads = 256;  // 4 waves
constexpr int kChunk = 64;      // vocabulary entries per K chunk of G4 (4 MFMA K steps)

struct GradArgs {
  int V, rank, d, gamma, n_rows, n_pad, vp, e_slabs, e_groups;
  const uint16_t* W1;
  const uint16_t* W2t;
  const uint16_t* h;
  const float* w;
  const int32_t* x;  // x* [R][gamma + 1]
  const float* dz;   // [n_rows][V]
  const float* dl;   // [n_rows]
  uint16_t* w2;      // [rank][vp]
  uint16_t* et;      // [rank][n_pad]
  float* dep;        // [e_slabs][n_pad][rank]
  float* de;         // [n_rows][rank]
  float* dW1;
  float* dW2t;
  float* dh;
  float* dw;
};

__device__ __forceinline__ int row_token(const GradArgs& g, int row) {
  const int r = row / g.gamma, k = row % g.gamma;  // position k+1 reads x*_k
  return clamp_token(g.x[(size_t)r * (g.gamma + 1) + k], g.V);
}

// bf16 of an fp32 value, round to nearest even (values here are finite).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ bf16x8_t pack_bf16(const float (&v)[8]) {
  bf16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = __builtin_bit_cast(__bf16, bf16_rne(v[j]));
  return r;
}

// ---------------------------------------------------------------------------
// G2 / G3: 64 x 64 tiles through LDS.  src(row, col) is read along col and
// written transposed along row: dst[col][row], dst row stride ld.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGThreads) void transpose_w2(GradArgs g) {
  __shared__ uint16_t tile[64][66];
  const int v0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += kGThreads) {
    const int vv = i >> 6, nn = i & 63;
    const int v = v0 + vv, n = n0 + nn;
    tile[vv][nn] = (v < g.V && n < g.rank) ? g.W2t[(size_t)v * g.rank + n] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += kGThreads) {
    const int nn = i >> 6, vv = i & 63;
    const int v = v0 + vv, n = n0 + nn;
    if (n < g.rank && v < g.vp) g.w2[(size_t)n * g.vp + v] = tile[vv][nn];
  }
}

__global__ __launch_bounds__(kGThreads) void gather_et(GradArgs g) {
  __shared__ uint16_t tile[64][66];
  const int r0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += kGThreads) {
    const int rr = i >> 6, nn = i & 63;
    const int row = r0 + rr, n = n0 + nn;
    uint16_t v = 0;
    if (row < g.n_rows && n < g.rank) v = g.W1[(size_t)row_token(g, row) * g.rank + n];
    tile[rr][nn] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += kGThreads) {
    const int nn = i >> 6, rr = i & 63;
    const int row = r0 + rr, n = n0 + nn;
    if (n < g.rank && row < g.n_pad) g.et[(size_t)n * g.n_pad + row] = tile[rr][nn];
  }
}

// ---------------------------------------------------------------------------
// G4: wave q of workgroup (group, slab) owns rows 32 (4 group + q) .. +31 and
// all NC 32-wide rank chunks; it walks the slab's vocabulary in chunks of 64
// (4 K steps of 16).  MFMA operands for K step s (vocabulary v0 = 16 s):
//   A (rows x K):  lane (m = l%32, half h) holds dz[row m][v0 + 8h .. +7]
//   B (K x rank):  lane (n = l%32, half h) holds w2[c*32 + n][v0 + 8h .. +7]
// The dz rows of the next chunk are loaded while the current chunk multiplies.
// ---------------------------------------------------------------------------
template <int NC, bool kVec>
__global__ __launch_bounds__(kGThreads) void grad_e_partial(GradArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int grp = blockIdx.x % g.e_groups, slab = blockIdx.x / g.e_groups;
  const int rt = grp * 4 + wave;
  const int row = rt * 32 + col;
  const int rowc = row < g.n_rows ? row : g.n_rows - 1;
  const float* zrow = g.dz + (size_t)rowc * g.V;
  int c_begin, c_end;
  slab_range(slab, g.e_slabs, g.vp / kChunk, c_begin, c_end);

  f32x16_t acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x16_t{};

  // this lane's dz entries of chunk ch: v = 64 ch + 16 s + 8 half + j
  auto load_chunk = [&](float (&a)[4][8], int ch) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int vb = ch * kChunk + 16 * s + 8 * half;
      if (kVec && vb + 8 <= g.V) {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(zrow + vb);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(zrow + vb + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[s][j] = lo[j];
          a[s][4 + j] = hi[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) a[s][j] = vb + j < g.V ? zrow[vb + j] : 0.0f;
      }
    }
  };

  float cur[4][8], nxt[4][8];
  if (c_begin < c_end) load_chunk(cur, c_begin);
  for (int ch = c_begin; ch < c_end; ++ch) {
    if (ch + 1 < c_end) load_chunk(nxt, ch + 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int v0 = ch * kChunk + 16 * s + 8 * half;
      bf16x8_t b[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        b[c] = *reinterpret_cast<const bf16x8_t*>(g.w2 + (size_t)(c * 32 + col) * g.vp + v0);
      const bf16x8_t a = pack_bf16(cur[s]);
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[c], acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) cur[s][j] = nxt[s][j];
  }
  // accumulator i of lane l: row 8 (i/4) + 4 half + i%4 of the tile, rank c*32 + l%32
  float* out = g.dep + (size_t)slab * g.n_pad * g.rank;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = rt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      out[(size_t)rr * g.rank + c * 32 + col] = acc[c][i];
    }
}

// G5: dE = sum of the slab partials in slab order + dl w[d:].
__global__ __launch_bounds__(kGThreads) void grad_e_reduce(GradArgs g) {
  const size_t i = (size_t)blockIdx.x * kGThreads + threadIdx.x;
  if (i >= (size_t)g.n_rows * g.rank) return;
  const int row = (int)(i / g.rank), j = (int)(i % g.rank);
  float s = 0.0f;
  for (int sl = 0; sl < g.e_slabs; ++sl) s += g.dep[((size_t)sl * g.n_pad + row) * g.rank + j];
  g.de[i] = fmaf(g.dl[row], g.w[g.d + j], s);
}

// ---------------------------------------------------------------------------
// G6: wave (workgroup b, wave q) owns vocabulary tile vt = 4 b + q and all NC
// rank chunks; K runs over the rows in steps of 16:
//   A (vocab x K):  lane (m = l%32, half h) holds dz[r0 + 8h + j][32 vt + m]
//   B (K x rank):   lane (n = l%32, half h) holds et[c*32 + n][r0 + 8h .. +7]
// The dz loads of step r0 + 16 are issued before the MFMAs of step r0.
// ---------------------------------------------------------------------------
template <int NC>
__global__ __launch_bounds__(kGThreads) void grad_w2t(GradArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int vt = blockIdx.x * 4 + wave;
  if (vt * 32 >= g.V) return;  // no barriers below
  const int v = vt * 32 + col;
  const bool vin = v < g.V;
  const float* zcol = g.dz + (vin ? v : 0);

  f32x16_t acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x16_t{};
  auto load_step = [&](float (&a)[8], int r0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = r0 + 8 * half + j;
      a[j] = (vin && rr < g.n_rows) ? zcol[(size_t)rr * g.V] : 0.0f;
    }
  };
  float cur[8], nxt[8];
  load_step(cur, 0);
  for (int r0 = 0; r0 < g.n_pad; r0 += 16) {
    if (r0 + 16 < g.n_pad) load_step(nxt, r0 + 16);
    bf16x8_t b[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      b[c] = *reinterpret_cast<const bf16x8_t*>(g.et + (size_t)(c * 32 + col) * g.n_pad + r0 + 8 * half);
    const bf16x8_t a = pack_bf16(cur);
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[c], acc[c], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) cur[j] = nxt[j];
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int vv = vt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (vv < g.V) g.dW2t[(size_t)vv * g.rank + c * 32 + col] = acc[c][i];
    }
}

// G7: dW1 = 0, then scatter.
__global__ __launch_bounds__(kGThreads) void zero_floats(float* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * kGThreads + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// One workgroup per row; only the first row (in row order) of each token
// writes, the sum of that token's dE rows taken in row order.
__global__ __launch_bounds__(kGThreads) void scatter_dw1(GradArgs g) {
  const int row = blockIdx.x;
  const int tok = row_token(g, row);
  for (int r = 0; r < row; ++r)
    if (row_token(g, r) == tok) return;  // uniform across the workgroup
  for (int j = threadIdx.x; j < g.rank; j += kGThreads) {
    float s = 0.0f;
    for (int r = row; r < g.n_rows; ++r)
      if (row_token(g, r) == tok) s += g.de[(size_t)r * g.rank + j];
    g.dW1[(size_t)tok * g.rank + j] = s;
  }
}

// G8: dh = dl w[:d]; dw[j] = sum over rows (in order) of dl [h; e]_j.
__global__ __launch_bounds__(kGThreads) void grad_dh(GradArgs g) {
  const size_t i = (size_t)blockIdx.x * kGThreads + threadIdx.x;
  if (i >= (size_t)g.n_rows * g.d) return;
  const int row = (int)(i / g.d), j = (int)(i % g.d);
  g.dh[i] = g.dl[row] * g.w[j];
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

__global__ __launch_bounds__(kGThreads) void grad_dw(GradArgs g) {
  const int j = blockIdx.x * kGThreads + threadIdx.x;
  if (j >= g.d + g.rank) return;
  double s = 0.0;
  if (j < g.d) {
    for (int row = 0; row < g.n_rows; ++row)
      s += (double)g.dl[row] * (double)bf16_to_f32(g.h[(size_t)row * g.d + j]);
  } else {
    for (int row = 0; row < g.n_rows; ++row)
      s += (double)g.dl[row] * (double)bf16_to_f32(g.W1[(size_t)row_token(g, row) * g.rank + (j - g.d)]);
  }
  g.dw[j] = (float)s;
}

template <int NC>
hipError_t launch_gemms(const GradArgs& g, bool vec, hipStream_t stream) {
  if (vec)
    hipLaunchKernelGGL((grad_e_partial<NC, true>), dim3(g.e_groups * g.e_slabs), dim3(kGThreads), 0,
                       stream, g);
  else
    hipLaunchKernelGGL((grad_e_partial<NC, false>), dim3(g.e_groups * g.e_slabs), dim3(kGThreads), 0,
                       stream, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_vt = (g.V + 31) / 32;
  hipLaunchKernelGGL((grad_w2t<NC>), dim3((n_vt + 3) / 4), dim3(kGThreads), 0, stream, g);
  return hipGetLastError();
}

unsigned blocks_for(size_t n) { return (unsigned)((n + kGThreads - 1) / kGThreads); }

}  // namespace

hipError_t launch_train_grad_rest(const VerifyArgs& a, const TrainArgs& ta, const VerifyPlan& p,
                                  const TrainPlan& tp, hipStream_t stream) {
  GradArgs g{};
  g.V = a.V;
  g.rank = a.rank;
  g.d = ta.d;
  g.gamma = a.gamma;
  g.n_rows = p.n_rows;
  g.n_pad = tp.n_pad;
  g.vp = tp.vp;
  g.e_slabs = tp.e_slabs;
  g.e_groups = tp.e_groups;
  g.W1 = static_cast<const uint16_t*>(a.W1);
  g.W2t = static_cast<const uint16_t*>(a.W2t);
  g.h = static_cast<const uint16_t*>(ta.h);
  g.w = ta.w;
  g.x = a.x;
  g.dz = ta.dU;
  g.dl = reinterpret_cast<const float*>(a.ws + tp.off_dl);
  g.w2 = reinterpret_cast<uint16_t*>(a.ws + tp.off_w2);
  g.et = reinterpret_cast<uint16_t*>(a.ws + tp.off_et);
  g.dep = reinterpret_cast<float*>(a.ws + tp.off_dep);
  g.de = reinterpret_cast<float*>(a.ws + tp.off_de);
  g.dW1 = ta.dW1;
  g.dW2t = ta.dW2t;
  g.dh = ta.dh;
  g.dw = ta.dw;

  hipLaunchKernelGGL(transpose_w2, dim3(g.vp / 64, (g.rank + 63) / 64), dim3(kGThreads), 0, stream, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gather_et, dim3(g.n_pad / 64, (g.rank + 63) / 64), dim3(kGThreads), 0, stream, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool vec = (g.V % 4) == 0;
  switch (g.rank / 32) {
    case 1: e = launch_gemms<1>(g, vec, stream); break;
    case 2: e = launch_gemms<2>(g, vec, stream); break;
    case 3: e = launch_gemms<3>(g, vec, stream); break;
    case 4: e = launch_gemms<4>(g, vec, stream); break;
    case 5: e = launch_gemms<5>(g, vec, stream); break;
    case 6: e = launch_gemms<6>(g, vec, stream); break;
    case 7: e = launch_gemms<7>(g, vec, stream); break;
    case 8: e = launch_gemms<8>(g, vec, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(grad_e_reduce, dim3(blocks_for((size_t)g.n_rows * g.rank)), dim3(kGThreads), 0,
                     stream, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(zero_floats, dim3(blocks_for((size_t)g.V * g.rank)), dim3(kGThreads), 0, stream,
                     g.dW1, (size_t)g.V * g.rank);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scatter_dw1, dim3(g.n_rows), dim3(kGThreads), 0, stream, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(grad_dh, dim3(blocks_for((size_t)g.n_rows * g.d)), dim3(kGThreads), 0, stream, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(grad_dw, dim3(blocks_for((size_t)(g.d + g.rank))), dim3(kGThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace dspark

// RNN head [P1 "DSpark" §2.4; P3 アーキテクチャ]: a block-internal state s_k
// updated by a gate from the previous state, the previous token's embedding
// e_k = W1[x_{k-1}] and the backbone state h_k, read as a GRU cell (gate
// order reset, update, new; s_0 = 0):
//   r = sigma(W_ir [e;h] + b_ir + W_hr s + b_hr)
//   z = sigma(W_iz [e;h] + b_iz + W_hz s + b_hz)
//   n = tanh(W_in [e;h] + b_in + r * (W_hn s + b_hn))
//   s_k = (1 - z) n + z s_{k-1}
// bf16(s_k) then takes the place of e_k in the draft step's bias (the step
// kernel reads it through StepArgs::E_rows).
//
//   R1 rnn_input_proj   before the block, for every (request, position):
//      P = W_ih[:, rank:] h + b_ih  [R*gamma][3 rank] fp32 (bf16 MFMA, K = d);
//      h does not depend on the drafted tokens.
//   R2 rnn_state_step   per step k, after step k-1's winner is known:
//      the e part W_ih[:, :rank] e (bf16 MFMA, exact products) and the
//      recurrent part W_hh s (s split into two bf16 terms, hi + lo, so the
//      fp32 state keeps about 16 bits through the product), then the gates;
//      writes s_k (fp32) and bf16(s_k) for the step.
#include "dspark_kernels.h"
#include "dspark_device.h"

namespace dspark {

namespace {

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ bf16x8_t bf16x8_of(const float (&v)[8]) {
  bf16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = __builtin_bit_cast(__bf16, bf16_bits_rne(v[j]));
  return r;
}

// R1: wave (workgroup (bx, by), wave q) computes the 32 x 32 tile of rows
// 32 bx .. and outputs 32 (4 by + q) ..; A = h rows, B = W_ih rows (columns
// rank + k), both holding K contiguously.  Lane (l%32, half) supplies the 8
// k = 16 s + 8 half .. +7 of its row for K step s.
__global__ __launch_bounds__(256) void rnn_input_proj(RnnArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int n_rows = a.R * a.gamma, n_out = 3 * a.rank;
  const int nt = blockIdx.y * 4 + wave;
  if (nt * 32 >= n_out) return;  // no barriers in this kernel
  const int row = blockIdx.x * 32 + col;
  const int rowc = row < n_rows ? row : n_rows - 1;
  const uint16_t* hrow = a.h + (size_t)rowc * a.d + 8 * half;
  const uint16_t* wrow = a.W_ih + (size_t)(nt * 32 + col) * (a.rank + a.d) + a.rank + 8 * half;
  f32x16_t acc = f32x16_t{};
#pragma unroll 4
  for (int k0 = 0; k0 < a.d; k0 += 16) {
    const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(hrow + k0);
    const bf16x8_t wv = *reinterpret_cast<const bf16x8_t*>(wrow + k0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, wv, acc, 0, 0, 0);
  }
  // accumulator i: row 8 (i/4) + 4 half + i%4 of the tile, output nt*32 + col
  const int o = nt * 32 + col;
  const float b = a.b_ih[o];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = blockIdx.x * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (rr < n_rows) a.P[(size_t)rr * n_out + o] = acc[i] + b;
  }
}

// R2: wave (workgroup (jb, rt)) owns requests 32 rt .. +31 and state entries
// 32 jb .. +31.  MFMA M = requests, N = state entries, K = rank:
//   A  e:  W1[x_{k-1}[m]][k ..]       s:  hi / lo bf16 terms of s_{k-1}[m][k ..]
//   B  W_ih[g rank + n][k ..] (the e columns), W_hh[g rank + n][k ..]
__global__ __launch_bounds__(64) void rnn_state_step(RnnArgs a, int k, const float* s_prev,
                                                     float* s_next) {
  const int lane = threadIdx.x;
  const int half = lane >> 5, col = lane & 31;
  const int jb = blockIdx.x, rt = blockIdx.y;
  const int H = a.rank;
  const int m = rt * 32 + col;
  const int mc = m < a.R ? m : a.R - 1;
  int tok;
  if (k > 1)
    tok = winner_id(a.best[(size_t)(k - 2) * a.R + mc]);
  else
    tok = a.x[(size_t)mc * (a.gamma + 1)];
  tok = clamp_token(tok, a.V);
  const uint16_t* erow = a.W1 + (size_t)tok * H + 8 * half;
  const float* srow = s_prev + (size_t)mc * H + 8 * half;
  const int n = jb * 32 + col;

  f32x16_t gi[3], gh[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    gi[g] = f32x16_t{};
    gh[g] = f32x16_t{};
  }
  for (int k0 = 0; k0 < H; k0 += 16) {
    const bf16x8_t e = *reinterpret_cast<const bf16x8_t*>(erow + k0);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      const bf16x8_t wv = *reinterpret_cast<const bf16x8_t*>(
          a.W_ih + (size_t)(g * H + n) * (H + a.d) + k0 + 8 * half);
      gi[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e, wv, gi[g], 0, 0, 0);
    }
    if (k > 1) {  // s_0 = 0: the recurrent products vanish at the first step
      float hi[8], lo[8];
      const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(srow + k0);
      const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(srow + k0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[j] = s0[j];
        hi[4 + j] = s1[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = hi[j];
        hi[j] = bf16_value(bf16_bits_rne(v));
        lo[j] = v - hi[j];
      }
      const bf16x8_t shi = bf16x8_of(hi), slo = bf16x8_of(lo);
#pragma unroll
      for (int g = 0; g < 3; ++g) {
        const bf16x8_t wv = *reinterpret_cast<const bf16x8_t*>(a.W_hh + (size_t)(g * H + n) * H + k0 +
                                                               8 * half);
        gh[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(shi, wv, gh[g], 0, 0, 0);
        gh[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(slo, wv, gh[g], 0, 0, 0);
      }
    }
  }
  // accumulator i: request 32 rt + 8 (i/4) + 4 half + i%4, state entry n
  const float bhr = a.b_hh[n], bhz = a.b_hh[H + n], bhn = a.b_hh[2 * H + n];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (r >= a.R) continue;
    const float* pre = a.P + ((size_t)r * a.gamma + (k - 1)) * (3 * H);
    const float sp = k > 1 ? s_prev[(size_t)r * H + n] : 0.0f;
    const float rg = 1.0f / (1.0f + expf(-(gi[0][i] + pre[n] + gh[0][i] + bhr)));
    const float zg = 1.0f / (1.0f + expf(-(gi[1][i] + pre[H + n] + gh[1][i] + bhz)));
    const float ng = tanhf(gi[2][i] + pre[2 * H + n] + rg * (gh[2][i] + bhn));
    const float s = (1.0f - zg) * ng + zg * sp;
    s_next[(size_t)r * H + n] = s;
    a.E[(size_t)r * H + n] = bf16_bits_rne(s);
  }
}

}  // namespace

hipError_t launch_rnn_input_proj(const RnnArgs& a, hipStream_t stream) {
  const int n_rows = a.R * a.gamma, n_tiles = 3 * a.rank / 32;
  hipLaunchKernelGGL(rnn_input_proj, dim3((n_rows + 31) / 32, (n_tiles + 3) / 4), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_rnn_state_step(const RnnArgs& a, int k, const float* s_prev, float* s_next,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(rnn_state_step, dim3(a.rank / 32, (a.R + 31) / 32), dim3(64), 0, stream, a,
                     k, s_prev, s_next);
  return hipGetLastError();
}

}  // namespace dspark

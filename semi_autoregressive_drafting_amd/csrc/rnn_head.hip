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
//      P = W_ih[:, rank:] h + b_ih  [R*gamma][3 rank] fp32 (bf16 MFMA, K = d),
//      as kProjSplit partial sums over quarters of K; rnn_proj_reduce adds
//      them in order into the step-major Pk [gamma][R][3 rank].  h does not
//      depend on the drafted tokens.
//   R2 rnn_state_step   per step k, after step k-1's winner is known:
//      the e part W_ih[:, :rank] e (bf16 MFMA, exact products) and the
//      recurrent part W_hh s (s split into two bf16 terms, hi + lo, so the
//      fp32 state keeps about 16 bits through the product), then the gates;
//      writes s_k (fp32) and bf16(s_k) for the step.  rank <= 256.
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

// R1: workgroup (bx, by, z) computes the 128 x 128 block of rows 128 bx ..
// and outputs 128 by .. over the z-th of kProjSplit K ranges (partial sums
// P[z], the input bias in the first); wave q owns rows 64 (q / 2) .. +63 by
// outputs 64 (q % 2) .. +63 (2 x 2 MFMA tiles).  A = h rows, B = W_ih rows
// (columns rank + k); each 64-wide K chunk of both is copied into LDS once
// (16 bytes per thread and piece, rows padded to 72 elements), the next
// chunk's pieces loaded into registers while the current one multiplies.
// Lane (l%32, half) reads the 8 k = 16 s + 8 half .. +7 of its row for K
// step s.  K past d (a partial last chunk) reads as zero.
constexpr int kProjTile = 128;
constexpr int kProjRow = 72;  // LDS row stride (elements)

__global__ __launch_bounds__(256) void rnn_input_proj(RnnArgs a) {
  __shared__ __align__(16) uint16_t lA[kProjTile * kProjRow];
  __shared__ __align__(16) uint16_t lB[kProjTile * kProjRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int n_rows = a.R * a.gamma, n_out = 3 * a.rank;
  const int row0 = blockIdx.x * kProjTile, out0 = blockIdx.y * kProjTile;
  const int chunks = (a.d + 63) / 64, cq = (chunks + kProjSplit - 1) / kProjSplit;
  const int c_begin = min(chunks, (int)blockIdx.z * cq), c_end = min(chunks, c_begin + cq);

  // this thread's 4 pieces of each chunk: tile row p / 8, 8 K values at 8 (p % 8)
  const uint16_t* asrc[4];
  const uint16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pc = tid + 256 * i, r = pc >> 3;
    asrc[i] = a.h + (size_t)min(row0 + r, n_rows - 1) * a.d + 8 * (pc & 7);
    bsrc[i] = a.W_ih + (size_t)min(out0 + r, n_out - 1) * (a.rank + a.d) + a.rank + 8 * (pc & 7);
  }
  u32x4_t ra[4], rb[4];
  auto load = [&](int ch) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = ch * 64 + 8 * ((tid + 256 * i) & 7);
      const bool in = k0 < a.d;  // d % 16 == 0: a piece is wholly inside or outside
      ra[i] = in ? *reinterpret_cast<const u32x4_t*>(asrc[i] + ch * 64) : u32x4_t{};
      rb[i] = in ? *reinterpret_cast<const u32x4_t*>(bsrc[i] + ch * 64) : u32x4_t{};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + 256 * i, r = pc >> 3, q = pc & 7;
      *reinterpret_cast<u32x4_t*>(lA + r * kProjRow + 8 * q) = ra[i];
      *reinterpret_cast<u32x4_t*>(lB + r * kProjRow + 8 * q) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = f32x16_t{};
  const int mr = 64 * (wave >> 1), nr = 64 * (wave & 1);
  if (c_begin < c_end) {
    load(c_begin);
    store();
    __syncthreads();
    for (int ch = c_begin; ch < c_end; ++ch) {
      if (ch + 1 < c_end) load(ch + 1);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t x[2], wv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          x[t] = *reinterpret_cast<const bf16x8_t*>(lA + (mr + 32 * t + col) * kProjRow + 16 * s + 8 * half);
          wv[t] = *reinterpret_cast<const bf16x8_t*>(lB + (nr + 32 * t + col) * kProjRow + 16 * s + 8 * half);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[t], wv[u], acc[t][u], 0, 0, 0);
      }
      __syncthreads();  // every wave is past its reads of this chunk
      if (ch + 1 < c_end) {
        store();
        __syncthreads();
      }
    }
  }
  // accumulator i of tile (t, u): row row0 + mr + 32 t + 8 (i/4) + 4 half + i%4,
  // output out0 + nr + 32 u + col
  float* P = a.P + (size_t)blockIdx.z * n_rows * n_out;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = out0 + nr + 32 * u + col;
    if (o >= n_out) continue;
    const float b = blockIdx.z == 0 ? a.b_ih[o] : 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = row0 + mr + 32 * t + 8 * (i >> 2) + 4 * half + (i & 3);
        if (rr < n_rows) P[(size_t)rr * n_out + o] = acc[t][u][i] + b;
      }
  }
}

// R1b: Pk[k-1][r][o] = sum of the K quarters of P[.][r gamma + k - 1][o] in
// quarter order: one pass that also makes each step's projections one
// contiguous block (a step reads R * 3 rank values at once).
__global__ __launch_bounds__(256) void rnn_proj_reduce(RnnArgs a) {
  const int n_out = 3 * a.rank;
  const size_t total = (size_t)a.R * a.gamma * n_out;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int o = (int)(i % n_out);
  const size_t kr = i / n_out;  // (k - 1) * R + r
  const int r = (int)(kr % a.R), km1 = (int)(kr / a.R);
  const size_t src = ((size_t)r * a.gamma + km1) * n_out + o;
  float v = a.P[src];
#pragma unroll
  for (int q = 1; q < kProjSplit; ++q) v += a.P[(size_t)q * total + src];
  a.Pk[i] = v;
}

// R2: workgroup (eb, rt) owns requests 32 rt .. +31 and state entries
// 8 eb .. +7, with 4 waves, wave q taking K quarter q.  MFMA M = requests,
// N = (gate, entry) pairs: column c = 8 g + j holds gate g (reset, update,
// new) of entry 8 eb + j; columns 24 .. 31 are zero.
//   A  e:  W1[x_{k-1}[m]][k ..]       s:  hi / lo bf16 terms of s_{k-1}[m][k ..]
//   B  W_ih[g rank + n][k ..] (the e columns), W_hh[g rank + n][k ..]
// Each output keeps its operands, its K quarters and their fixed reduction
// order whatever column it sits in, so the entry-group width only decides
// how the work spreads: 8 entries per workgroup put the update on 4x as many
// CUs as 32 would, and a CU's loads (the W slices of its entries, the e and
// s_{k-1} rows of its requests, the input projections) are what bound the
// kernel.  Every wave issues its loads at the start, the token first, so
// that only the row gather waits for it; s_{k-1} is read once per workgroup
// as whole rows into LDS.  The quarters meet in LDS in a fixed order, the
// first one bringing the input projection and the recurrent bias; then each
// of the 256 threads forms s_k for one (request, entry).
constexpr int kStateQ = 4;         // K quarters = waves
constexpr int kStateEnt = 8;       // state entries per workgroup
constexpr int kStateMaxSteps = 4;  // K steps per quarter at rank 256

// winner_id of a winner word from its low 32 bits alone (~id; an empty word
// gives -1 either way), so the load fills one register and nothing reuses a
// half of it while it is in flight.
__device__ __forceinline__ int winner_id_low(const unsigned long long* w) {
  return (int)~*reinterpret_cast<const uint32_t*>(w);
}

// s_{k-1} rows of the workgroup's 32 requests, staged once in LDS (row
// stride kSRow floats).
constexpr int kSRow = 256 + 4;

template <bool kRec>
__device__ __forceinline__ void state_step_body(const RnnArgs& a, int k, const float* s_prev,
                                                float* s_next, float (*red)[2][16][64],
                                                float (*sl)[kSRow]) {
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int eb = blockIdx.x, rt = blockIdx.y;
  const int H = a.rank, KS = H / 16;
  const int kq = (KS + kStateQ - 1) / kStateQ;
  const int s_begin = min(KS, q * kq), s_end = min(KS, s_begin + kq);
  const int mc = min(rt * 32 + col, a.R - 1);
  // column col: gate cg, entry n (columns past 3 kStateEnt read a valid row
  // and are zeroed before the MFMAs)
  const bool cin = col < 3 * kStateEnt;
  const int cg = cin ? col / kStateEnt : 0;
  const int n = eb * kStateEnt + (cin ? col % kStateEnt : 0);
  const uint16_t* wi = a.W_ih + (size_t)(cg * H + n) * (H + a.d) + 8 * half;
  const uint16_t* wh = a.W_hh + (size_t)(cg * H + n) * H + 8 * half;
  // The token first: vector loads return in order, so its wait below leaves
  // every later load in flight and the row gather goes out a round trip after
  // the start instead of after all of the workgroup's bulk loads.
  int tok = k > 1 ? winner_id_low(a.best + winner_index(k - 2, a.R, mc))
                  : a.x[(size_t)mc * (a.gamma + 1)];
  // loads that do not depend on the token
  bf16x8_t wiv[kStateMaxSteps], whv[kStateMaxSteps], ev[kStateMaxSteps];
  f32x4_t sv[kStateMaxSteps][2];
#pragma unroll
  for (int j = 0; j < kStateMaxSteps; ++j) {
    const int k0 = 16 * min(s_begin + j, KS - 1);
    wiv[j] = *reinterpret_cast<const bf16x8_t*>(wi + k0);
    if constexpr (kRec) whv[j] = *reinterpret_cast<const bf16x8_t*>(wh + k0);
  }
  // s_{k-1} of the 32 requests (rows past R repeat row R - 1): whole rows,
  // 16 bytes per thread and piece, into LDS
  constexpr int kPieces = 32 * 256 / 4;
  constexpr int kThreads = 64 * kStateQ;
  f32x4_t spc[kPieces / kThreads];
  const int pieces = 32 * H / 4;
  if constexpr (kRec) {
#pragma unroll
    for (int i = 0; i < kPieces / kThreads; ++i) {
      const int pc = threadIdx.x + i * kThreads;
      const int row = pc / (H / 4), c4 = pc % (H / 4);
      const int rr = min(rt * 32 + row, a.R - 1);
      if (pc < pieces) spc[i] = *reinterpret_cast<const f32x4_t*>(s_prev + (size_t)rr * H + 4 * c4);
    }
  }
  // the first quarter also brings the input projection of step k and the
  // recurrent bias of its columns
  float pre[16];
  float bh = 0.0f;
  if (q == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = min(rt * 32 + 8 * (i >> 2) + 4 * half + (i & 3), a.R - 1);
      pre[i] = a.Pk[((size_t)(k - 1) * a.R + r) * (3 * H) + cg * H + n];
    }
    bh = a.b_hh[cg * H + n];
  }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the token is used
  tok = checked_token(tok, a.V, a.err);
  const uint16_t* erow = a.W1 + (size_t)tok * H + 8 * half;
#pragma unroll
  for (int j = 0; j < kStateMaxSteps; ++j)
    ev[j] = *reinterpret_cast<const bf16x8_t*>(erow + 16 * min(s_begin + j, KS - 1));
  __builtin_amdgcn_sched_barrier(0);  // the row loads go out together, before any is used

  if constexpr (kRec) {
#pragma unroll
    for (int i = 0; i < kPieces / kThreads; ++i) {
      const int pc = threadIdx.x + i * kThreads;
      if (pc < pieces) {
        const int row = pc / (H / 4), c4 = pc % (H / 4);
        *reinterpret_cast<f32x4_t*>(&sl[row][4 * c4]) = spc[i];
      }
    }
  }
  __syncthreads();  // s_{k-1} rows in LDS (read below and by the blend)
  if constexpr (kRec) {
#pragma unroll
    for (int j = 0; j < kStateMaxSteps; ++j) {
      const int k0 = 16 * min(s_begin + j, KS - 1) + 8 * half;
      sv[j][0] = *reinterpret_cast<const f32x4_t*>(&sl[col][k0]);
      sv[j][1] = *reinterpret_cast<const f32x4_t*>(&sl[col][k0 + 4]);
    }
  }

  f32x16_t gi = f32x16_t{}, gh = f32x16_t{};
#pragma unroll
  for (int j = 0; j < kStateMaxSteps; ++j) {
    if (s_begin + j >= s_end) break;
    const bf16x8_t wij = cin ? wiv[j] : bf16x8_t{};
    gi = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ev[j], wij, gi, 0, 0, 0);
    if constexpr (kRec) {
      const bf16x8_t whj = cin ? whv[j] : bf16x8_t{};
      float hi[8], lo[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        hi[t] = sv[j][0][t];
        hi[4 + t] = sv[j][1][t];
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float v = hi[t];
        hi[t] = bf16_value(bf16_bits_rne(v));
        lo[t] = v - hi[t];
      }
      gh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16x8_of(hi), whj, gh, 0, 0, 0);
      gh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf16x8_of(lo), whj, gh, 0, 0, 0);
    }
  }
  // quarters in a fixed order over two LDS slots: slot 0 = (q0 + input
  // projection) + q2, slot 1 = q1 + q3 (the recurrent part likewise, with its
  // bias in q0), and the gate input is slot 0 + slot 1
  if (q < 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      red[q][0][i][lane] = q == 0 ? gi[i] + pre[i] : gi[i];
      red[q][1][i][lane] = q == 0 ? gh[i] + bh : gh[i];
    }
  }
  __syncthreads();
  if (q >= 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      red[q - 2][0][i][lane] += gi[i];
      red[q - 2][1][i][lane] += gh[i];
    }
  }
  __syncthreads();
  // thread t forms s_k of request 32 rt + m and entry 8 eb + j (m = t / 8,
  // j = t % 8); accumulator i of lane l holds request 8 (i/4) + 4 (l/32) + i%4
  // of column l%32
  const int m = threadIdx.x / kStateEnt, j = threadIdx.x % kStateEnt;
  const int r = rt * 32 + m;
  if (m >= 32 || r >= a.R) return;
  const int i = 4 * (m >> 3) + (m & 3), ll = 32 * ((m >> 2) & 1);
  auto part = [&](int gate, int which) {
    return red[0][which][i][ll + gate * kStateEnt + j] + red[1][which][i][ll + gate * kStateEnt + j];
  };
  const int nn = eb * kStateEnt + j;
  const float rg = 1.0f / (1.0f + expf(-(part(0, 0) + part(0, 1))));
  const float zg = 1.0f / (1.0f + expf(-(part(1, 0) + part(1, 1))));
  const float ng = tanhf(part(2, 0) + rg * part(2, 1));
  const float s = (1.0f - zg) * ng + zg * (kRec ? sl[m][nn] : 0.0f);
  s_next[(size_t)r * H + nn] = s;
  a.E[(size_t)r * H + nn] = bf16_bits_rne(s);
  if (a.rows_out) a.rows_out[((size_t)r * a.gamma + (k - 1)) * H + nn] = bf16_bits_rne(s);
}

__global__ __launch_bounds__(64 * kStateQ) void rnn_state_step(RnnArgs a, int k,
                                                               const float* s_prev,
                                                               float* s_next) {
  __shared__ float red[2][2][16][64];  // slot, input / recurrent part
  __shared__ __align__(16) float sl[32][kSRow];
  if (k > 1)
    state_step_body<true>(a, k, s_prev, s_next, red, sl);
  else
    state_step_body<false>(a, k, s_prev, s_next, red, sl);  // s_0 = 0
}

}  // namespace

hipError_t launch_rnn_input_proj(const RnnArgs& a, hipStream_t stream) {
  const int n_rows = a.R * a.gamma, n_out = 3 * a.rank;
  hipLaunchKernelGGL(rnn_input_proj,
                     dim3((n_rows + kProjTile - 1) / kProjTile, (n_out + kProjTile - 1) / kProjTile,
                          kProjSplit),
                     dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)n_rows * n_out;
  hipLaunchKernelGGL(rnn_proj_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rnn_state_step(const RnnArgs& a, int k, const float* s_prev, float* s_next,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(rnn_state_step, dim3(a.rank / kStateEnt, (a.R + 31) / 32), dim3(64 * kStateQ), 0,
                     stream, a, k, s_prev, s_next);
  return hipGetLastError();
}

}  // namespace dspark

// Verification of drafted blocks: per-position c* and lossless rejection
// sampling [P1 "DSpark" §3.1 eq. c*; the opening and §2.2 on standard
// rejection sampling; P3 問題定義 and アーキテクチャ (decoding cycle)].
//
// Rows are (request, position) pairs, row = r*gamma + (k-1), matching the
// [R][gamma][V] layout of U and the target logits.
//
//   V1 verify_target_lse  grid (chunks, rows): per vocabulary chunk of a
//      target row, online max / sum of 2^(t - m), t = target * log2e / T
//      (greedy: max and lowest argmax).
//   V2 verify_accept      one workgroup, one thread per request: merge V1's
//      chunks -> lse_t per row; run the acceptance chain over the admitted
//      prefix (u < p_t(x_j) / p_d(x_j)); flag the row that needs a sample
//      (1 = residual at the first rejection, 2 = bonus at row ell+1); write
//      n_accept, tau and tau_mean.  Greedy: also c* and the correction token.
//   V3 verify_main        (T > 0) one pass over W2t, U and the target logits
//      for all rows: bias tile by MFMA, p_d and p_t, sum |p_d - p_t|, and for
//      flagged rows the Gumbel race over max(p_t - p_d, 0) or p_t.
//   V4 verify_finalize    (T > 0) per row: fixed-order merge of V3's slab
//      partials -> c* = 1 - sum/2; the flagged row's winner -> next_token.
#include "dspark_kernels.h"
#include "mfma_stream.h"

namespace dspark {

namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ int chunk_size(int V, int chunks) {
  const int cs = (V + chunks - 1) / chunks;
  return (cs + 3) & ~3;
}

// ---------------------------------------------------------------------------
// V1: target normaliser partials.
// ---------------------------------------------------------------------------
template <bool kGreedy, bool kVec>
__global__ __launch_bounds__(256) void verify_target_lse(VerifyArgs a, VerifyPlan p) {
  __shared__ float sm[256];
  __shared__ float ss[256];
  __shared__ int si[256];
  const int row = blockIdx.y, c = blockIdx.x, t = threadIdx.x;
  const float* trow = a.target + (size_t)row * a.V;
  const int cs = chunk_size(a.V, p.lse_chunks);
  const int v0 = c * cs;
  const int v1 = min(a.V, v0 + cs);
  float m = -INFINITY, S = 0.0f;
  int idx = -1;
  for (int v = v0 + 4 * t; v < v1; v += 1024) {
    float x[4];
    if (kVec && v + 4 <= v1) {
      const f32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(trow + v));
      x[0] = q[0]; x[1] = q[1]; x[2] = q[2]; x[3] = q[3];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (v + i < v1) ? trow[v + i] : -INFINITY;
    }
    if constexpr (kGreedy) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool win = (v + i < v1) && (x[i] > m);
        m = win ? x[i] : m;
        idx = win ? v + i : idx;
      }
    } else {
      float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      const float mn = fmaxf(m, xm * a.kscale);
      S *= (mn == -INFINITY) ? 1.0f : fast_exp2(m - mn);
      m = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) S += fast_exp2(fmaf(x[i], a.kscale, -mn));
    }
  }
  sm[t] = m;
  ss[t] = S;
  si[t] = idx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) {
      const float m1 = sm[t], m2 = sm[t + s];
      if constexpr (kGreedy) {
        const int i1 = si[t], i2 = si[t + s];
        const bool take2 = (i2 >= 0) && (i1 < 0 || m2 > m1 || (m2 == m1 && i2 < i1));
        sm[t] = take2 ? m2 : m1;
        si[t] = take2 ? i2 : i1;
      } else {
        const float M = fmaxf(m1, m2);
        ss[t] = (M == -INFINITY) ? 0.0f
                                 : ss[t] * fast_exp2(m1 - M) + ss[t + s] * fast_exp2(m2 - M);
        sm[t] = M;
      }
    }
    __syncthreads();
  }
  if (t == 0) {
    float* out = reinterpret_cast<float*>(a.ws + p.off_lsepart) + ((size_t)row * p.lse_chunks + c) * 2;
    out[0] = sm[0];
    if (kGreedy) reinterpret_cast<int*>(out)[1] = si[0];
    else out[1] = ss[0];
  }
}

// ---------------------------------------------------------------------------
// V2: acceptance chain, one thread per request.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void verify_accept(VerifyArgs a, VerifyPlan p) {
  __shared__ int stau[512];
  const int r = threadIdx.x;
  float* lse_t2 = reinterpret_cast<float*>(a.ws + p.off_lse_t);
  int* targmax = reinterpret_cast<int*>(a.ws + p.off_lse_t);  // greedy reuses the slot
  int* flag = reinterpret_cast<int*>(a.ws + p.off_flag);
  const float* lp = reinterpret_cast<const float*>(a.ws + p.off_lsepart);
  int tau = 0;
  if (r < a.R) {
    for (int k = 1; k <= a.gamma; ++k) {
      const int row = r * a.gamma + (k - 1);
      const float* q = lp + (size_t)row * p.lse_chunks * 2;
      if (a.greedy) {
        float m = -INFINITY;
        int idx = -1;
        for (int c = 0; c < p.lse_chunks; ++c) {
          const float mc = q[2 * c];
          const int ic = reinterpret_cast<const int*>(q)[2 * c + 1];
          const bool take = (ic >= 0) && (idx < 0 || mc > m || (mc == m && ic < idx));
          m = take ? mc : m;
          idx = take ? ic : idx;
        }
        targmax[row] = idx;
        a.c_star[row] = (a.x[(size_t)r * (a.gamma + 1) + k] == idx) ? 1.0f : 0.0f;
      } else {
        float m = -INFINITY, S = 0.0f;
        for (int c = 0; c < p.lse_chunks; ++c) {
          const float mc = q[2 * c], sc = q[2 * c + 1];
          const float M = fmaxf(m, mc);
          S = (M == -INFINITY) ? 0.0f : S * fast_exp2(m - M) + sc * fast_exp2(mc - M);
          m = M;
        }
        lse_t2[row] = m + log2f(S);
      }
      flag[row] = 0;
    }
    int n_acc = 0, nxt = -1;
    bool rejected = false;
    int ell = a.ell[r];
    ell = ell < 0 ? 0 : (ell > a.gamma ? a.gamma : ell);  // device values are not validated
    for (int j = 1; j <= ell; ++j) {
      const int row = r * a.gamma + (j - 1);
      int xj = a.x[(size_t)r * (a.gamma + 1) + j];
      xj = xj < 0 ? 0 : (xj >= a.V ? a.V - 1 : xj);
      float ratio;
      if (a.greedy) {
        ratio = (xj == targmax[row]) ? 1.0f : 0.0f;
      } else {
        const float pt = exp2f(fmaf(a.target[(size_t)row * a.V + xj], a.kscale, -lse_t2[row]));
        ratio = pt / a.p_d_x[row];
      }
      const float u = bits_to_uniform(pcg(row_key(a.seed, kStreamAccept, (uint32_t)r, (uint32_t)j)));
      if (u < ratio) {
        ++n_acc;
      } else {
        flag[row] = 1;
        if (a.greedy) nxt = targmax[row];
        rejected = true;
        break;
      }
    }
    if (!rejected && ell < a.gamma) {
      const int row = r * a.gamma + ell;
      flag[row] = 2;
      if (a.greedy) nxt = targmax[row];
    }
    a.n_accept[r] = n_acc;
    a.tau[r] = n_acc + 1;
    a.next_token[r] = nxt;
    tau = n_acc + 1;
  }
  stau[r] = tau;
  __syncthreads();
  for (int s = 256; s > 0; s >>= 1) {
    if (r < s) stau[r] += stau[r + s];
    __syncthreads();
  }
  if (r == 0) *a.tau_mean = (float)stau[0] / (float)a.R;
}

// ---------------------------------------------------------------------------
// V3: the fused pass over all rows (T > 0).
// ---------------------------------------------------------------------------
template <bool kVec>
struct VerifyEpi {
  const float* urow;
  const float* trow;
  int V, half;
  float kscale, lse2_d, lse2_t;
  int flag;
  uint32_t state_row;
  float ucur[16], unext[16], tcur[16], tnext[16];
  float sabs, bE, bLn;
  int bV;

  __device__ void prefetch(int vt) {
    load16<kVec>(unext, urow, vt * kVTile + 16 * half, V);
    load16<kVec>(tnext, trow, vt * kVTile + 16 * half, V);
  }
  __device__ void advance() {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ucur[i] = unext[i];
      tcur[i] = tnext[i];
    }
  }
  __device__ void consume(const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * half;
    const bool full = (vt + 1) * kVTile <= V;
    float pd[16], pt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = full || (vb + i < V);
      pd[i] = ok ? fast_exp2(fmaf(ucur[i] + acc[i], kscale, -lse2_d)) : 0.0f;
      pt[i] = ok ? fast_exp2(fmaf(tcur[i], kscale, -lse2_t)) : 0.0f;
      sabs += fabsf(pd[i] - pt[i]);
    }
    if (__ballot(flag != 0) != 0ull) {
      const uint32_t s0 = state_row + (uint32_t)vb * kLcgMul;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = (flag == 1) ? fmaxf(pt[i] - pd[i], 0.0f) : pt[i];
        const float ln = fast_log2(bits_to_uniform(rxs_m_xs(s0 + (uint32_t)i * kLcgMul)));
        const bool win = e * bLn < bE * ln;
        bE = win ? e : bE;
        bLn = win ? ln : bLn;
        bV = win ? vb + i : bV;
      }
    }
  }
};

template <class W, bool kVec>
__global__ __launch_bounds__(kStreamThreads) void verify_main(VerifyArgs a, VerifyPlan p) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int b = blockIdx.x;
  int slab, grp;
  if (p.n_groups == 1 || p.n_slabs % 8 != 0) {
    slab = b % p.n_slabs;
    grp = b / p.n_slabs;
  } else {
    grp = (b >> 3) % p.n_groups;
    slab = (b / (8 * p.n_groups)) * 8 + (b & 7);
  }
  const int t_begin = (int)(((long long)slab * p.n_vtiles) / p.n_slabs);
  const int t_end = (int)(((long long)(slab + 1) * p.n_vtiles) / p.n_slabs);

  const int row = (grp * kWaves + wave) * kVTile + col;
  const int rowc = row < p.n_rows ? row : p.n_rows - 1;
  const int r = rowc / a.gamma, k = rowc % a.gamma + 1;
  typename W::frag_t e[W::kMaxKs];
  load_e_frags<W>(e, a.W1, a.x[(size_t)r * (a.gamma + 1) + (k - 1)], a.rank, a.V, half);

  const int* flag = reinterpret_cast<const int*>(a.ws + p.off_flag);
  VerifyEpi<kVec> epi;
  epi.urow = a.U + (size_t)rowc * a.V;
  epi.trow = a.target + (size_t)rowc * a.V;
  epi.V = a.V;
  epi.half = half;
  epi.kscale = a.kscale;
  epi.lse2_d = a.lse_d[rowc] * kLog2e;
  epi.lse2_t = reinterpret_cast<const float*>(a.ws + p.off_lse_t)[rowc];
  epi.flag = row < p.n_rows ? flag[rowc] : 0;
  const uint32_t stream = epi.flag == 1 ? kStreamResid : kStreamBonus;
  epi.state_row = row_key(a.seed, stream, (uint32_t)r, (uint32_t)k) * kLcgMul + kLcgInc;
  epi.sabs = 0.0f;
  epi.bE = 0.0f;
  epi.bLn = -1.0f;
  epi.bV = -1;
  shared_a_stream<W>(a.W2t, a.V, a.rank, t_begin, t_end, e, lds, epi);

  // merge the two lane halves of each row
  const float s_o = __shfl_xor(epi.sabs, 32);
  float key = (epi.bV >= 0 && epi.bE > 0.0f) ? fast_log2(epi.bE) - fast_log2(-epi.bLn) : -INFINITY;
  int idx = (epi.bV >= 0 && epi.bE > 0.0f) ? epi.bV : -1;
  const float key_o = __shfl_xor(key, 32);
  const int idx_o = __shfl_xor(idx, 32);
  if (rec_beats(key_o, idx_o, key, idx)) {
    key = key_o;
    idx = idx_o;
  }
  if (half == 0 && row < p.n_rows) {
    const size_t plane = (size_t)p.n_rows * p.n_slabs;
    float* part = reinterpret_cast<float*>(a.ws + p.off_part);
    const size_t o = (size_t)row * p.n_slabs + slab;
    part[o] = epi.sabs + s_o;
    part[plane + o] = key;
    reinterpret_cast<int*>(part)[2 * plane + o] = idx;
  }
}

// ---------------------------------------------------------------------------
// V4: per-row finalisation (T > 0).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void verify_finalize(VerifyArgs a, VerifyPlan p) {
  const int row = blockIdx.x, t = threadIdx.x;
  const size_t plane = (size_t)p.n_rows * p.n_slabs;
  const float* part = reinterpret_cast<const float*>(a.ws + p.off_part) + (size_t)row * p.n_slabs;
  const int* pidx = reinterpret_cast<const int*>(a.ws + p.off_part) + 2 * plane + (size_t)row * p.n_slabs;
  float s = 0.0f, key = -INFINITY;
  int idx = -1;
  for (int j = t; j < p.n_slabs; j += 64) {
    s += part[j];
    const float kj = part[plane + j];
    const int ij = pidx[j];
    if (rec_beats(kj, ij, key, idx)) {
      key = kj;
      idx = ij;
    }
  }
  for (int m = 32; m > 0; m >>= 1) {
    s += __shfl_xor(s, m);
    const float ko = __shfl_xor(key, m);
    const int io = __shfl_xor(idx, m);
    if (rec_beats(ko, io, key, idx)) {
      key = ko;
      idx = io;
    }
  }
  if (t == 0) {
    a.c_star[row] = 1.0f - 0.5f * s;
    const int f = reinterpret_cast<const int*>(a.ws + p.off_flag)[row];
    if (f != 0) a.next_token[row / a.gamma] = idx;
  }
}

template <class W>
hipError_t launch_main(const VerifyArgs& a, const VerifyPlan& p, hipStream_t stream) {
  const int grid = p.n_slabs * p.n_groups;
  if (a.V % 4 == 0)
    hipLaunchKernelGGL((verify_main<W, true>), dim3(grid), dim3(kStreamThreads),
                       stream_lds_bytes<W>(a.rank), stream, a, p);
  else
    hipLaunchKernelGGL((verify_main<W, false>), dim3(grid), dim3(kStreamThreads),
                       stream_lds_bytes<W>(a.rank), stream, a, p);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

VerifyPlan plan_verify(int R, int V, int gamma) {
  VerifyPlan p{};
  p.n_rows = R * gamma;
  p.n_rtiles = (p.n_rows + kVTile - 1) / kVTile;
  p.n_groups = (p.n_rtiles + kWaves - 1) / kWaves;
  p.n_vtiles = (V + kVTile - 1) / kVTile;
  int slabs = kResidentWgs / p.n_groups;
  if (p.n_groups > 1) slabs = (slabs / 8) * 8;
  if (slabs < 8) slabs = 8;
  if (slabs > p.n_vtiles) slabs = p.n_vtiles;
  if (p.n_groups > 1 && slabs % 8 != 0 && p.n_vtiles >= 8) slabs = (p.n_vtiles / 8) * 8;
  p.n_slabs = slabs;
  int chunks = (2048 + p.n_rows - 1) / p.n_rows;
  const int max_chunks = (V + 1023) / 1024;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks > 64) chunks = 64;
  if (chunks < 1) chunks = 1;
  p.lse_chunks = chunks;
  size_t off = 0;
  p.off_lse_t = off;
  off = align256(off + (size_t)p.n_rows * 4);
  p.off_tx = off;  // reserved
  p.off_flag = off;
  off = align256(off + (size_t)p.n_rows * 4);
  p.off_lsepart = off;
  off = align256(off + (size_t)p.n_rows * p.lse_chunks * 8);
  p.off_part = off;
  off = align256(off + (size_t)3 * p.n_rows * p.n_slabs * 4);
  p.ws_bytes = off;
  return p;
}

hipError_t launch_verify(const VerifyArgs& a, const VerifyPlan& p, hipStream_t stream) {
  const bool vec = (a.V % 4) == 0;
  const dim3 g1(p.lse_chunks, p.n_rows);
  if (a.greedy) {
    if (vec) hipLaunchKernelGGL((verify_target_lse<true, true>), g1, dim3(256), 0, stream, a, p);
    else hipLaunchKernelGGL((verify_target_lse<true, false>), g1, dim3(256), 0, stream, a, p);
  } else {
    if (vec) hipLaunchKernelGGL((verify_target_lse<false, true>), g1, dim3(256), 0, stream, a, p);
    else hipLaunchKernelGGL((verify_target_lse<false, false>), g1, dim3(256), 0, stream, a, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_accept, dim3(1), dim3(512), 0, stream, a, p);
  e = hipGetLastError();
  if (e != hipSuccess || a.greedy) return e;
  e = a.bf16 ? launch_main<WBf16>(a, p, stream) : launch_main<WF32>(a, p, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_finalize, dim3(p.n_rows), dim3(64), 0, stream, a, p);
  return hipGetLastError();
}

}  // namespace dspark

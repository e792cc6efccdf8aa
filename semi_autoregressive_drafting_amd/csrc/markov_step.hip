// Fused DSpark Markov draft step for gfx950.
//
// One sequential step k over R requests [P1 "DSpark" §2.2 eq. p_k, §2.3 eq. B,
// §3.1 eq. c_k, §1.1 eq. a_j; the §6.2 vLLM loop fixes the per-position order]:
//
//   pass 1 (markov_partial_*): for a vocabulary slab, gather E = W1[x_{k-1}],
//     form the bias tile E . W2 with bf16 (or fp32) MFMA, add the base logits
//     U_k, and fold the tile into an online max / sum-exp and a Gumbel race,
//     so the R x V bias never reaches HBM.  The race is argmax_v s_v + G_v in
//     its exponential-race form: the winner maximises e_v / L_v with
//     e_v = 2^(t_v - m) (already needed for the sum) and L_v = -log2 u_v, which
//     costs one logarithm per entry.  Each workgroup (shared shape) or wave
//     (private shape) writes one partial record per request.
//   pass 2 (markov_combine): one workgroup per request merges the records in a
//     fixed order -> x_k, p_k(x_k), lse_k; then the confidence head and the
//     survival product.
//
// Launch shapes (see mfma_stream.h):
//   shared : R > 96.  4 waves = 4 request tiles (128 requests); each wave keeps
//            its E fragments in VGPRs for the whole step and the W2t tile is
//            staged once per workgroup in LDS.  W2t leaves HBM once per group of
//            128 requests; the groups of one slab share an XCD (blockIdx % 8)
//            so that their repeated W2t reads hit that XCD's L2.
//   private: R <= 96.  Every wave streams its own vocabulary tiles with the W2t
//            fragment loaded straight into VGPRs; grid.y = request tile.
#include "dspark_kernels.h"
#include "mfma_stream.h"

namespace dspark {

namespace {

constexpr int kWaves = 4;

// Per-lane online state over the lane's vocabulary entries of one request.
struct LaneState {
  float m;    // running max of t = z * kscale
  float S;    // sum of 2^(t - m)
  float bE;   // race winner's 2^(t - m) (rescaled with m); greedy: best z
  float bLn;  // race winner's log2(u) < 0
  int bV;     // winner id, -1 if none
};

template <bool kGreedy, bool kDebug, bool kVec>
struct DraftEpi {
  const float* urow;
  float* zdbg;
  int V, R, r, half;
  float kscale;
  uint32_t state_row;  // LCG state of vocabulary entry 0 of this row
  float ucur[16], unext[16];
  LaneState st;

  __device__ DraftEpi(const StepArgs& a, int r_, int rc, int half_)
      : zdbg(a.z_debug), V(a.V), R(a.R), r(r_), half(half_), kscale(a.kscale) {
    urow = a.U + ((size_t)rc * a.gamma + (a.k - 1)) * a.V;
    state_row = row_key(a.seed, kStreamDraft, (uint32_t)rc, (uint32_t)a.k) * kLcgMul + kLcgInc;
    st.m = -INFINITY;
    st.S = 0.0f;
    st.bE = kGreedy ? -INFINITY : 0.0f;
    st.bLn = -1.0f;
    st.bV = -1;
  }
  __device__ void prefetch(int vt) { load16<kVec>(unext, urow, vt * kVTile + 16 * half, V); }
  __device__ void advance() {
#pragma unroll
    for (int i = 0; i < 16; ++i) ucur[i] = unext[i];
  }

  template <bool kMasked>
  __device__ __forceinline__ void fold(const float (&z)[16], int vb) {
    if constexpr (kGreedy) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool win = (!kMasked || vb + i < V) && (z[i] > st.bE);
        st.bE = win ? z[i] : st.bE;
        st.bV = win ? vb + i : st.bV;
      }
    } else {
      float zm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) zm = (!kMasked || vb + i < V) ? fmaxf(zm, z[i]) : zm;
      const float mnew = fmaxf(st.m, zm * kscale);
      const float f = (mnew == -INFINITY) ? 1.0f : fast_exp2(st.m - mnew);
      st.S *= f;
      st.bE *= f;
      st.m = mnew;
      const float negm = -mnew;
      const uint32_t s0 = state_row + (uint32_t)vb * kLcgMul;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float e = fast_exp2(fmaf(z[i], kscale, negm));
        if constexpr (kMasked) e = (vb + i < V) ? e : 0.0f;
        st.S += e;
        const float ln = fast_log2(bits_to_uniform(rxs_m_xs(s0 + (uint32_t)i * kLcgMul)));
        // e / L > bE / bL  <=>  e * bLn < bE * ln     (L = -ln > 0)
        const bool win = e * st.bLn < st.bE * ln;
        st.bE = win ? e : st.bE;
        st.bLn = win ? ln : st.bLn;
        st.bV = win ? vb + i : st.bV;
      }
    }
  }

  __device__ void consume(const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * half;
    float z[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = ucur[i] + acc[i];
    if constexpr (kDebug) {
      if (r < R) {
        for (int i = 0; i < 16; ++i)
          if (vb + i < V) zdbg[(size_t)r * V + vb + i] = z[i];
      }
    }
    if ((vt + 1) * kVTile <= V)
      fold<false>(z, vb);
    else
      fold<true>(z, vb);
  }

  __device__ Rec record() const {
    Rec q;
    if (kGreedy) {
      q.m = st.bE;
      q.S = 0.0f;
      q.key = st.bE;
      q.tbest = st.bE;
      q.idx = st.bV;
    } else {
      q.m = st.m;
      q.S = st.S;
      if (st.bV >= 0 && st.bE > 0.0f) {
        q.tbest = st.m + fast_log2(st.bE);
        q.key = q.tbest - fast_log2(-st.bLn);
        q.idx = st.bV;
      } else {
        q.tbest = -INFINITY;
        q.key = -INFINITY;
        q.idx = -1;
      }
    }
    return q;
  }
};

__device__ __forceinline__ void store_rec(float* part, int R, int P, int r, int slot, const Rec& q) {
  const size_t plane = (size_t)R * P;
  const size_t o = (size_t)r * P + slot;
  part[o] = q.m;
  part[plane + o] = q.S;
  part[2 * plane + o] = q.key;
  part[3 * plane + o] = q.tbest;
  reinterpret_cast<int*>(part)[4 * plane + o] = q.idx;
}

template <class W, bool kGreedy, bool kDebug, bool kVec>
__global__ __launch_bounds__(kStreamThreads) void markov_partial_shared(StepArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;

  // blockIdx -> (slab, group); the groups of one slab land on the same XCD.
  const int b = blockIdx.x;
  int slab, grp;
  if (a.n_groups == 1 || a.n_slabs % 8 != 0) {
    slab = b % a.n_slabs;
    grp = b / a.n_slabs;
  } else {
    grp = (b >> 3) % a.n_groups;
    slab = (b / (8 * a.n_groups)) * 8 + (b & 7);
  }
  const int t_begin = (int)(((long long)slab * a.n_vtiles) / a.n_slabs);
  const int t_end = (int)(((long long)(slab + 1) * a.n_vtiles) / a.n_slabs);

  const int r = (grp * kWaves + wave) * kVTile + col;
  const int rc = r < a.R ? r : a.R - 1;  // padded lanes recompute row R-1, never stored
  typename W::frag_t e[W::kMaxKs];
  load_e_frags<W>(e, a.W1, a.x[(size_t)rc * (a.gamma + 1) + (a.k - 1)], a.rank, a.V, half);

  DraftEpi<kGreedy, kDebug, kVec> epi(a, r, rc, half);
  shared_a_stream<W>(a.W2t, a.V, a.rank, t_begin, t_end, e, lds, epi);

  Rec q = epi.record();
  q = rec_merge(q, rec_shfl_xor(q, 32));
  if (half == 0 && r < a.R) store_rec(a.part, a.R, a.n_parts, r, slab, q);
}

template <class W, bool kGreedy, bool kDebug, bool kVec>
__global__ __launch_bounds__(kStreamThreads) void markov_partial_private(StepArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int ws = blockIdx.x * kWaves + wave;
  const int t_begin = (int)(((long long)ws * a.n_vtiles) / a.n_parts);
  const int t_end = (int)(((long long)(ws + 1) * a.n_vtiles) / a.n_parts);

  const int r = blockIdx.y * kVTile + col;
  const int rc = r < a.R ? r : a.R - 1;
  typename W::frag_t e[W::kMaxKs];
  load_e_frags<W>(e, a.W1, a.x[(size_t)rc * (a.gamma + 1) + (a.k - 1)], a.rank, a.V, half);

  DraftEpi<kGreedy, kDebug, kVec> epi(a, r, rc, half);
  private_a_stream<W>(a.W2t, a.V, a.rank, t_begin, t_end, e, epi);

  Rec q = epi.record();
  q = rec_merge(q, rec_shfl_xor(q, 32));
  if (half == 0 && r < a.R) store_rec(a.part, a.R, a.n_parts, r, ws, q);
}

// One workgroup per request: fixed-order merge of the partial records, then
// the confidence head and the survival product.
template <class W>
__global__ __launch_bounds__(256) void markov_combine(StepArgs a) {
  using store_t = typename W::store_t;
  __shared__ Rec srec[256];
  __shared__ float sbuf[256];
  const int r = blockIdx.x, t = threadIdx.x;
  const size_t plane = (size_t)a.R * a.n_parts;
  const float* pm = a.part + (size_t)r * a.n_parts;
  const int* pidx = reinterpret_cast<const int*>(a.part) + 4 * plane + (size_t)r * a.n_parts;

  Rec acc{-INFINITY, 0.0f, -INFINITY, -INFINITY, -1};
  for (int j = t; j < a.n_parts; j += 256) {
    const Rec q{pm[j], pm[plane + j], pm[2 * plane + j], pm[3 * plane + j], pidx[j]};
    acc = rec_merge(acc, q);
  }
  srec[t] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) srec[t] = rec_merge(srec[t], srec[t + s]);
    __syncthreads();
  }

  const size_t o = (size_t)r * a.gamma + (a.k - 1);
  int xp = a.x[(size_t)r * (a.gamma + 1) + (a.k - 1)];
  xp = xp < 0 ? 0 : (xp >= a.V ? a.V - 1 : xp);
  const bool conf = a.h != nullptr && a.w != nullptr;
  float dot = 0.0f;
  if (conf) {
    const store_t* hrow = reinterpret_cast<const store_t*>(a.h) + o * a.d;
    const store_t* erow = reinterpret_cast<const store_t*>(a.W1) + (size_t)xp * a.rank;
    dot = block_sum256(conf_partial<W>(hrow, erow, a.w, a.d, a.rank, t), sbuf);
  }
  if (t == 0) {
    const Rec f = srec[0];
    a.x[(size_t)r * (a.gamma + 1) + a.k] = f.idx;
    if (a.greedy) {
      a.p[o] = 1.0f;
      a.lse[o] = f.m;
    } else {
      const float lse2 = f.m + log2f(f.S);
      a.p[o] = exp2f(f.tbest - lse2);
      a.lse[o] = lse2 * kLn2;
    }
    if (conf) {
      const float c = sigmoid_f32(dot);
      const float prev = (a.k == 1) ? 1.0f : a.a[o - 1];
      a.c[o] = c;
      a.a[o] = __fmul_rn(prev, c);
    }
  }
}

template <class W, bool kGreedy, bool kDebug, bool kVec>
void launch_partial(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  if (plan.shared) {
    hipLaunchKernelGGL((markov_partial_shared<W, kGreedy, kDebug, kVec>), dim3(plan.grid_x),
                       dim3(kStreamThreads), stream_lds_bytes<W>(a.rank), stream, a);
  } else {
    hipLaunchKernelGGL((markov_partial_private<W, kGreedy, kDebug, kVec>),
                       dim3(plan.grid_x, plan.grid_y), dim3(kStreamThreads), 0, stream, a);
  }
}

template <class W, bool kGreedy>
void launch_partial_g(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  const bool vec = (a.V % 4) == 0;
  if (a.z_debug != nullptr) {
    if (vec) launch_partial<W, kGreedy, true, true>(a, plan, stream);
    else launch_partial<W, kGreedy, true, false>(a, plan, stream);
  } else {
    if (vec) launch_partial<W, kGreedy, false, true>(a, plan, stream);
    else launch_partial<W, kGreedy, false, false>(a, plan, stream);
  }
}

template <class W>
hipError_t launch_step_w(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  if (a.greedy) launch_partial_g<W, true>(a, plan, stream);
  else launch_partial_g<W, false>(a, plan, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((markov_combine<W>), dim3(a.R), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Launch planning depends only on the sizes (never on the device), so every
// run of a given problem merges its partial results in the same order.
StepPlan plan_draft_step(int R, int V) {
  StepPlan p{};
  p.n_vtiles = (V + kVTile - 1) / kVTile;
  const int rt = (R + kVTile - 1) / kVTile;
  if (rt >= 4) {
    p.shared = true;
    p.n_groups = (rt + kWaves - 1) / kWaves;
    // Two resident workgroups on each of the 256 CUs (the T > 0 kernel needs
    // about 230 registers per lane, so two waves per SIMD).
    int slabs = kResidentWgs / p.n_groups;
    if (p.n_groups > 1) slabs = (slabs / 8) * 8;
    if (slabs < 8 && p.n_groups > 1) slabs = 8;
    if (slabs > p.n_vtiles) slabs = p.n_vtiles;
    if (slabs < 1) slabs = 1;
    if (p.n_groups > 1 && slabs % 8 != 0 && p.n_vtiles >= 8) slabs = (p.n_vtiles / 8) * 8;
    // (fewer than 8 tiles: plain slab-major order, see markov_partial_shared)
    p.n_slabs = slabs;
    p.n_parts = slabs;
    p.grid_x = slabs * p.n_groups;
    p.grid_y = 1;
  } else {
    p.shared = false;
    p.n_groups = 1;
    int wgs = 512 / rt;
    const int max_wgs = (p.n_vtiles + kWaves - 1) / kWaves;
    if (wgs > max_wgs) wgs = max_wgs;
    if (wgs < 1) wgs = 1;
    p.n_slabs = wgs * kWaves;
    p.n_parts = wgs * kWaves;
    p.grid_x = wgs;
    p.grid_y = rt;
  }
  p.ws_bytes = (size_t)5 * (size_t)R * (size_t)p.n_parts * 4u;
  return p;
}

hipError_t launch_draft_step(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  return a.bf16 ? launch_step_w<WBf16>(a, plan, stream) : launch_step_w<WF32>(a, plan, stream);
}

}  // namespace dspark

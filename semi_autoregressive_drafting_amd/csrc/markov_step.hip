// Fused DSpark Markov draft step for gfx950: one kernel per sequential step.
//
// Step k over R requests [P1 "DSpark" §2.2 eq. p_k, §2.3 eq. B, §3.1 eq. c_k,
// §1.1 eq. a_j; the §6.2 vLLM loop fixes the per-position order]:
//
//  1. Confidence head (waves of the first workgroups of each request group, one
//     wave per request): c_k = sigma(w . [h_k; W1[x_{k-1}]]), a_k = a_{k-1} c_k.
//  2. Stream a vocabulary slab: gather E = W1[x_{k-1}] once into VGPRs, form
//     each 32 x 32 bias tile E . W2 with bf16 (or fp32) MFMA, add the base
//     logits U_k and fold the tile into an online max / sum-exp and a Gumbel
//     race, so the R x V bias never reaches HBM.  The race is argmax_v s_v + G_v
//     in its exponential-race form: the winner maximises e_v / L_v with
//     e_v = 2^(t_v - m) (already needed for the sum) and L_v = -log2 u_v, one
//     logarithm per entry.
//  3. Write one partial record per request (slab-major, device-scope atomic
//     writes), then merge in two levels without a second kernel: the last
//     workgroup of a team of slabs to arrive (device-scope counter) merges the
//     team's records; the last team to arrive merges the team records in a
//     fixed order and writes x_k, p_k(x_k) and lse_k.  Nobody waits on anybody:
//     a workgroup that is not last simply exits.  No L2-wide fence is needed
//     because every cross-workgroup value travels through device-scope
//     atomics.  Counters are reset by their last user, so the workspace must
//     be zero-filled once before its first use.
//
// Launch shapes (see mfma_stream.h):
//   shared : R > 96.  A workgroup = 4 waves = 4 request tiles (a group of 128
//            requests); each wave keeps its E fragments in VGPRs for the whole
//            step and each W2t tile is staged once per workgroup in LDS.  W2t
//            leaves HBM once per request group; the groups of one slab share an
//            XCD (blockIdx % 8) so repeated W2t reads hit that XCD's L2.
//   private: R <= 96.  A group = one request tile; the 4 waves of a workgroup
//            stream interleaved tiles of the slab with W2t fragments loaded
//            straight into VGPRs, then merge their records in LDS.
#include "dspark_kernels.h"
#include "mfma_stream.h"

namespace dspark {

namespace {

constexpr int kWaves = 4;
constexpr int kTeamSize = 32;  // slabs merged by one team closer
constexpr int kMaxTeams = 16;  // teams per request group (n_slabs <= 512)

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
  float ubuf[2][16];  // U of the current and the prefetched tile (alternating)
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
  template <int S>
  __device__ void prefetch(int vt) {
    load16<kVec>(ubuf[S], urow, vt * kVTile + 16 * half, V, (vt + 1) * kVTile <= V);
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

  template <int S>
  __device__ void consume(const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * half;
    float z[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = ubuf[S][i] + acc[i];
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

// Records live in slab-major planes: rec[(slot * 5 + field) * R + r], so the
// 32 or 128 requests a workgroup writes for one slot are contiguous.
//
// Records cross workgroups (and XCDs) inside one launch, so they are written
// and read with device-scope atomics, which the hardware keeps coherent
// without writing back or invalidating whole L2 caches.  Each write is an
// exchange whose returned old value the caller folds into `chk`: using `chk`
// before the workgroup barrier makes every write complete at the coherence
// point before the arrival counter is incremented.
__device__ __forceinline__ unsigned xchg(float* p, float v) {
  return __float_as_uint(
      __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ unsigned put_rec(float* base, int R, int slot, int r, const Rec& q) {
  float* p = base + (size_t)slot * 5 * R + r;
  unsigned chk = xchg(p, q.m);
  chk ^= xchg(p + R, q.S);
  chk ^= xchg(p + 2 * R, q.key);
  chk ^= xchg(p + 3 * R, q.tbest);
  chk ^= xchg(p + 4 * R, __int_as_float(q.idx));
  return chk;
}

__device__ __forceinline__ float ld(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ Rec get_rec(const float* base, int R, int slot, int r) {
  const float* p = base + (size_t)slot * 5 * R + r;
  return Rec{ld(p), ld(p + R), ld(p + 2 * R), ld(p + 3 * R), __float_as_int(ld(p + 4 * R))};
}

__device__ __forceinline__ Rec empty_rec() { return Rec{-INFINITY, 0.0f, -INFINITY, -INFINITY, -1}; }

// Fixed-order merge of records [j0, j1) of request r by kTpr consecutive
// threads (a power of two <= 64, inside one wave): each thread loads its
// contiguous chunk of at most kChunk records at once (one memory round trip),
// folds it in order, then a butterfly over the kTpr lanes.
template <int kTpr, int kChunk>
__device__ __forceinline__ Rec merge_range(const float* base, int R, int r, int j0, int j1,
                                           int sub) {
  const int n = j1 - j0;
  const int chunk = (n + kTpr - 1) / kTpr;  // <= kChunk by construction of the plan
  const int b = j0 + sub * chunk;
  const int e = min(j1, b + chunk);
  Rec buf[kChunk];
#pragma unroll
  for (int i = 0; i < kChunk; ++i)
    if (b + i < e) buf[i] = get_rec(base, R, b + i, r);
  Rec acc = empty_rec();
#pragma unroll
  for (int i = 0; i < kChunk; ++i)
    if (b + i < e) acc = rec_merge(acc, buf[i]);
#pragma unroll
  for (int m = 1; m < kTpr; m <<= 1) {
    const Rec o = rec_shfl_xor(acc, m);
    acc = (sub & m) ? rec_merge(o, acc) : rec_merge(acc, o);
  }
  return acc;
}

// Final outputs of request r from its merged record.
__device__ __forceinline__ void write_outputs(const StepArgs& a, int r, const Rec& f) {
  const size_t o = (size_t)r * a.gamma + (a.k - 1);
  a.x[(size_t)r * (a.gamma + 1) + a.k] = f.idx;
  if (a.greedy) {
    a.p[o] = 1.0f;
    a.lse[o] = f.m;
  } else {
    const float lse2 = f.m + log2f(f.S);
    a.p[o] = exp2f(f.tbest - lse2);
    a.lse[o] = lse2 * kLn2;
  }
}

// Confidence head for request r, computed by one whole wave.
template <class W>
__device__ __forceinline__ void confidence_wave(const StepArgs& a, int r, int lane) {
  using store_t = typename W::store_t;
  const size_t o = (size_t)r * a.gamma + (a.k - 1);
  const int xp = clamp_token(a.x[(size_t)r * (a.gamma + 1) + (a.k - 1)], a.V);
  const store_t* hrow = reinterpret_cast<const store_t*>(a.h) + o * a.d;
  const store_t* erow = reinterpret_cast<const store_t*>(a.W1) + (size_t)xp * a.rank;
  const float dot = conf_dot_wave<W>(hrow, erow, a.w, a.d, a.rank, lane);
  if (lane == 0) {
    const float c = sigmoid_f32(dot);
    const float prev = (a.k == 1) ? 1.0f : a.a[o - 1];
    a.c[o] = c;
    a.a[o] = __fmul_rn(prev, c);
  }
}

// Arrival at a device-scope counter; returns true in every thread of the last
// workgroup to arrive.  `chk` (the folded exchange results of this thread's
// record writes) is consumed before the barrier, so all writes of the
// workgroup are complete before thread 0 increments the counter.  The last
// arriver resets the counter for the next call.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected, unsigned chk,
                                            int* sflag) {
  if (chk == 0x7FC00001u) *sflag = 2;  // never true in practice; forces the wait on chk
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old + 1u == expected;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sflag = last ? 1 : 0;
  }
  __syncthreads();
  return *sflag == 1;
}

// Level-1 records of this workgroup are at slot `slab`; the group covers
// requests [r0, r0 + nr) (nr <= kNr).
template <int kNr>
__device__ __forceinline__ void merge_levels(const StepArgs& a, int grp, int slab, int r0, int nr,
                                             unsigned chk) {
  __shared__ int sflag;
  const int team = slab / a.team_size;
  const int t0 = team * a.team_size;
  const int t1 = min(a.n_slabs, t0 + a.team_size);
  unsigned* cnt = a.counters + (size_t)grp * (a.n_teams + 1);
  if (!arrive_last(cnt + team, (unsigned)(t1 - t0), chk, &sflag)) return;

  constexpr int kTpr = kStreamThreads / kNr;  // threads per request
  constexpr int kChunk = (kTeamSize + kTpr - 1) / kTpr;
  const int rl = threadIdx.x / kTpr, sub = threadIdx.x % kTpr;
  const int r = r0 + rl;
  const int rr = (rl < nr) ? r : r0;  // idle threads shadow request r0, never stored
  Rec q = merge_range<kTpr, kChunk>(a.part, a.R, rr, t0, t1, sub);
  chk = 0u;
  if (sub == 0 && rl < nr) chk = put_rec(a.part2, a.R, team, r, q);

  if (!arrive_last(cnt + a.n_teams, (unsigned)a.n_teams, chk, &sflag)) return;
  q = merge_range<kTpr, (kMaxTeams + kTpr - 1) / kTpr>(a.part2, a.R, rr, 0, a.n_teams, sub);
  if (sub == 0 && rl < nr) write_outputs(a, r, q);
}

template <class W, int kKs, bool kGreedy, bool kDebug, bool kVec>
__global__ __launch_bounds__(kStreamThreads) void markov_step_shared(StepArgs a) {
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
  const int r0 = grp * kWaves * kVTile;
  if (a.h != nullptr && slab < kVTile) {  // 32 workgroups x 4 waves cover the group
    const int rq = r0 + slab * kWaves + wave;
    if (rq < a.R) confidence_wave<W>(a, rq, lane);
  }
  int t_begin, t_end;
  slab_range(slab, a.n_slabs, a.n_vtiles, t_begin, t_end);

  const int r = r0 + wave * kVTile + col;
  const int rc = r < a.R ? r : a.R - 1;  // padded lanes recompute row R-1, never stored
  typename W::frag_t e[W::kMaxKs];
  load_e_frags<W, kKs>(e, a.W1, a.x[(size_t)rc * (a.gamma + 1) + (a.k - 1)], a.rank, a.V, half);

  DraftEpi<kGreedy, kDebug, kVec> epi(a, r, rc, half);
  shared_a_stream<W, kKs>(a.W2t, a.V, a.rank, t_begin, t_end, e, lds, epi);

  Rec q = epi.record();
  q = rec_merge(q, rec_shfl_xor(q, 32));
  unsigned chk = 0u;
  if (half == 0 && r < a.R) chk = put_rec(a.part, a.R, slab, r, q);
  merge_levels<kWaves * kVTile>(a, grp, slab, r0, min(kWaves * kVTile, a.R - r0), chk);
}

template <class W, int kKs, bool kGreedy, bool kDebug, bool kVec>
__global__ __launch_bounds__(kStreamThreads) void markov_step_private(StepArgs a) {
  __shared__ Rec srec[kWaves][kVTile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int slab = blockIdx.x % a.n_slabs;
  const int grp = blockIdx.x / a.n_slabs;  // request tile
  const int r0 = grp * kVTile;
  if (a.h != nullptr && slab < kVTile / kWaves) {  // 8 workgroups x 4 waves
    const int rq = r0 + slab * kWaves + wave;
    if (rq < a.R) confidence_wave<W>(a, rq, lane);
  }
  int t_begin, t_end;
  slab_range(slab, a.n_slabs, a.n_vtiles, t_begin, t_end);

  const int r = r0 + col;
  const int rc = r < a.R ? r : a.R - 1;
  typename W::frag_t e[W::kMaxKs];
  load_e_frags<W, kKs>(e, a.W1, a.x[(size_t)rc * (a.gamma + 1) + (a.k - 1)], a.rank, a.V, half);

  DraftEpi<kGreedy, kDebug, kVec> epi(a, r, rc, half);
  private_a_stream<W, kKs>(a.W2t, a.V, a.rank, t_begin + wave, t_end, kWaves, e, epi);

  Rec q = epi.record();
  q = rec_merge(q, rec_shfl_xor(q, 32));
  if (half == 0) srec[wave][col] = q;
  __syncthreads();
  unsigned chk = 0u;
  if (wave == 0 && half == 0) {
    Rec m = srec[0][col];
    for (int w = 1; w < kWaves; ++w) m = rec_merge(m, srec[w][col]);
    if (r < a.R) chk = put_rec(a.part, a.R, slab, r, m);
  }
  merge_levels<kVTile>(a, grp, slab, r0, min(kVTile, a.R - r0), chk);
}

template <class W, int kKs, bool kGreedy, bool kDebug, bool kVec>
void launch_one(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  if (plan.shared)
    hipLaunchKernelGGL((markov_step_shared<W, kKs, kGreedy, kDebug, kVec>), dim3(plan.grid_x),
                       dim3(kStreamThreads), stream_lds_bytes<W>(a.rank), stream, a);
  else
    hipLaunchKernelGGL((markov_step_private<W, kKs, kGreedy, kDebug, kVec>), dim3(plan.grid_x),
                       dim3(kStreamThreads), 0, stream, a);
}

template <class W, int kKs, bool kGreedy>
void launch_g(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  const bool vec = (a.V % 4) == 0;
  if (a.z_debug != nullptr) {
    if (vec) launch_one<W, kKs, kGreedy, true, true>(a, plan, stream);
    else launch_one<W, kKs, kGreedy, true, false>(a, plan, stream);
  } else {
    if (vec) launch_one<W, kKs, kGreedy, false, true>(a, plan, stream);
    else launch_one<W, kKs, kGreedy, false, false>(a, plan, stream);
  }
}

template <class W, int kKs>
hipError_t launch_k(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  if (a.greedy) launch_g<W, kKs, true>(a, plan, stream);
  else launch_g<W, kKs, false>(a, plan, stream);
  return hipGetLastError();
}

// The Qwen3-family rank (256 bf16 = 16 MFMA K-steps) gets a branch-free MFMA loop.
template <class W>
hipError_t launch_w(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  if (W::kKStep * W::kMaxKs == a.rank) return launch_k<W, W::kMaxKs>(a, plan, stream);
  return launch_k<W, 0>(a, plan, stream);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

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
    int slabs = kResidentWgs / p.n_groups;
    if (p.n_groups > 1) slabs = (slabs / 8) * 8;
    if (slabs < kVTile) slabs = kVTile;  // the confidence head uses 32 slabs per group
    p.n_slabs = slabs;
  } else {
    p.shared = false;
    p.n_groups = rt;
    int slabs = kResidentWgs / rt;
    const int max_slabs = (p.n_vtiles + kWaves - 1) / kWaves;
    if (slabs > max_slabs) slabs = max_slabs;
    if (slabs < kVTile / kWaves) slabs = kVTile / kWaves;  // 8 slabs carry the confidence head
    p.n_slabs = slabs;
  }
  p.grid_x = p.n_slabs * p.n_groups;
  p.grid_y = 1;
  p.team_size = kTeamSize;
  p.n_teams = (p.n_slabs + p.team_size - 1) / p.team_size;  // <= kMaxTeams
  p.off_part2 = align256((size_t)p.n_slabs * 5 * R * 4);
  p.off_counters = p.off_part2 + align256((size_t)p.n_teams * 5 * R * 4);
  p.ws_bytes = p.off_counters + align256((size_t)p.n_groups * (p.n_teams + 1) * 4);
  return p;
}

hipError_t launch_draft_step(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  return a.bf16 ? launch_w<WBf16>(a, plan, stream) : launch_w<WF32>(a, plan, stream);
}

}  // namespace dspark

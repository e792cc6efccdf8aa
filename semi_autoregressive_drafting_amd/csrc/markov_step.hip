// DSpark Markov draft step for gfx950: a streaming kernel per sequential step
// and one finalisation kernel per call.
//
// Step k over R requests [P1 "DSpark" §2.2 eq. p_k, §2.3 eq. B; the §6.2 vLLM
// loop fixes the per-position order]:
//
//  markov_step_*   Each workgroup streams one vocabulary slab: it gathers
//     E = W1[x_{k-1}] into VGPRs, forms each 32 x 32 bias tile E . W2 with bf16
//     (or fp32) MFMA, adds the base logits U_k and folds the tile into an
//     online max / sum-exp and a Gumbel race, so the R x V bias never reaches
//     HBM.  Sampling is the Gumbel-max trick at two levels over aligned blocks
//     of 16 ids (each lane's 16 entries of a tile are exactly one block): the
//     stream races blocks, maximising M_b / L_b with M_b = sum_{v in b}
//     2^(t_v - m) (the block's share of the softmax sum) and L_b = -log2 u_b
//     (one uniform and one logarithm per block), and keeps the 16 logits of
//     the lane's leading block in registers.  After the stream each lane draws
//     an id inside its leading block by the same race over the block's ids
//     (e_v / L_v, a second noise stream).  The workgroup then stores one
//     partial record per request (m, S, block key, t of the drawn id, id) with
//     plain stores and publishes its winner with one 64-bit atomic max of
//     (order-preserving block key, ~id): the maximum is independent of the
//     order in which workgroups arrive and keeps the lowest block (hence the
//     lowest id) on equal keys.  The next step reads x_k from that word, so
//     nothing waits for a merge.
//
//     The first slabs (the ones with the lighter share of tiles) also run the
//     confidence head for one request each after their stream:
//     c_k = sigma(w . [h_k; W1[x_{k-1}]]) [P1 §3.1 eq. c_k] and the survival
//     product a_k = a_{k-1} c_k [P1 §1.1 eq. a_j] (a_{k-1} comes from the
//     previous launch).
//
//  draft_merge  One workgroup per (32 requests, position) merges the records
//     of the step in a fixed tree order (so the result is bit-reproducible):
//     x_k, p_k(x_k) = 2^(t_best - lse), lse_k.  It clears the atomic words it
//     consumed, so the workspace stays zero between calls.
//
// Launch shape of the streaming kernel (see mfma_stream.h): a workgroup = 4
// waves = 4 request tiles (a group of 128 requests); each wave keeps its E
// fragments in VGPRs for the whole step and each W2t tile is staged once per
// workgroup in LDS.  W2t leaves HBM once per request group; the groups of one
// slab share an XCD (blockIdx % 8) so repeated W2t reads hit that XCD's L2.
// Odd steps walk each slab's tiles upward and even steps downward, so a step
// starts on the W2t tiles the previous step read last.  The L2 does not keep
// them across the launch (the L2 misses per step stay the same); the most
// recently read tiles are the likeliest to be served by the memory-side cache
// (MALL) rather than by DRAM, and the step is faster this way.  The races
// break ties by id, so the visiting order changes no tie.
// Batches below 128 requests run the same shape with the missing rows padded
// (their lanes recompute row R-1 and store nothing): the bytes, not the
// arithmetic, set the step's time, and a shape whose waves stream separate
// tiles with W2t loaded straight into VGPRs measured slower at every batch
// size from 1 to 96 requests.
#include "draft_step.h"
#include "mfma_stream.h"

namespace dspark {

namespace {

constexpr int kWaves = 4;
// Workgroups of a draft step (in total over the request groups): two per CU.
// Two independent 4-wave pipelines per CU hide memory latency better than one
// 8-wave workgroup whose waves meet at every barrier.
constexpr int kDraftWgs = 512;

// Prefetch distance of the shared stream: 2 for bf16 weights; fp32 weights
// (E fragments twice as large) keep 1 to stay within the register budget.
template <class W>
constexpr int draft_dist() {
  return std::is_same<W, WBf16>::value ? 2 : 1;
}

// LDS bytes of the shared draft stream (the skewed stream keeps two W2t slots).
template <class W, int kKs>
__host__ __device__ inline size_t draft_stream_lds(int rank) {
  return stream_lds_bytes<W>(rank, kKs > 0 ? 1 : draft_dist<W>());
}

// Order-preserving map of a float to uint32 (larger float -> larger code).
__device__ __forceinline__ uint32_t ordered(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit word of a race winner: larger key first, then lower id.  0 = none.
__device__ __forceinline__ unsigned long long pack_winner(float key, int idx) {
  return idx < 0 ? 0ull
                 : ((unsigned long long)ordered(key) << 32) |
                       (unsigned long long)(~(uint32_t)idx);
}

// Per-lane online state over the lane's vocabulary entries of one request.
struct LaneState {
  float m;    // running max of t = z * kscale
  float S;    // sum of 2^(t - m)
  float bE;   // leading block's mass sum 2^(t - m) (rescaled with m); greedy: best z
  float bLn;  // leading block's log2(u) < 0
  int bV;     // leading block's first id (greedy: best id), -1 if none
};

// U rows of the wave's 32 requests: with kVec (16-byte aligned rows) read as
// whole lines and passed through the wave's LDS patch (RowTiles); otherwise
// each lane loads its own row's 16 entries.
template <bool kGreedy, bool kDebug, bool kVec>
struct DraftEpi {
  const float* urow;
  float* zdbg;
  float* patch;  // this wave's LDS patch (kVec)
  int V, R, r, half;
  float kscale;
  uint32_t state_row;  // LCG state of block 0 of this row (block stream)
  uint32_t state_ent;  // LCG state of id 0 of this row (id stream)
  float zb[kGreedy ? 1 : 16];                    // logits of the leading block
  float ubuf[kVec ? 1 : kMaxDist + 1][16];       // own-row U (scalar path)
  RowTiles<1, kVec ? kMaxDist + 1 : 1> rows;     // line-coalesced U (kVec)
  LaneState st;
  static constexpr int kLoads = kVec ? 4 : 16;

  // r0w: first request of the wave's 32-row tile.
  __device__ DraftEpi(const StepArgs& a, int k, int r_, int rc, int half_, int r0w, float* patch_)
      : zdbg(a.z_debug), patch(patch_), V(a.V), R(a.R), r(r_), half(half_), kscale(a.kscale) {
    if constexpr (kVec) {
      const int jmax = a.R - 1 - r0w;
      const size_t rstride = (size_t)a.gamma * a.V;
      rows.init([&](int j) { return (size_t)(r0w + (j < jmax ? j : jmax)) * rstride; });
    }
    next_step(a, k, rc);
  }
  // Point at step k (logit rows, noise streams) and reset the lane state.
  __device__ __forceinline__ void next_step(const StepArgs& a, int k, int rc) {
    urow = a.U + ((size_t)rc * a.gamma + (k - 1)) * a.V;
    if constexpr (kVec) rows.base[0] = a.U + (size_t)(k - 1) * a.V;
    state_row = row_key(a.seed, kStreamDraft, (uint32_t)rc, (uint32_t)k) * kLcgMul + kLcgInc;
    state_ent = kGreedy ? 0u
                        : row_key(a.seed, kStreamDraftEntry, (uint32_t)rc, (uint32_t)k) * kLcgMul +
                              kLcgInc;
#pragma unroll
    for (int i = 0; i < (kGreedy ? 1 : 16); ++i) zb[i] = 0.0f;
    st.m = -INFINITY;
    st.S = 0.0f;
    st.bE = kGreedy ? -INFINITY : 0.0f;
    st.bLn = -1.0f;
    st.bV = -1;
  }
  template <int S>
  __device__ void prefetch(int vt) {
    if constexpr (kVec)
      rows.template load<S>(vt);
    else
      load16<false>(ubuf[S], urow, (vt < 0 ? 0 : vt * kVTile) + 16 * half);
  }

  template <bool kMasked>
  __device__ __forceinline__ void fold(const float (&z)[16], int vb) {
    if constexpr (kGreedy) {
      // the tile's best (ids rise inside it, so strict > keeps the lowest id
      // among equal logits), then merged into the running best with the same
      // rule whatever order the tiles come in
      float zt = -INFINITY;
      int it = -1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool w = (!kMasked || vb + i < V) && z[i] > zt;
        zt = w ? z[i] : zt;
        it = w ? vb + i : it;
      }
      const bool win = it >= 0 && (zt > st.bE || (zt == st.bE && it < st.bV));
      st.bE = win ? zt : st.bE;
      st.bV = win ? it : st.bV;
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
      // the block's mass (vb is a multiple of 16: the lane's entries are one block)
      float sb = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float e = fast_exp2(fmaf(z[i], kscale, negm));
        if constexpr (kMasked) e = (vb + i < V) ? e : 0.0f;
        sb += e;
      }
      st.S += sb;
      const float ln = fast_log2(
          bits_to_uniform(rxs_m_xs(state_row + (uint32_t)(vb / kDraftBlock) * kLcgMul)));
      // sb / L > bE / bL  <=>  sb * bLn < bE * ln     (L = -ln > 0); on equal
      // keys the lower block, whatever order the tiles come in
      const float lhs = sb * st.bLn, rhs = st.bE * ln;
      const bool win = lhs < rhs || (lhs == rhs && st.bV >= 0 && vb < st.bV);
      st.bE = win ? sb : st.bE;
      st.bLn = win ? ln : st.bLn;
      st.bV = win ? vb : st.bV;
#pragma unroll
      for (int i = 0; i < 16; ++i) zb[i] = win ? z[i] : zb[i];
    }
  }

  template <bool kMasked>
  __device__ __forceinline__ void fold_tile(const float (&u)[16], const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * half;
    float z[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = u[i] + acc[i];
    if constexpr (kDebug) {
      if (r < R) {
        for (int i = 0; i < 16; ++i)
          if (vb + i < V) zdbg[(size_t)r * V + vb + i] = z[i];
      }
    }
    fold<kMasked>(z, vb);
  }

  template <int S>
  __device__ void consume(const f32x16_t& acc, int vt) {
    if constexpr (kVec) {
      float u[1][16];
      rows.template to_lanes<S>(patch, u);
      fold_tile<false>(u[0], acc, vt);
    } else {
      fold_tile<false>(ubuf[S], acc, vt);
    }
  }

  __device__ void tail(const f32x16_t& acc, int vt) {
    float u[16];
    load16_masked(u, urow, vt * kVTile + 16 * half, V, 0.0f);
    fold_tile<true>(u, acc, vt);
  }

  // The record of the lane's request over both halves of the wave (lanes l and
  // l ^ 32 hold the same request, different ids): the softmax statistics merged,
  // the leading block of the two (larger block key; the lower block on equal
  // keys), and the id drawn inside that block by the race e_v / L_v with
  // e_v = 2^(t_v - t_max) and L_v = -log2 u_v from the id stream, the two lanes
  // taking 8 ids each.  Both lanes return the same record.
  __device__ Rec row_record() const {
    Rec q;
    if constexpr (kGreedy) {
      q.m = st.bE;
      q.S = 0.0f;
      q.key = st.bE;
      q.tbest = st.bE;
      q.idx = st.bV;
      return rec_merge(q, rec_shfl_xor(q, 32));
    } else {
      const bool has = st.bV >= 0 && st.bE > 0.0f;
      const float key = has ? st.m + fast_log2(st.bE) - fast_log2(-st.bLn) : -INFINITY;
      const int vb = has ? st.bV : -1;
      const float okey = __shfl_xor(key, 32);
      const int ovb = __shfl_xor(vb, 32);
      const bool take_o = rec_beats(okey, ovb, key, vb);
      const int wvb = take_o ? ovb : vb;
      q.key = take_o ? okey : key;
      // softmax statistics (the same bits in both lanes: IEEE addition commutes)
      const float om = __shfl_xor(st.m, 32), oS = __shfl_xor(st.S, 32);
      q.m = fmaxf(st.m, om);
      q.S = (q.m == -INFINITY) ? 0.0f
                               : st.S * fast_exp2(st.m - q.m) + oS * fast_exp2(om - q.m);
      // the leading block's logits in both lanes
      float zw[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float oz = __shfl_xor(zb[i], 32);
        zw[i] = take_o ? oz : zb[i];
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = (wvb + i < V) ? fmaxf(tmax, zw[i] * kscale) : tmax;
      // this lane's 8 ids: wvb + 8 half + j
      const int i0 = wvb + 8 * half;
      const uint32_t s0 = state_ent + (uint32_t)i0 * kLcgMul;
      float eE = 0.0f, eLn = -1.0f, tsel = -INFINITY;
      int isel = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = (half ? zw[8 + j] : zw[j]) * kscale;
        float e = fast_exp2(t - tmax);
        e = (i0 + j < V) ? e : 0.0f;
        const float ln = fast_log2(bits_to_uniform(rxs_m_xs(s0 + (uint32_t)j * kLcgMul)));
        const bool win = e * eLn < eE * ln;
        eE = win ? e : eE;
        eLn = win ? ln : eLn;
        tsel = win ? t : tsel;
        isel = win ? j : isel;
      }
      // the two halves' winners: the upper ids (half 1) win only on a strictly
      // larger ratio
      const float oE = __shfl_xor(eE, 32), oLn = __shfl_xor(eLn, 32), ot = __shfl_xor(tsel, 32);
      const int oi = __shfl_xor(isel, 32);
      const float aE = half ? oE : eE, aLn = half ? oLn : eLn, bE2 = half ? eE : oE,
                  bLn2 = half ? eLn : oLn;
      const bool hi = bE2 * aLn < aE * bLn2;
      const float t_lo = half ? ot : tsel, t_hi = half ? tsel : ot;
      const int i_lo = half ? oi : isel, i_hi = half ? isel : oi;
      q.tbest = hi ? t_hi : t_lo;
      q.idx = wvb < 0 ? -1 : wvb + (hi ? 8 + i_hi : i_lo);
      if (wvb < 0) {
        q.key = -INFINITY;
        q.tbest = -INFINITY;
      }
      return q;
    }
  }
};

// Token x_{k-1} of request rc: the anchor column, the column written by the
// previous call's finalisation, or (inside a block) the previous step's
// winner word.
__device__ __forceinline__ int prev_token(const StepArgs& a, int k, bool pfb, int rc) {
  if (k > 1 && pfb) return winner_id(a.best[winner_index(k - 2, a.R, rc)]);
  return a.x[(size_t)rc * (a.gamma + 1) + (k - 1)];
}

// Tokens x_{k-1} of a wave's 32 requests r0w .. r0w + 31 (past R - 1: request
// R - 1).  The words are read through the scalar cache with wave-uniform
// addresses: scalar loads are counted apart from the vector loads, so the
// tokens arrive without waiting behind the first tiles' vector loads (vector
// loads retire in issue order); only the row gather queues behind those.
// issue() starts the 32 loads, token() waits for them and gives lane l the
// token of request r0w + l % 32.
struct WaveTokens {
  typedef const __attribute__((address_space(4))) uint32_t* cptr;
  uint32_t t[32];
  bool from_best;
  __device__ __forceinline__ void issue(const StepArgs& a, int k, bool pfb, int r0w) {
    r0w = __builtin_amdgcn_readfirstlane(r0w);
    // word j of the wave sits at base + j * stride (32-bit words)
    from_best = k > 1 && pfb;
    cptr base;
    size_t stride;
    if (from_best) {  // the low word of each winner word holds ~id
      base = (cptr)(uintptr_t)a.best + 2 * winner_index(k - 2, a.R, r0w);
      stride = 2 * kWinnerStride;
    } else {
      base = (cptr)(uintptr_t)a.x + (size_t)r0w * (a.gamma + 1) + (k - 1);
      stride = (size_t)(a.gamma + 1);
    }
    const int last = __builtin_amdgcn_readfirstlane(min(31, a.R - 1 - r0w));
#pragma unroll
    for (int j = 0; j < 32; ++j) t[j] = base[(size_t)(j < last ? j : last) * stride];
  }
  __device__ __forceinline__ int token() const {
    const int col = threadIdx.x & 31;
    int tok = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) tok = (col == j) ? (int)t[j] : tok;
    return from_best ? ~tok : tok;
  }
};

// Records of step k live in slab-major planes: rec[(slab * 5 + field) * R + r].
__device__ __forceinline__ void put_rec(float* base, int R, int slab, int r, const Rec& q) {
  float* p = base + (size_t)slab * 5 * R + r;
  p[0] = q.m;
  p[R] = q.S;
  p[2 * R] = q.key;
  p[3 * R] = q.tbest;
  p[4 * R] = __int_as_float(q.idx);
}

__device__ __forceinline__ void publish(const StepArgs& a, int k, int slab, int r, const Rec& q) {
  put_rec(a.rec + (size_t)(k - 1) * a.rec_step_f, a.R, slab, r, q);
  if (q.idx >= 0) atomicMax(a.best + winner_index(k - 1, a.R, r), pack_winner(q.key, q.idx));
}

// Confidence head and survival product of step k for requests r0 + slab,
// r0 + slab + n_slabs, ... < r0 + nr.  Called by the whole workgroup.
template <class W>
__device__ __forceinline__ void step_confidence(const StepArgs& a, int k, bool pfb, int slab,
                                                int r0, int nr) {
  using store_t = typename W::store_t;
  __shared__ float red[4];
  for (int q = slab; q < nr; q += a.n_slabs) {
    const int r = r0 + q;
    const size_t o = (size_t)r * a.gamma + (k - 1);
    const int xp = checked_token(prev_token(a, k, pfb, r), a.V, a.err);
    const store_t* hrow = reinterpret_cast<const store_t*>(a.h) + o * a.d;
    const store_t* erow = reinterpret_cast<const store_t*>(a.W1) + (size_t)xp * a.rank;
    const float c = sigmoid_f32(conf_dot_wg<W>(hrow, erow, a.w, a.d, a.rank, red));
    if (threadIdx.x == 0) {
      const float prev = (k == 1) ? 1.0f : a.a[o - 1];
      a.c[o] = c;
      a.a[o] = __fmul_rn(prev, c);
    }
  }
}

// The end of a draft step in the shared launch: the confidence head's row loads
// (preloaded form), the request's record and winner word, then the confidence
// head and survival product of request r0 + slab.  conf_tok holds its token.
template <class W, class Epi>
__device__ __forceinline__ void finish_step(const StepArgs& a, int k, bool pfb, Epi& epi, int slab,
                                            int r0, int nr, int r, bool conf_pre,
                                            const int& conf_tok, float* conf_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int conf_n = a.d + a.rank;
  ConfPreload cp;
  float a_prev = 1.0f;
  size_t co = 0;
  if (conf_pre) {
    lds_barrier();  // conf_tok, written during the gather
    co = (size_t)(r0 + slab) * a.gamma + (k - 1);
    const int n4 = ((conf_n + 3) / 4 + 7) / 8 * 8;
    const int j0 = min(conf_n, wave * n4), j1 = min(conf_n, j0 + n4);
    cp.load(reinterpret_cast<const uint16_t*>(a.h) + co * a.d,
            reinterpret_cast<const uint16_t*>(a.W1) + (size_t)conf_tok * a.rank, a.w, a.d, j0,
            j1, lane);
    if (k > 1) a_prev = a.a[co - 1];
  }
  const Rec q = epi.row_record();
  if (half == 0 && r < a.R) publish(a, k, slab, r, q);
  if (conf_pre) {
    const float part = cp.dot();
    if (lane == 0) conf_red[wave] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float c = sigmoid_f32(((conf_red[0] + conf_red[1]) + conf_red[2]) + conf_red[3]);
      a.c[co] = c;
      a.a[co] = __fmul_rn(a_prev, c);
    }
  } else if (a.h != nullptr) {
    step_confidence<W>(a, k, pfb, slab, r0, nr);
  }
}

// Whether the preloaded confidence head applies to request r0 + slab.
template <class W>
__device__ __forceinline__ bool conf_preloadable(const StepArgs& a, int slab, int nr) {
  return std::is_same<W, WBf16>::value && a.h != nullptr && !a.E_rows && slab < nr &&
         a.d % 8 == 0 && a.d + a.rank <= 4 * 64 * 8 * kConfChunks &&
         ((reinterpret_cast<uintptr_t>(a.h) | reinterpret_cast<uintptr_t>(a.W1) |
           reinterpret_cast<uintptr_t>(a.w)) & 15u) == 0;
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
  int t_begin, t_end;
  slab_range(slab, a.n_slabs, a.n_vtiles, t_begin, t_end);

  const int r = r0 + wave * kVTile + col;
  const int rc = r < a.R ? r : a.R - 1;  // padded lanes recompute row R-1, never stored
  typename W::frag_t e[W::kMaxKs];
  float* patch = reinterpret_cast<float*>(lds + draft_stream_lds<W, kKs>(a.rank)) +
                 wave * kPatchFloats;
  DraftEpi<kGreedy, kDebug, kVec> epi(a, a.k, r, rc, half, r0 + wave * kVTile, patch);
  WaveTokens toks;
  if (!a.E_rows) toks.issue(a, a.k, a.prev_from_best, r0 + wave * kVTile);
  // The confidence head of request r0 + slab (one per workgroup at most: there
  // are never fewer slabs than requests in a group).  With bf16 rows that fit
  // the preloaded form, its token is kept in LDS from the gather and its row
  // loads are issued right after the stream, under the id draw and the publish.
  const int nr = min(kWaves * kVTile, a.R - r0);
  __shared__ int conf_tok;
  __shared__ float conf_red[4];
  const bool conf_pre = conf_preloadable<W>(a, slab, nr);
  auto gather = [&](typename W::frag_t(&ef)[W::kMaxKs]) {
    const void* base = a.E_rows ? a.E_rows : a.W1;
    const int row = a.E_rows ? rc : checked_token(toks.token(), a.V, a.err);
    if (conf_pre && wave == (slab >> 5) && lane == (slab & 31)) conf_tok = row;
    if constexpr (std::is_same<W, WBf16>::value && kKs > 0 && kKs % 4 == 0 && kVec)
      load_e_frags_lines<kKs>(ef, reinterpret_cast<const uint16_t*>(base), row, patch);
    else
      load_e_frags<W, kKs>(ef, base, row, a.rank, a.E_rows ? a.R : a.V, half);
  };
  if constexpr (kKs > 0)
    shared_a_stream_skew<W, kKs>(a.W2t, a.V, t_begin, t_end, e, gather, lds, epi,
                                 (a.k & 1) == 0);
  else
    shared_a_stream<W, kKs, draft_dist<W>()>(a.W2t, a.V, a.rank, t_begin, t_end, e, gather, lds,
                                             epi);

  finish_step<W>(a, a.k, a.prev_from_best, epi, slab, r0, nr, r, conf_pre, conf_tok, conf_red);
}

// ---------------------------------------------------------------------------
// Merge of the records of step k = k0 + blockIdx.y for requests
// r0 = 32 * blockIdx.x .. r0 + 31.  Wave w takes slabs [w * spw, (w+1) * spw);
// lane (h, rl) = (lane / 32, lane % 32) folds slabs w * spw + h, + 2, + 4, ...
// of request r0 + rl in order (each load instruction reads 32 consecutive
// requests of two slabs), the two halves merge (h = 0 first), then thread rl
// merges the 16 wave results in wave order.
// ---------------------------------------------------------------------------
constexpr int kMergeWaves = 16;
constexpr int kMergeRounds = kResidentWgs / kMergeWaves / 2;  // load rounds per lane

struct MergeAcc {
  float m, S, tb;
  unsigned long long wb;  // largest winner word seen
};

__device__ __forceinline__ MergeAcc macc_merge(const MergeAcc& x, const MergeAcc& y) {
  MergeAcc o;
  o.m = fmaxf(x.m, y.m);
  o.S = (o.m == -INFINITY) ? 0.0f : x.S * fast_exp2(x.m - o.m) + y.S * fast_exp2(y.m - o.m);
  const bool ty = y.wb > x.wb;
  o.wb = ty ? y.wb : x.wb;
  o.tb = ty ? y.tb : x.tb;
  return o;
}

__global__ __launch_bounds__(64 * kMergeWaves) void draft_merge(StepArgs a, int k0) {
  __shared__ MergeAcc sacc[kMergeWaves][kVTile];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, rl = lane & 31;
  const int k = k0 + blockIdx.y;
  const int r = blockIdx.x * kVTile + rl;
  const int rc = r < a.R ? r : a.R - 1;
  const float* base = a.rec + (size_t)(k - 1) * a.rec_step_f + rc;
  const int spw = (a.n_slabs + kMergeWaves - 1) / kMergeWaves;
  const int s0 = wave * spw, s1 = min(a.n_slabs, s0 + spw);

  MergeAcc acc{-INFINITY, 0.0f, -INFINITY, 0ull};
  for (int c0 = s0; c0 < s1; c0 += 2 * kMergeRounds) {  // chunks of 2 * kMergeRounds slabs
    float rm[kMergeRounds], rS[kMergeRounds], rkey[kMergeRounds], rt[kMergeRounds];
    int rid[kMergeRounds];
#pragma unroll
    for (int i = 0; i < kMergeRounds; ++i) {
      const int sl = c0 + 2 * i + h;
      const bool ok = sl < s1;
      const float* p = base + (size_t)(ok ? sl : 0) * 5 * a.R;
      rm[i] = ok ? p[0] : -INFINITY;
      rS[i] = ok ? p[a.R] : 0.0f;
      rkey[i] = ok ? p[2 * a.R] : -INFINITY;
      rt[i] = ok ? p[3 * a.R] : -INFINITY;
      rid[i] = ok ? __float_as_int(p[4 * a.R]) : -1;
    }
#pragma unroll
    for (int i = 0; i < kMergeRounds; ++i)
      acc = macc_merge(acc, MergeAcc{rm[i], rS[i], rt[i], pack_winner(rkey[i], rid[i])});
  }
  MergeAcc o;
  o.m = __shfl_xor(acc.m, 32);
  o.S = __shfl_xor(acc.S, 32);
  o.tb = __shfl_xor(acc.tb, 32);
  o.wb = __shfl_xor(acc.wb, 32);
  acc = h == 0 ? macc_merge(acc, o) : macc_merge(o, acc);
  if (h == 0) sacc[wave][rl] = acc;
  __syncthreads();
  if (wave == 0 && h == 0 && r < a.R) {
    MergeAcc f = sacc[0][rl];
    for (int w = 1; w < kMergeWaves; ++w) f = macc_merge(f, sacc[w][rl]);
    const size_t oi = (size_t)r * a.gamma + (k - 1);
    a.x[(size_t)r * (a.gamma + 1) + k] = winner_id(f.wb);
    if (a.greedy) {
      a.p[oi] = 1.0f;
      a.lse[oi] = f.m;
    } else {
      const float lse2 = f.m + log2f(f.S);
      a.p[oi] = exp2f(f.tb - lse2);
      a.lse[oi] = lse2 * kLn2;
    }
    a.best[winner_index(k - 1, a.R, r)] = 0ull;  // leave the workspace zeroed for the next call
  }
}

template <class W, int kKs, bool kGreedy, bool kDebug, bool kVec>
void launch_one(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  hipLaunchKernelGGL((markov_step_shared<W, kKs, kGreedy, kDebug, kVec>), dim3(plan.grid_x),
                     dim3(kStreamThreads),
                     (draft_stream_lds<W, kKs>(a.rank) + kWaves * kPatchFloats * sizeof(float)),
                     stream, a);
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
StepPlan plan_draft_step(int R, int V, int gamma) {
  StepPlan p{};
  p.n_vtiles = (V + kVTile - 1) / kVTile;
  const int rt = (R + kVTile - 1) / kVTile;
  p.n_groups = (rt + kWaves - 1) / kWaves;
  // at most 4 groups (R <= 512), so a group never has more requests (128)
  // than slabs (128 or more): one confidence head per workgroup at most
  int slabs = kDraftWgs / p.n_groups;
  if (p.n_groups > 1) slabs = (slabs / 8) * 8;
  p.n_slabs = slabs;
  p.grid_x = p.n_slabs * p.n_groups;
  p.grid_y = 1;
  p.rec_step = align256((size_t)p.n_slabs * 5 * R * 4);
  p.off_best = p.rec_step * gamma;
  p.ws_bytes = p.off_best + align256((size_t)gamma * R * 8 * kWinnerStride);
  return p;
}

hipError_t launch_draft_steps(StepArgs a, const StepPlan& plan, hipStream_t stream) {
  for (int k = 1; k <= a.gamma; ++k) {
    a.k = k;
    a.prev_from_best = k > 1;  // x_{k-1} straight from step k-1's winner word
    const hipError_t err = launch_draft_step(a, plan, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_draft_step(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  return a.bf16 ? launch_w<WBf16>(a, plan, stream) : launch_w<WF32>(a, plan, stream);
}

// Zero the winner words of a block (a workspace whose earlier contents are
// unknown): n 64-bit words from `best`, plain vector stores.
__global__ __launch_bounds__(256) void clear_words(unsigned long long* best, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    best[i] = 0ull;
}

hipError_t launch_clear_winners(const StepArgs& a, const StepPlan& plan, hipStream_t stream) {
  const size_t n = (plan.ws_bytes - plan.off_best) / sizeof(unsigned long long);
  const int blocks = (int)min((size_t)1024, (n + 255) / 256);
  hipLaunchKernelGGL(clear_words, dim3(blocks), dim3(256), 0, stream, a.best, n);
  return hipGetLastError();
}

hipError_t launch_draft_finalize(const StepArgs& a, const StepPlan& plan, int k0, int nk,
                                 hipStream_t stream) {
  (void)plan;
  const dim3 grid((a.R + kVTile - 1) / kVTile, nk), block(64 * kMergeWaves);
  hipLaunchKernelGGL(draft_merge, grid, block, 0, stream, a, k0);
  return hipGetLastError();
}

}  // namespace dspark

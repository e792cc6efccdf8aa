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
//   V2 verify_accept      one workgroup: per row (thread per row) merge V1's
//      chunks -> lse_t and test u < p_t(x_j) / p_d(x_j); per request the
//      acceptance chain over the admitted prefix; pick the one row per request that
//      needs a sample (residual at the first rejection, or bonus at row
//      ell+1); write n_accept, tau and tau_mean; clear the accumulators of
//      V3 and V5.  Greedy: also c* and the correction token (V3-V5 skipped).
//   V3 verify_tv          (T > 0) one pass over W2t, U and the target logits
//      for all rows: bias tile by MFMA, p_d and p_t, sum |p_d - p_t| per row,
//      accumulated across workgroups as exact fixed-point (2^-40) integers so
//      the result does not depend on the order of arrival.
//   V5 verify_sample      (T > 0) the same stream over only the sampled rows
//      (at most one per request): Gumbel race over max(p_t - p_d, 0)
//      (residual) or p_t (bonus), merged across workgroups with a 64-bit
//      atomic max of (order-preserving key, ~id), which is order-independent
//      and keeps the lowest id on ties.  When no 32-row tile meets more than
//      two requests (within gamma <= 16 that is gamma = 16), V3 runs this
//      race itself from the p_d and p_t it already holds and V5 is not
//      launched.
//   V4 verify_finalize    (T > 0) c* = 1 - sum/2 per row; winner -> next_token.
#include "dspark_kernels.h"
#include "mfma_stream.h"

namespace dspark {

namespace {

constexpr int kWaves = 4;        // sampling pass: waves (row tiles) per workgroup
constexpr int kTvWaves = 4;      // c* pass: waves (row tiles) per workgroup
constexpr int kTvThreads = 64 * kTvWaves;
constexpr int kTvResidentWgs = kResidentWgs * kStreamThreads / kTvThreads;  // one per CU
constexpr int kVerifyDist = 1;  // prefetch distance of the shared stream (two rows per entry)
constexpr double kFix = 1099511627776.0;  // 2^40, fixed-point unit of sum |p_d - p_t|

__device__ __forceinline__ int chunk_size(int V, int chunks) {
  const int cs = (V + chunks - 1) / chunks;
  return (cs + 3) & ~3;
}

// Order-preserving map of a float to uint32 (larger float -> larger code).
__device__ __forceinline__ uint32_t ordered(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
  int v = v0 + 4 * t;
  if constexpr (kVec && !kGreedy) {
    // Four 16-byte loads in flight per thread, folded together.
    for (; v + 3 * 1024 + 4 <= v1; v += 4096) {
      f32x4_t q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        q[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(trow + v + 1024 * j));
      float xm = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) xm = fmaxf(xm, fmaxf(fmaxf(q[j][0], q[j][1]), fmaxf(q[j][2], q[j][3])));
      const float mn = fmaxf(m, xm * a.kscale);
      S *= (mn == -INFINITY) ? 1.0f : fast_exp2(m - mn);
      m = mn;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) S += fast_exp2(fmaf(q[j][i], a.kscale, -mn));
    }
  }
  for (; v < v1; v += 1024) {
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
      const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
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
// V2: acceptance, one workgroup of 1024 threads.
//   Phase 1, one thread per row (r, j) (rows t, t + 1024, ...): merge V1's
//   chunks -> lse_t (greedy: lowest argmax); the acceptance test of drafted
//   token x_j, u(stream 2, r, j) < p_t(x_j) / p_d(x_j), kept as one byte in
//   LDS (tested for every j, used only up to ell[r]).  All rows' loads are
//   independent, so they are in flight together.
//   Phase 2, one thread per request: the first rejected position inside the
//   admitted prefix, the row that needs a sample, n_accept, tau; tau_mean by a
//   fixed-order tree over the requests.
// ---------------------------------------------------------------------------
constexpr int kAcceptThreads = 1024;
constexpr int kAcceptMaxRows = 512 * 16;  // R * gamma at the largest sizes

__global__ __launch_bounds__(kAcceptThreads) void verify_accept(VerifyArgs a, VerifyPlan p) {
  __shared__ unsigned char acc_ok[kAcceptMaxRows];
  __shared__ int stau[kAcceptThreads];
  const int t = threadIdx.x;
  float* lse_t2 = reinterpret_cast<float*>(a.ws + p.off_lse_t);
  int* targmax = reinterpret_cast<int*>(a.ws + p.off_lse_t);  // greedy reuses the slot
  int* srow = reinterpret_cast<int*>(a.ws + p.off_srow);      // sampled k (1-based) or 0
  int* skind = reinterpret_cast<int*>(a.ws + p.off_skind);    // 1 residual, 2 bonus
  unsigned long long* tvsum = reinterpret_cast<unsigned long long*>(a.ws + p.off_tv);
  unsigned long long* best = reinterpret_cast<unsigned long long*>(a.ws + p.off_best);
  const float* lp = reinterpret_cast<const float*>(a.ws + p.off_lsepart);
  const int n_rows = a.R * a.gamma;

  for (int row = t; row < n_rows; row += kAcceptThreads) {
    const int r = row / a.gamma, j = row - r * a.gamma + 1;  // drafted position j = k
    const float* q = lp + (size_t)row * p.lse_chunks * 2;
    const int xraw = a.x[(size_t)r * (a.gamma + 1) + j];
    const int xj = checked_token(xraw, a.V, a.err);
    bool ok;
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
      a.c_star[row] = (xraw == idx) ? 1.0f : 0.0f;
      ok = xj == idx;  // ratio 1 or 0 against u in [2^-24, 1)
    } else {
      const float tx = a.target[(size_t)row * a.V + xj];
      const float pdx = a.p_d_x[row];
      float m = -INFINITY, S = 0.0f;
      for (int c = 0; c < p.lse_chunks; ++c) {
        const float mc = q[2 * c], sc = q[2 * c + 1];
        const float M = fmaxf(m, mc);
        S = (M == -INFINITY) ? 0.0f : S * fast_exp2(m - M) + sc * fast_exp2(mc - M);
        m = M;
      }
      const float l2 = m + log2f(S);
      lse_t2[row] = l2;
      tvsum[row] = 0ull;
      const float pt = exp2f(fmaf(tx, a.kscale, -l2));
      const float u = bits_to_uniform(pcg(row_key(a.seed, kStreamAccept, (uint32_t)r, (uint32_t)j)));
      ok = u < pt / pdx;
    }
    acc_ok[row] = ok ? 1 : 0;
  }
  __syncthreads();

  int tau = 0;
  if (t < a.R) {
    const int r = t;
    best[r] = 0ull;
    int ell = a.ell[r];
    ell = ell < 0 ? 0 : (ell > a.gamma ? a.gamma : ell);  // device values are not validated
    int n_acc = 0, kind = 0, ks = 0, nxt = -1;
    for (int j = 1; j <= ell; ++j) {
      if (acc_ok[r * a.gamma + (j - 1)]) {
        ++n_acc;
      } else {
        kind = 1;
        ks = j;
        break;
      }
    }
    if (kind == 0 && ell < a.gamma) {
      kind = 2;
      ks = ell + 1;
    }
    if (a.greedy && kind != 0) nxt = targmax[r * a.gamma + (ks - 1)];
    srow[r] = ks;
    skind[r] = kind;
    a.n_accept[r] = n_acc;
    a.tau[r] = n_acc + 1;
    a.next_token[r] = nxt;
    tau = n_acc + 1;
  }
  stau[t] = tau;
  __syncthreads();
  for (int s = kAcceptThreads / 2; s > 0; s >>= 1) {
    if (t < s) stau[t] += stau[t + s];
    __syncthreads();
  }
  if (t == 0) *a.tau_mean = (float)stau[0] / (float)a.R;
}

// E fragments of request r at position k: the caller's bias rows (RNN head)
// or the Markov rows W1[x_{k-1}].
template <class W, int kKs>
__device__ __forceinline__ void verify_gather(typename W::frag_t (&ef)[W::kMaxKs],
                                              const VerifyArgs& a, int r, int k, int half) {
  if (a.E_rows)
    load_e_frags<W, kKs>(ef, a.E_rows, r * a.gamma + (k - 1), a.rank, a.R * a.gamma, half);
  else
    load_e_frags<W, kKs>(ef, a.W1,
                         checked_token(a.x[(size_t)r * (a.gamma + 1) + (k - 1)], a.V, a.err),
                         a.rank, a.V, half);
}

// Map blockIdx to (slab, group); the groups of one slab share an XCD.
__device__ __forceinline__ void slab_group(int b, int n_slabs, int n_groups, int& slab, int& grp) {
  if (n_groups == 1 || n_slabs % 8 != 0) {
    slab = b % n_slabs;
    grp = b / n_slabs;
  } else {
    grp = (b >> 3) % n_groups;
    slab = (b / (8 * n_groups)) * 8 + (b & 7);
  }
}

// ---------------------------------------------------------------------------
// V3: sum |p_d - p_t| over all rows (T > 0).
// ---------------------------------------------------------------------------
// Rows of U and of the target logits: with kVec read as whole lines through
// the wave's LDS patch (RowTiles), otherwise each lane loads its own row.
template <bool kVec>
struct UTRows {
  const float* urow;
  const float* trow;
  float* patch;
  int V, half;
  float ubuf[kVec ? 1 : kVerifyDist + 1][16], tbuf[kVec ? 1 : kVerifyDist + 1][16];
  RowTiles<2, kVec ? kVerifyDist + 1 : 1> rows;
  static constexpr int kLoads = kVec ? 8 : 32;

  template <int S>
  __device__ __forceinline__ void prefetch(int vt) {
    if constexpr (kVec) {
      rows.template load<S>(vt);
    } else {
      const int vb = (vt < 0 ? 0 : vt * kVTile) + 16 * half;
      load16<false>(ubuf[S], urow, vb);
      load16<false>(tbuf[S], trow, vb);
    }
  }
  // Lane-layout U and target of slot S.
  template <int S>
  __device__ __forceinline__ void get(float (&ut)[2][16]) {
    if constexpr (kVec) {
      rows.template to_lanes<S>(patch, ut);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ut[0][i] = ubuf[S][i];
        ut[1][i] = tbuf[S][i];
      }
    }
  }
  __device__ __forceinline__ void get_tail(float (&ut)[2][16], int vt) {
    load16_masked(ut[0], urow, vt * kVTile + 16 * half, V, 0.0f);
    load16_masked(ut[1], trow, vt * kVTile + 16 * half, V, 0.0f);
  }
};

// Gumbel race of the rows that need a sample, run inside the c* pass when a
// row tile holds the sampled rows of at most two requests (slot 0: the tile's
// first request, slot 1: the next one).  The lanes holding such a row publish
// the tile's p_d and p_t of that row through a per-wave LDS slot; then lane l
// races entry l % 32 of slot l / 32, so the race costs one entry per lane and
// tile instead of sixteen.  Per entry it is the same race as the sampling pass
// (same weights, same generator draws), merged across lanes and workgroups by
// the same order-independent (key, ~id) maximum.
struct SampleRace {
  float* slot;     // per wave: [2 slots][p_d 32 | p_t 32] floats
  int pub;         // this lane's row is the sampled row of slot pub (or -1)
  bool active;     // the slot this lane races has a sampled row
  int kind;        // 1 residual max(p_t - p_d, 0), 2 bonus p_t
  uint32_t state;  // generator state of the sampled row
  float bE, bLn;
  int bV;

  template <bool kMasked>
  __device__ __forceinline__ void step(const float (&pd)[16], const float (&pt)[16], int vt,
                                       int half, int lane, int V) {
    if (pub >= 0) {
      float* dst = slot + pub * 64 + 16 * half;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * j;
        *reinterpret_cast<f32x4_t*>(dst + i) = f32x4_t{pd[i], pd[i + 1], pd[i + 2], pd[i + 3]};
        *reinterpret_cast<f32x4_t*>(dst + 32 + i) = f32x4_t{pt[i], pt[i + 1], pt[i + 2], pt[i + 3]};
      }
    }
    // A wave's LDS operations complete in issue order, so the reads below see
    // the stores above (and the next tile's stores come after these reads).
    const float* src = slot + (lane >> 5) * 64 + (lane & 31);
    const float d = src[0], t = src[32];
    const int v = vt * kVTile + (lane & 31);
    float e = (kind == 1) ? fmaxf(t - d, 0.0f) : t;
    if (!active || (kMasked && v >= V)) e = 0.0f;
    const float ln = fast_log2(bits_to_uniform(rxs_m_xs(state + (uint32_t)v * kLcgMul)));
    const bool win = e * bLn < bE * ln;  // e / L > bE / bL with L = -ln
    bE = win ? e : bE;
    bLn = win ? ln : bLn;
    bV = win ? v : bV;
  }
};

// kMu also accumulates sum_v sign(p_d - p_t) p_d, the row constant of the
// derivative of the TV term (training gradients).  kSample also runs the
// sampling race (SampleRace).
template <bool kVec, bool kMu, bool kSample = false>
struct TvEpi : UTRows<kVec> {
  float kscale, lse2_d, lse2_t;
  float sabs, smu;
  SampleRace race;

  template <bool kMasked>
  __device__ __forceinline__ void fold(const float (&ut)[2][16], const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * this->half;
    float pd[16], pt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pd[i] = fast_exp2(fmaf(ut[0][i] + acc[i], kscale, -lse2_d));
      pt[i] = fast_exp2(fmaf(ut[1][i], kscale, -lse2_t));
      const float d = fabsf(pd[i] - pt[i]);
      const bool in = !kMasked || vb + i < this->V;
      sabs += in ? d : 0.0f;
      if constexpr (kMu) smu += (in && pd[i] != pt[i]) ? (pd[i] > pt[i] ? pd[i] : -pd[i]) : 0.0f;
    }
    if constexpr (kSample)
      race.template step<kMasked>(pd, pt, vt, this->half, threadIdx.x & 63, this->V);
  }
  template <int S>
  __device__ void consume(const f32x16_t& acc, int vt) {
    float ut[2][16];
    this->template get<S>(ut);
    fold<false>(ut, acc, vt);
  }
  __device__ void tail(const f32x16_t& acc, int vt) {
    float ut[2][16];
    this->get_tail(ut, vt);
    fold<true>(ut, acc, vt);
  }
};

template <class W, int kKs, bool kVec, bool kMu = false, bool kSample = false>
__global__ __launch_bounds__(kTvThreads) void verify_tv(VerifyArgs a, VerifyPlan p,
                                                        unsigned long long* mu_acc = nullptr) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  int slab, grp;
  slab_group(blockIdx.x, p.n_slabs, p.n_groups, slab, grp);
  int t_begin, t_end;
  slab_range(slab, p.n_slabs, p.n_vtiles, t_begin, t_end);

  const int row = (grp * kTvWaves + wave) * kVTile + col;
  const int rowc = row < p.n_rows ? row : p.n_rows - 1;
  const int r = rowc / a.gamma, k = rowc % a.gamma + 1;
  typename W::frag_t e[W::kMaxKs];
  TvEpi<kVec, kMu, kSample> epi;
  epi.urow = a.U + (size_t)rowc * a.V;
  epi.trow = a.target + (size_t)rowc * a.V;
  epi.V = a.V;
  epi.half = half;
  epi.patch = reinterpret_cast<float*>(lds + stream_lds_bytes<W>(a.rank, kVerifyDist)) +
              wave * kPatchFloats;
  if constexpr (kVec) {
    const int row0 = (grp * kTvWaves + wave) * kVTile;
    epi.rows.base[0] = a.U;
    epi.rows.base[1] = a.target;
    epi.rows.init([&](int j) {
      const int rr = row0 + j < p.n_rows ? row0 + j : p.n_rows - 1;
      return (size_t)rr * a.V;
    });
  }
  epi.kscale = a.kscale;
  epi.lse2_d = a.lse_d[rowc] * kLog2e;
  epi.lse2_t = reinterpret_cast<const float*>(a.ws + p.off_lse_t)[rowc];
  epi.sabs = 0.0f;
  epi.smu = 0.0f;
  int race_r = 0;
  if constexpr (kSample) {
    // The sampled rows of the (at most two) requests that meet this row tile.
    const int row0 = (grp * kTvWaves + wave) * kVTile;
    const int rlast = min(row0 + kVTile - 1, p.n_rows - 1);
    const int* srow = reinterpret_cast<const int*>(a.ws + p.off_srow);
    const int* skind = reinterpret_cast<const int*>(a.ws + p.off_skind);
    int scol[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int rq = row0 / a.gamma + q;
      const int ks = rq < a.R ? srow[rq] : 0;
      const int sr = rq * a.gamma + ks - 1;
      scol[q] = (ks > 0 && sr >= row0 && sr <= rlast) ? sr - row0 : -1;
    }
    SampleRace& rc = epi.race;
    rc.slot = reinterpret_cast<float*>(lds + stream_lds_bytes<W>(a.rank, kVerifyDist)) +
              kTvWaves * kPatchFloats + wave * 128;
    rc.pub = col == scol[0] ? 0 : (col == scol[1] ? 1 : -1);
    const int q = lane >> 5;
    race_r = row0 / a.gamma + q;
    rc.active = scol[q] >= 0;
    const int rr = rc.active ? race_r : 0;
    rc.kind = rc.active ? skind[rr] : 2;
    const uint32_t stream = rc.kind == 1 ? kStreamResid : kStreamBonus;
    rc.state = row_key(a.seed, stream, (uint32_t)rr, (uint32_t)(rc.active ? srow[rr] : 1)) *
                   kLcgMul + kLcgInc;
    rc.bE = 0.0f;
    rc.bLn = -1.0f;
    rc.bV = -1;
  }
  auto gather = [&](typename W::frag_t(&ef)[W::kMaxKs]) { verify_gather<W, kKs>(ef, a, r, k, half); };
  shared_a_stream<W, kKs, kVerifyDist, kTvThreads>(a.W2t, a.V, a.rank, t_begin, t_end, e, gather,
                                                   lds, epi);
  if constexpr (kSample) {
    const SampleRace& rc = epi.race;
    float key = (rc.bV >= 0 && rc.bE > 0.0f) ? fast_log2(rc.bE) - fast_log2(-rc.bLn) : -INFINITY;
    int idx = (rc.bV >= 0 && rc.bE > 0.0f) ? rc.bV : -1;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      const float ko = __shfl_xor(key, m);
      const int io = __shfl_xor(idx, m);
      if (rec_beats(ko, io, key, idx)) {
        key = ko;
        idx = io;
      }
    }
    if (col == 0 && rc.active && idx >= 0) {
      const unsigned long long packed =
          ((unsigned long long)ordered(key) << 32) | (unsigned long long)(~(uint32_t)idx);
      atomicMax(reinterpret_cast<unsigned long long*>(a.ws + p.off_best) + race_r, packed);
    }
  }

  const float s = epi.sabs + __shfl_xor(epi.sabs, 32);
  if (half == 0 && row < p.n_rows) {
    const unsigned long long q = (unsigned long long)llrint((double)s * kFix);
    atomicAdd(reinterpret_cast<unsigned long long*>(a.ws + p.off_tv) + row, q);
  }
  if constexpr (kMu) {
    // signed fixed point in two's complement: the wrapping 64-bit sum is exact
    const float sm = epi.smu + __shfl_xor(epi.smu, 32);
    if (half == 0 && row < p.n_rows)
      atomicAdd(mu_acc + row, (unsigned long long)llrint((double)sm * kFix));
  }
}

// ---------------------------------------------------------------------------
// V5: Gumbel race over the sampled rows (T > 0), one virtual row per request.
// ---------------------------------------------------------------------------
template <bool kVec>
struct SampleEpi : UTRows<kVec> {
  int kind;
  float kscale, lse2_d, lse2_t;
  uint32_t state_row;
  float bE, bLn;
  int bV;

  template <bool kMasked>
  __device__ __forceinline__ void fold(const float (&ut)[2][16], const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * this->half;
    const uint32_t s0 = state_row + (uint32_t)vb * kLcgMul;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pd = fast_exp2(fmaf(ut[0][i] + acc[i], kscale, -lse2_d));
      const float pt = fast_exp2(fmaf(ut[1][i], kscale, -lse2_t));
      float e = (kind == 1) ? fmaxf(pt - pd, 0.0f) : pt;
      if constexpr (kMasked) e = (vb + i < this->V) ? e : 0.0f;
      const float ln = fast_log2(bits_to_uniform(rxs_m_xs(s0 + (uint32_t)i * kLcgMul)));
      // e / L > bE / bL  <=>  e * bLn < bE * ln     (L = -ln > 0)
      const bool win = e * bLn < bE * ln;
      bE = win ? e : bE;
      bLn = win ? ln : bLn;
      bV = win ? vb + i : bV;
    }
  }
  template <int S>
  __device__ void consume(const f32x16_t& acc, int vt) {
    float ut[2][16];
    this->template get<S>(ut);
    fold<false>(ut, acc, vt);
  }
  __device__ void tail(const f32x16_t& acc, int vt) {
    float ut[2][16];
    this->get_tail(ut, vt);
    fold<true>(ut, acc, vt);
  }
};

template <class W, int kKs, bool kVec>
__global__ __launch_bounds__(kStreamThreads) void verify_sample(VerifyArgs a, VerifyPlan p) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  int slab, grp;
  slab_group(blockIdx.x, p.s_slabs, p.s_groups, slab, grp);
  int t_begin, t_end;
  slab_range(slab, p.s_slabs, p.n_vtiles, t_begin, t_end);

  const int r = (grp * kWaves + wave) * kVTile + col;
  const int rc = r < a.R ? r : a.R - 1;
  const int* srow = reinterpret_cast<const int*>(a.ws + p.off_srow);
  const int* skind = reinterpret_cast<const int*>(a.ws + p.off_skind);
  const int ks = srow[rc];
  const int k = ks > 0 ? ks : 1;  // lanes without a sample run row 1 and never store
  const int row = rc * a.gamma + (k - 1);
  typename W::frag_t e[W::kMaxKs];
  SampleEpi<kVec> epi;
  epi.urow = a.U + (size_t)row * a.V;
  epi.trow = a.target + (size_t)row * a.V;
  epi.V = a.V;
  epi.half = half;
  epi.patch = reinterpret_cast<float*>(lds + stream_lds_bytes<W>(a.rank, kVerifyDist)) +
              wave * kPatchFloats;
  if constexpr (kVec) {
    const int r0w = (grp * kWaves + wave) * kVTile;
    epi.rows.base[0] = a.U;
    epi.rows.base[1] = a.target;
    epi.rows.init([&](int j) {
      const int rq = r0w + j < a.R ? r0w + j : a.R - 1;
      const int kq = srow[rq] > 0 ? srow[rq] : 1;
      return ((size_t)rq * a.gamma + (kq - 1)) * a.V;
    });
  }
  epi.kind = skind[rc];
  epi.kscale = a.kscale;
  epi.lse2_d = a.lse_d[row] * kLog2e;
  epi.lse2_t = reinterpret_cast<const float*>(a.ws + p.off_lse_t)[row];
  const uint32_t stream = epi.kind == 1 ? kStreamResid : kStreamBonus;
  epi.state_row = row_key(a.seed, stream, (uint32_t)rc, (uint32_t)k) * kLcgMul + kLcgInc;
  epi.bE = 0.0f;
  epi.bLn = -1.0f;
  epi.bV = -1;
  auto gather = [&](typename W::frag_t(&ef)[W::kMaxKs]) { verify_gather<W, kKs>(ef, a, rc, k, half); };
  shared_a_stream<W, kKs, kVerifyDist>(a.W2t, a.V, a.rank, t_begin, t_end, e, gather, lds, epi);

  float key = (epi.bV >= 0 && epi.bE > 0.0f) ? fast_log2(epi.bE) - fast_log2(-epi.bLn) : -INFINITY;
  int idx = (epi.bV >= 0 && epi.bE > 0.0f) ? epi.bV : -1;
  const float key_o = __shfl_xor(key, 32);
  const int idx_o = __shfl_xor(idx, 32);
  if (rec_beats(key_o, idx_o, key, idx)) {
    key = key_o;
    idx = idx_o;
  }
  if (half == 0 && r < a.R && ks > 0 && idx >= 0) {
    const unsigned long long packed =
        ((unsigned long long)ordered(key) << 32) | (unsigned long long)(~(uint32_t)idx);
    atomicMax(reinterpret_cast<unsigned long long*>(a.ws + p.off_best) + r, packed);
  }
}

// ---------------------------------------------------------------------------
// V4: finalisation (T > 0): c* for every row, the sampled token per request.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void verify_finalize(VerifyArgs a, VerifyPlan p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < p.n_rows) {
    const unsigned long long q = reinterpret_cast<const unsigned long long*>(a.ws + p.off_tv)[i];
    a.c_star[i] = (float)(1.0 - 0.5 * ((double)q / kFix));
  }
  if (i < a.R) {
    const int ks = reinterpret_cast<const int*>(a.ws + p.off_srow)[i];
    const unsigned long long b = reinterpret_cast<const unsigned long long*>(a.ws + p.off_best)[i];
    if (ks > 0 && b != 0ull) a.next_token[i] = (int)(~(uint32_t)(b & 0xFFFFFFFFull));
  }
}

// ---------------------------------------------------------------------------
// Training losses [P1 §5]: T1 the draft normaliser of every row (r, k) with
// the target block as the Markov input (teacher forcing), and the draft logit
// of the target token x*_k; then the target normalisers (V1), the c* pass (V3)
// and the confidence head reused as they are, and T3 the weighted sums.
// ---------------------------------------------------------------------------
// U rows only (the draft side), line-coalesced through the wave's LDS patch
// with kVec.
template <bool kVec>
struct URows {
  const float* urow;
  float* patch;
  int V, half;
  float ubuf[kVec ? 1 : kVerifyDist + 1][16];
  RowTiles<1, kVec ? kVerifyDist + 1 : 1> rows;
  static constexpr int kLoads = kVec ? 4 : 16;

  template <int S>
  __device__ __forceinline__ void prefetch(int vt) {
    if constexpr (kVec)
      rows.template load<S>(vt);
    else
      load16<false>(ubuf[S], urow, (vt < 0 ? 0 : vt * kVTile) + 16 * half);
  }
  template <int S>
  __device__ __forceinline__ void get(float (&u)[1][16]) {
    if constexpr (kVec) {
      rows.template to_lanes<S>(patch, u);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) u[0][i] = ubuf[S][i];
    }
  }
};

// Online max / sum of 2^t (t = z * log2(e) / T) over the lane's entries, and
// t at the row's target token.
template <bool kVec>
struct DraftLseEpi : URows<kVec> {
  float kscale, m, S, tx;
  int xs;  // target token of the lane's row

  template <bool kMasked>
  __device__ __forceinline__ void fold(const float (&u)[16], const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * this->half;
    float t[16];
    float tm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      t[i] = (u[i] + acc[i]) * kscale;
      if (kMasked && vb + i >= this->V) t[i] = -INFINITY;
      tm = fmaxf(tm, t[i]);
      tx = (vb + i == xs) ? t[i] : tx;
    }
    const float mn = fmaxf(m, tm);
    if (mn == -INFINITY) return;  // nothing seen yet (a tile past the vocabulary end)
    S *= fast_exp2(m - mn);
    m = mn;
#pragma unroll
    for (int i = 0; i < 16; ++i) S += fast_exp2(t[i] - mn);
  }
  template <int S_>
  __device__ void consume(const f32x16_t& acc, int vt) {
    float u[1][16];
    this->template get<S_>(u);
    fold<false>(u[0], acc, vt);
  }
  __device__ void tail(const f32x16_t& acc, int vt) {
    float u[16];
    load16_masked(u, this->urow, vt * kVTile + 16 * this->half, this->V, 0.0f);
    fold<true>(u, acc, vt);
  }
};

// T1: per (row group, slab) records {m, S, t_x} of every row, planes
// [slab][3][n_rows] in the workspace.
template <class W, int kKs, bool kVec>
__global__ __launch_bounds__(kTvThreads) void train_draft_lse(VerifyArgs a, VerifyPlan p,
                                                              TrainPlan tp) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  int slab, grp;
  slab_group(blockIdx.x, p.n_slabs, p.n_groups, slab, grp);
  int t_begin, t_end;
  slab_range(slab, p.n_slabs, p.n_vtiles, t_begin, t_end);

  const int row = (grp * kTvWaves + wave) * kVTile + col;
  const int rowc = row < p.n_rows ? row : p.n_rows - 1;
  const int r = rowc / a.gamma, k = rowc % a.gamma + 1;
  typename W::frag_t e[W::kMaxKs];
  DraftLseEpi<kVec> epi;
  epi.urow = a.U + (size_t)rowc * a.V;
  epi.V = a.V;
  epi.half = half;
  epi.patch = reinterpret_cast<float*>(lds + stream_lds_bytes<W>(a.rank, kVerifyDist)) +
              wave * kPatchFloats;
  if constexpr (kVec) {
    const int row0 = (grp * kTvWaves + wave) * kVTile;
    epi.rows.base[0] = a.U;
    epi.rows.init([&](int j) {
      const int rr = row0 + j < p.n_rows ? row0 + j : p.n_rows - 1;
      return (size_t)rr * a.V;
    });
  }
  epi.kscale = a.kscale;
  epi.m = -INFINITY;
  epi.S = 0.0f;
  epi.tx = -INFINITY;
  epi.xs = a.x[(size_t)r * (a.gamma + 1) + k];
  auto gather = [&](typename W::frag_t(&ef)[W::kMaxKs]) {
    load_e_frags<W, kKs>(ef, a.W1,
                         checked_token(a.x[(size_t)r * (a.gamma + 1) + (k - 1)], a.V, a.err),
                         a.rank, a.V, half);
  };
  shared_a_stream<W, kKs, kVerifyDist, kTvThreads>(a.W2t, a.V, a.rank, t_begin, t_end, e, gather,
                                                   lds, epi);
  // both halves of the tile: merge (half 0 first), lane half 0 stores
  const float m_o = __shfl_xor(epi.m, 32), s_o = __shfl_xor(epi.S, 32);
  const float t_o = __shfl_xor(epi.tx, 32);
  const float M = fmaxf(epi.m, m_o);
  const float Ssum = (M == -INFINITY) ? 0.0f
                                      : (half == 0 ? epi.S * fast_exp2(epi.m - M) + s_o * fast_exp2(m_o - M)
                                                   : s_o * fast_exp2(m_o - M) + epi.S * fast_exp2(epi.m - M));
  const float tx = fmaxf(epi.tx, t_o);
  if (half == 0 && row < p.n_rows) {
    float* rec = reinterpret_cast<float*>(a.ws + tp.off_dlse) + (size_t)slab * 3 * p.n_rows + row;
    rec[0] = M;
    rec[p.n_rows] = Ssum;
    rec[2 * (size_t)p.n_rows] = tx;
  }
}

// T2: per row, the draft normaliser and log2 p_d(x*) from the slab records
// (slab order), the target normaliser from V1's chunks, and a cleared c*
// accumulator.
__global__ __launch_bounds__(256) void train_merge(VerifyArgs a, VerifyPlan p, TrainPlan tp) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= p.n_rows) return;
  const float* rec = reinterpret_cast<const float*>(a.ws + tp.off_dlse);
  float m = -INFINITY, S = 0.0f, tx = -INFINITY;
  for (int sl = 0; sl < p.n_slabs; ++sl) {
    const float* q = rec + (size_t)sl * 3 * p.n_rows + row;
    const float ms = q[0], ss = q[p.n_rows];
    const float M = fmaxf(m, ms);
    S = (M == -INFINITY) ? 0.0f : S * fast_exp2(m - M) + ss * fast_exp2(ms - M);
    m = M;
    tx = fmaxf(tx, q[2 * (size_t)p.n_rows]);
  }
  const float l2 = m + log2f(S);
  reinterpret_cast<float*>(a.ws + tp.off_lse_d)[row] = l2 * kLn2;  // natural log, as V3 expects
  reinterpret_cast<float*>(a.ws + tp.off_ce)[row] = (l2 - tx) * kLn2;
  const float* lp = reinterpret_cast<const float*>(a.ws + p.off_lsepart) + (size_t)row * p.lse_chunks * 2;
  float mt = -INFINITY, St = 0.0f;
  for (int c = 0; c < p.lse_chunks; ++c) {
    const float mc = lp[2 * c], sc = lp[2 * c + 1];
    const float M = fmaxf(mt, mc);
    St = (M == -INFINITY) ? 0.0f : St * fast_exp2(mt - M) + sc * fast_exp2(mc - M);
    mt = M;
  }
  reinterpret_cast<float*>(a.ws + p.off_lse_t)[row] = mt + log2f(St);
  reinterpret_cast<unsigned long long*>(a.ws + p.off_tv)[row] = 0ull;
  reinterpret_cast<unsigned long long*>(a.ws + tp.off_mu)[row] = 0ull;
}

// T3: per-position terms (ce, tv, conf, c) and the weighted sums in a fixed
// order: thread t folds rows t, t + 1024, ... in order (fp64), then a tree.
constexpr int kAssembleThreads = 1024;

__global__ __launch_bounds__(kAssembleThreads) void train_assemble(VerifyArgs a, VerifyPlan p,
                                                                   TrainPlan tp, TrainArgs ta) {
  __shared__ double red[3][kAssembleThreads];
  const int t = threadIdx.x;
  double s_ce = 0.0, s_tv = 0.0, s_cf = 0.0;
  for (int row = t; row < p.n_rows; row += kAssembleThreads) {
    const int k = row % a.gamma + 1;
    const double wk = exp(-(double)(k - 1) / (double)ta.lambda);
    const float ce = reinterpret_cast<const float*>(a.ws + tp.off_ce)[row];
    const unsigned long long q = reinterpret_cast<const unsigned long long*>(a.ws + p.off_tv)[row];
    const double tv = (double)q / kFix;
    const double cs = 1.0 - 0.5 * tv;
    const double c = (double)ta.c[row];
    const double cf = -(cs * log(c) + (1.0 - cs) * log1p(-c));
    float* out = ta.terms + (size_t)row * 4;
    out[0] = ce;
    out[1] = (float)tv;
    out[2] = (float)cf;
    out[3] = (float)c;
    // derivative of the weighted total with respect to the confidence logit
    reinterpret_cast<float*>(a.ws + tp.off_dl)[row] = (float)(wk * (double)ta.alpha_conf * (c - cs));
    s_ce += wk * (double)ce;
    s_tv += wk * tv;
    s_cf += wk * cf;
  }
  red[0][t] = s_ce;
  red[1][t] = s_tv;
  red[2][t] = s_cf;
  __syncthreads();
  for (int s = kAssembleThreads / 2; s > 0; s >>= 1) {
    if (t < s)
      for (int j = 0; j < 3; ++j) red[j][t] += red[j][t + s];
    __syncthreads();
  }
  if (t == 0) {
    ta.sums[0] = red[0][0];
    ta.sums[1] = red[1][0];
    ta.sums[2] = red[2][0];
    ta.sums[3] = (double)ta.alpha_ce * red[0][0] + (double)ta.alpha_tv * red[1][0] +
                 (double)ta.alpha_conf * red[2][0];
  }
}


// ---------------------------------------------------------------------------
// G1: gradient of the weighted total with respect to the logits z = U + e.W2
// (dL/dU, equal to dL/dz), one pass over W2t, U and the target logits:
//   dz_v = (w_k / T) [a_CE (p_d(v) - [v = x*_k]) + a_TV p_d(v) (s_v - mu)],
//   s_v = sign(p_d(v) - p_t(v)), mu = sum_u s_u p_d(u) (from V3 with kMu),
// with c* held constant [P1 "DSpark" §5; the TV term is differentiated as the
// L1 norm, whose sign is 0 where p_d = p_t].
// ---------------------------------------------------------------------------
template <bool kVec>
struct GradEpi : UTRows<kVec> {
  float kscale, lse2_d, lse2_t, mu, sce, stv;
  int xs;
  float* drow;  // dU row of the lane; null for a row past the end
  float* dU;    // with kVec: full tiles leave through the wave's LDS patch as whole row lines
  bool line_ok[4];  // the row of this lane's line store q exists

  template <bool kMasked>
  __device__ __forceinline__ void fold(const float (&ut)[2][16], const f32x16_t& acc, int vt) {
    const int vb = vt * kVTile + 16 * this->half;
    float g[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pd = fast_exp2(fmaf(ut[0][i] + acc[i], kscale, -lse2_d));
      const float pt = fast_exp2(fmaf(ut[1][i], kscale, -lse2_t));
      const float sg = pd > pt ? 1.0f : (pd < pt ? -1.0f : 0.0f);
      const float hot = (vb + i == xs) ? 1.0f : 0.0f;
      g[i] = fmaf(sce, pd - hot, stv * pd * (sg - mu));
    }
    if constexpr (kVec && !kMasked) {
      // the inverse of the row loads' patch pass: lane layout in, row lines
      // out (the patch is free once this tile's inputs were read from it)
      const int l = threadIdx.x & 63;
      float* wr = this->patch + (l & 31) * kPatchRowFloats + 16 * (l >> 5);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<f32x4_t*>(wr + 4 * c) = f32x4_t{g[4 * c], g[4 * c + 1], g[4 * c + 2], g[4 * c + 3]};
      const float* rd = this->patch + (l >> 3) * kPatchRowFloats + 4 * (l & 7);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(rd + 8 * q * kPatchRowFloats);
        if (line_ok[q]) *reinterpret_cast<f32x4_t*>(dU + this->rows.off[q] + vt * kVTile) = v;
      }
      return;
    }
    if (drow == nullptr) return;
    {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!kMasked || vb + i < this->V) drow[vb + i] = g[i];
    }
  }
  template <int S>
  __device__ void consume(const f32x16_t& acc, int vt) {
    float ut[2][16];
    this->template get<S>(ut);
    fold<false>(ut, acc, vt);
  }
  __device__ void tail(const f32x16_t& acc, int vt) {
    float ut[2][16];
    this->get_tail(ut, vt);
    fold<true>(ut, acc, vt);
  }
};

template <class W, int kKs, bool kVec>
__global__ __launch_bounds__(kTvThreads) void train_grad_logits(VerifyArgs a, VerifyPlan p,
                                                                TrainPlan tp, TrainArgs ta) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  int slab, grp;
  slab_group(blockIdx.x, p.n_slabs, p.n_groups, slab, grp);
  int t_begin, t_end;
  slab_range(slab, p.n_slabs, p.n_vtiles, t_begin, t_end);

  const int row = (grp * kTvWaves + wave) * kVTile + col;
  const int rowc = row < p.n_rows ? row : p.n_rows - 1;
  const int r = rowc / a.gamma, k = rowc % a.gamma + 1;
  typename W::frag_t e[W::kMaxKs];
  GradEpi<kVec> epi;
  epi.urow = a.U + (size_t)rowc * a.V;
  epi.trow = a.target + (size_t)rowc * a.V;
  epi.V = a.V;
  epi.half = half;
  epi.patch = reinterpret_cast<float*>(lds + stream_lds_bytes<W>(a.rank, kVerifyDist)) +
              wave * kPatchFloats;
  if constexpr (kVec) {
    const int row0 = (grp * kTvWaves + wave) * kVTile;
    epi.rows.base[0] = a.U;
    epi.rows.base[1] = a.target;
    epi.rows.init([&](int j) {
      const int rr = row0 + j < p.n_rows ? row0 + j : p.n_rows - 1;
      return (size_t)rr * a.V;
    });
  }
  // the same p_d and p_t expressions as V3, so the signs match its mu
  epi.kscale = a.kscale;
  epi.lse2_d = a.lse_d[rowc] * kLog2e;
  epi.lse2_t = reinterpret_cast<const float*>(a.ws + p.off_lse_t)[rowc];
  const long long mq = (long long)reinterpret_cast<const unsigned long long*>(a.ws + tp.off_mu)[rowc];
  epi.mu = (float)((double)mq / kFix);
  const double wk = exp(-(double)(k - 1) / (double)ta.lambda) * (double)ta.inv_t;
  epi.sce = (float)(wk * (double)ta.alpha_ce);
  epi.stv = (float)(wk * (double)ta.alpha_tv);
  epi.xs = a.x[(size_t)r * (a.gamma + 1) + k];
  epi.drow = row < p.n_rows ? ta.dU + (size_t)row * a.V : nullptr;
  epi.dU = ta.dU;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    epi.line_ok[q] = (grp * kTvWaves + wave) * kVTile + 8 * q + (lane >> 3) < p.n_rows;
  auto gather = [&](typename W::frag_t(&ef)[W::kMaxKs]) {
    load_e_frags<W, kKs>(ef, a.W1,
                         checked_token(a.x[(size_t)r * (a.gamma + 1) + (k - 1)], a.V, a.err),
                         a.rank, a.V, half);
  };
  shared_a_stream<W, kKs, kVerifyDist, kTvThreads>(a.W2t, a.V, a.rank, t_begin, t_end, e, gather,
                                                   lds, epi);
}

template <class W, int kKs, bool kVec>
hipError_t launch_train_passes(const VerifyArgs& a, const VerifyPlan& p, const TrainPlan& tp,
                               bool mu, hipStream_t stream) {
  const size_t lds = stream_lds_bytes<W>(a.rank, kVerifyDist) + kWaves * kPatchFloats * 4;
  hipLaunchKernelGGL((train_draft_lse<W, kKs, kVec>), dim3(p.n_slabs * p.n_groups),
                     dim3(kTvThreads), lds, stream, a, p, tp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(train_merge, dim3((p.n_rows + 255) / 256), dim3(256), 0, stream, a, p, tp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mu)
    hipLaunchKernelGGL((verify_tv<W, kKs, kVec, true>), dim3(p.n_slabs * p.n_groups),
                       dim3(kTvThreads), lds, stream, a, p,
                       reinterpret_cast<unsigned long long*>(a.ws + tp.off_mu));
  else
    hipLaunchKernelGGL((verify_tv<W, kKs, kVec>), dim3(p.n_slabs * p.n_groups), dim3(kTvThreads),
                       lds, stream, a, p, nullptr);
  return hipGetLastError();
}

template <class W, int kKs, bool kVec>
hipError_t launch_grad_pass(const VerifyArgs& a, const VerifyPlan& p, const TrainPlan& tp,
                            const TrainArgs& ta, hipStream_t stream) {
  const size_t lds = stream_lds_bytes<W>(a.rank, kVerifyDist) + kWaves * kPatchFloats * 4;
  hipLaunchKernelGGL((train_grad_logits<W, kKs, kVec>), dim3(p.n_slabs * p.n_groups),
                     dim3(kTvThreads), lds, stream, a, p, tp, ta);
  return hipGetLastError();
}

template <class W, bool kVec>
hipError_t launch_train_w(const VerifyArgs& a, const VerifyPlan& p, const TrainPlan& tp,
                          bool mu, hipStream_t stream) {
  if (W::kKStep * W::kMaxKs == a.rank) return launch_train_passes<W, W::kMaxKs, kVec>(a, p, tp, mu, stream);
  return launch_train_passes<W, 0, kVec>(a, p, tp, mu, stream);
}

template <bool kVec>
hipError_t launch_grad_w(const VerifyArgs& a, const VerifyPlan& p, const TrainPlan& tp,
                         const TrainArgs& ta, hipStream_t stream) {
  using W = WBf16;
  if (W::kKStep * W::kMaxKs == a.rank) return launch_grad_pass<W, W::kMaxKs, kVec>(a, p, tp, ta, stream);
  return launch_grad_pass<W, 0, kVec>(a, p, tp, ta, stream);
}

template <class W, int kKs, bool kVec>
hipError_t launch_passes(const VerifyArgs& a, const VerifyPlan& p, hipStream_t stream) {
  // W2t slots, then one LDS patch per wave (U and target rows pass in turn).
  const size_t lds = stream_lds_bytes<W>(a.rank, kVerifyDist) + kWaves * kPatchFloats * 4;
  if (p.fuse_sample) {
    // the sampling race rides on the c* pass: one race slot pair per wave
    hipLaunchKernelGGL((verify_tv<W, kKs, kVec, false, true>), dim3(p.n_slabs * p.n_groups),
                       dim3(kTvThreads), lds + kTvWaves * 128 * 4, stream, a, p, nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((verify_tv<W, kKs, kVec>), dim3(p.n_slabs * p.n_groups), dim3(kTvThreads),
                     lds, stream, a, p, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_sample<W, kKs, kVec>), dim3(p.s_slabs * p.s_groups),
                     dim3(kStreamThreads), lds, stream, a, p);
  return hipGetLastError();
}

template <class W, bool kVec>
hipError_t launch_w(const VerifyArgs& a, const VerifyPlan& p, hipStream_t stream) {
  if (W::kKStep * W::kMaxKs == a.rank) return launch_passes<W, W::kMaxKs, kVec>(a, p, stream);
  return launch_passes<W, 0, kVec>(a, p, stream);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int plan_slabs(int n_groups, int n_vtiles, int resident) {
  int slabs = resident / n_groups;
  if (n_groups > 1) slabs = (slabs / 8) * 8;
  if (slabs < 8) slabs = 8;
  if (slabs > n_vtiles) slabs = n_vtiles;
  if (n_groups > 1 && slabs % 8 != 0 && n_vtiles >= 8) slabs = (n_vtiles / 8) * 8;
  return slabs;
}

}  // namespace

VerifyPlan plan_verify(int R, int V, int gamma) {
  VerifyPlan p{};
  p.n_rows = R * gamma;
  p.n_rtiles = (p.n_rows + kVTile - 1) / kVTile;
  p.n_groups = (p.n_rtiles + kTvWaves - 1) / kTvWaves;
  p.n_vtiles = (V + kVTile - 1) / kVTile;
  p.n_slabs = plan_slabs(p.n_groups, p.n_vtiles, kTvResidentWgs);
  p.s_groups = ((R + kVTile - 1) / kVTile + kWaves - 1) / kWaves;
  p.s_slabs = plan_slabs(p.s_groups, p.n_vtiles, kResidentWgs);
  // The race rides on the c* pass when no row tile meets more than two requests.
  p.fuse_sample = 1;
  for (int t = 0; t < p.n_rtiles && p.fuse_sample; ++t) {
    const int last = t * kVTile + kVTile - 1 < p.n_rows - 1 ? t * kVTile + kVTile - 1 : p.n_rows - 1;
    if (last / gamma - (t * kVTile) / gamma > 1) p.fuse_sample = 0;
  }
  int chunks = (2048 + p.n_rows - 1) / p.n_rows;
  const int max_chunks = (V + 1023) / 1024;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks > 64) chunks = 64;
  if (chunks < 1) chunks = 1;
  p.lse_chunks = chunks;
  size_t off = 0;
  p.off_lse_t = off;
  off = align256(off + (size_t)p.n_rows * 4);
  p.off_tv = off;
  off = align256(off + (size_t)p.n_rows * 8);
  p.off_best = off;
  off = align256(off + (size_t)R * 8);
  p.off_srow = off;
  off = align256(off + (size_t)R * 4);
  p.off_skind = off;
  off = align256(off + (size_t)R * 4);
  p.off_lsepart = off;
  off = align256(off + (size_t)p.n_rows * p.lse_chunks * 8);
  p.ws_bytes = off;
  return p;
}

TrainPlan plan_train(int R, int V, int rank, int d, int gamma) {
  const VerifyPlan p = plan_verify(R, V, gamma);
  TrainPlan t{};
  size_t off = p.ws_bytes;
  t.off_dlse = off;
  off = align256(off + (size_t)p.n_slabs * 3 * p.n_rows * 4);
  t.off_lse_d = off;
  off = align256(off + (size_t)p.n_rows * 4);
  t.off_ce = off;
  off = align256(off + (size_t)p.n_rows * 4);
  t.off_c = off;
  off = align256(off + (size_t)p.n_rows * 4);
  t.off_surv = off;
  off = align256(off + (size_t)p.n_rows * 4);
  t.off_mu = off;
  off = align256(off + (size_t)p.n_rows * 8);
  t.off_dl = off;
  off = align256(off + (size_t)p.n_rows * 4);
  t.ws_bytes = off;
  // gradients
  t.n_pad = (p.n_rows + 127) / 128 * 128;
  t.vp = (V + 63) / 64 * 64;
  t.e_groups = t.n_pad / 128;
  const int chunks = t.vp / 64;
  int slabs = kResidentWgs / t.e_groups;
  if (slabs < 1) slabs = 1;
  if (slabs > chunks) slabs = chunks;
  t.e_slabs = slabs;
  t.off_w2 = off;
  off = align256(off + (size_t)rank * t.vp * 2);
  t.off_et = off;
  off = align256(off + (size_t)rank * t.n_pad * 2);
  t.off_dep = off;
  off = align256(off + (size_t)t.e_slabs * t.n_pad * rank * 4);
  t.off_de = off;
  off = align256(off + (size_t)p.n_rows * rank * 4);
  t.off_dwp = off;
  off = align256(off + (size_t)16 * (d + rank) * 8);
  t.ws_grad_bytes = off;
  return t;
}

hipError_t launch_train(const VerifyArgs& va, const TrainArgs& ta, const VerifyPlan& p,
                        const TrainPlan& tp, hipStream_t stream) {
  VerifyArgs a = va;
  a.lse_d = reinterpret_cast<const float*>(a.ws + tp.off_lse_d);
  const bool vec = (a.V % 4) == 0;
  const bool grad = ta.dU != nullptr;
  const dim3 g1(p.lse_chunks, p.n_rows);
  if (vec) hipLaunchKernelGGL((verify_target_lse<false, true>), g1, dim3(256), 0, stream, a, p);
  else hipLaunchKernelGGL((verify_target_lse<false, false>), g1, dim3(256), 0, stream, a, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.bf16) e = vec ? launch_train_w<WBf16, true>(a, p, tp, grad, stream) : launch_train_w<WBf16, false>(a, p, tp, grad, stream);
  else e = vec ? launch_train_w<WF32, true>(a, p, tp, grad, stream) : launch_train_w<WF32, false>(a, p, tp, grad, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(train_assemble, dim3(1), dim3(kAssembleThreads), 0, stream, a, p, tp, ta);
  if ((e = hipGetLastError()) != hipSuccess || !grad) return e;
  if (!a.bf16) return hipErrorInvalidValue;
  e = vec ? launch_grad_w<true>(a, p, tp, ta, stream) : launch_grad_w<false>(a, p, tp, ta, stream);
  if (e != hipSuccess) return e;
  return launch_train_grad_rest(a, ta, p, tp, stream);
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
  hipLaunchKernelGGL(verify_accept, dim3(1), dim3(kAcceptThreads), 0, stream, a, p);
  e = hipGetLastError();
  if (e != hipSuccess || a.greedy) return e;
  if (a.bf16) e = vec ? launch_w<WBf16, true>(a, p, stream) : launch_w<WBf16, false>(a, p, stream);
  else e = vec ? launch_w<WF32, true>(a, p, stream) : launch_w<WF32, false>(a, p, stream);
  if (e != hipSuccess) return e;
  const int n = p.n_rows > a.R ? p.n_rows : a.R;
  hipLaunchKernelGGL(verify_finalize, dim3((n + 255) / 256), dim3(256), 0, stream, a, p);
  return hipGetLastError();
}

}  // namespace dspark

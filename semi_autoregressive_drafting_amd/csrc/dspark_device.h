// Device-side building blocks shared by the DSpark kernels (gfx950 only).
//
//  * Counter-based generator: the PCG hash of Jarzynski & Olano ("Hash Functions
//    for GPU Rendering", JCGT 9(3), 2020) -- one step of the 32-bit LCG with
//    multiplier 747796405 and increment 2891336453, then PCG's RXS-M-XS output
//    permutation with multiplier 277803737.  A row (seed, stream, request,
//    position) gets a key by folding the seed's low word, its high word, the
//    stream id, the request and the position into the hash one after another;
//    element v of the row draws bits = pcg(key + v) and u = ((bits >> 9) + 0.5)
//    * 2^-23, an odd multiple of 2^-24 that fp32 holds exactly.
//  * MFMA fragment traits for bf16 (v_mfma_f32_32x32x16_bf16) and fp32
//    (v_mfma_f32_32x32x2f32) weights.  Both produce the 32x32 fp32 tile in the
//    same lane layout: lane l holds column l % 32 and, in accumulator i, row
//    8*(i/4) + 4*(l/32) + i%4.
//  * The partial-result record of the online softmax + Gumbel race and its
//    merge (commutative; callers fix the merge order so results are
//    bit-reproducible).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr uint32_t kLcgMul = 747796405u;
constexpr uint32_t kLcgInc = 2891336453u;
constexpr uint32_t kRxsMul = 277803737u;

constexpr uint32_t kStreamDraft = 1, kStreamAccept = 2, kStreamResid = 3, kStreamBonus = 4,
                   kStreamDraftEntry = 5;
// Ids per block of the two-level draft sampler (aligned vocabulary blocks).
constexpr int kDraftBlock = 16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Output permutation applied to an LCG state.
__device__ __forceinline__ uint32_t rxs_m_xs(uint32_t state) {
  uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * kRxsMul;
  return (word >> 22u) ^ word;
}

__device__ __forceinline__ uint32_t pcg(uint32_t v) { return rxs_m_xs(v * kLcgMul + kLcgInc); }

__device__ __forceinline__ uint32_t row_key(uint64_t seed, uint32_t stream, uint32_t req,
                                            uint32_t k) {
  uint32_t h = pcg((uint32_t)(seed & 0xFFFFFFFFull));
  h = pcg(h ^ (uint32_t)(seed >> 32));
  h = pcg(h ^ stream);
  h = pcg(h ^ req);
  return pcg(h ^ k);
}

// LCG state of element v of a row with key `key`: (key + v) * mul + inc.  For
// consecutive v the states differ by kLcgMul, so the first multiply is hoisted.
__device__ __forceinline__ uint32_t row_state(uint32_t key, uint32_t v) {
  return (key + v) * kLcgMul + kLcgInc;
}

// ((bits >> 9) + 0.5) * 2^-23, built as the float 1 + (bits >> 9) * 2^-23
// (exponent 127 funnel-shifted onto the top 23 bits) minus (1 - 2^-24).  Both
// operands lie within a factor of two of each other, so the difference is exact
// (Sterbenz) and equals the value above bit for bit.
__device__ __forceinline__ float bits_to_uniform(uint32_t bits) {
  return __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, bits, 9u)) - (1.0f - 0x1p-24f);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// MFMA weight traits.  `row` points at one rank-vector (a row of W1 or W2t).
// ---------------------------------------------------------------------------
struct WBf16 {
  using store_t = uint16_t;
  using frag_t = bf16x8_t;
  static constexpr int kKStep = 16;  // k per MFMA
  static constexpr int kHalf = 8;    // k per lane half
  static constexpr int kMaxKs = 16;  // rank <= 256
  __device__ static frag_t load(const store_t* row, int ks, int half) {
    return *reinterpret_cast<const bf16x8_t*>(row + ks * kKStep + half * kHalf);
  }
  __device__ static frag_t zero() { return frag_t{}; }
  __device__ static f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static float to_f32(store_t v) { return __uint_as_float((uint32_t)v << 16); }
};

struct WF32 {
  using store_t = float;
  using frag_t = float;
  static constexpr int kKStep = 2;
  static constexpr int kHalf = 1;
  static constexpr int kMaxKs = 64;  // rank <= 128
  __device__ static frag_t load(const store_t* row, int ks, int half) {
    return row[ks * kKStep + half * kHalf];
  }
  __device__ static frag_t zero() { return 0.0f; }
  __device__ static f32x16_t mma(frag_t a, frag_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static float to_f32(store_t v) { return v; }
};

// MFMA row m of a 32-wide vocabulary tile is mapped to tile column perm(m) so
// that accumulator i of lane l holds vocabulary entry 16*(l/32) + i: each lane
// then owns 16 consecutive entries of one request.
__device__ __forceinline__ int tile_perm(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// ---------------------------------------------------------------------------
// Partial result of the online softmax + Gumbel race over a vocabulary range,
// in log2 units of s = z / T (t = s * log2 e):
//   m     running maximum of t          S     sum of 2^(t - m)
//   key   t_best - log2(L_best), L = -log2(u) (an exponential variate up to
//         the factor ln 2): the winner's Gumbel-perturbed score in log2 units,
//         up to a constant common to all entries; larger wins, ties -> lower id
//   tbest t of the winner               idx   winner's vocabulary id (-1: none)
// Greedy (T = 0) reuses the record with t = z, key = z, S unused.
// ---------------------------------------------------------------------------
struct Rec {
  float m, S, key, tbest;
  int idx;
};

__device__ __forceinline__ bool rec_beats(float k1, int i1, float k2, int i2) {
  if (i2 < 0) return i1 >= 0;
  if (i1 < 0) return false;
  return (k1 > k2) || (k1 == k2 && i1 < i2);
}

__device__ __forceinline__ Rec rec_merge(const Rec& a, const Rec& b) {
  Rec r;
  r.m = fmaxf(a.m, b.m);
  if (r.m == -INFINITY) {
    r.S = 0.0f;
  } else {
    r.S = a.S * fast_exp2(a.m - r.m) + b.S * fast_exp2(b.m - r.m);
  }
  bool take_a = rec_beats(a.key, a.idx, b.key, b.idx);
  r.key = take_a ? a.key : b.key;
  r.tbest = take_a ? a.tbest : b.tbest;
  r.idx = take_a ? a.idx : b.idx;
  return r;
}

__device__ __forceinline__ Rec rec_shfl_xor(const Rec& a, int mask) {
  Rec r;
  r.m = __shfl_xor(a.m, mask);
  r.S = __shfl_xor(a.S, mask);
  r.key = __shfl_xor(a.key, mask);
  r.tbest = __shfl_xor(a.tbest, mask);
  r.idx = __shfl_xor(a.idx, mask);
  return r;
}

// ---------------------------------------------------------------------------
// Confidence head c = sigma(w[0:d] . h + w[d:] . e)  [P1 §3.1, eq. c_k] of one
// (request, position), computed by the 4 waves of a workgroup: over the
// concatenated vector v = [h; e] of length n = d + rank, wave q takes the
// quarter [q * n4, (q + 1) * n4) (n4 a multiple of the 16-byte chunk), its
// lanes accumulate lane-strided fp32 partial sums, a butterfly reduces the
// wave, and the four wave sums are added in wave order.  The draft step and
// the batched confidence kernel both call conf_dot_wg, so their c values are
// bit-identical.
// ---------------------------------------------------------------------------
template <class W>
__device__ __forceinline__ float conf_dot_part(const typename W::store_t* hrow,
                                               const typename W::store_t* erow, const float* w,
                                               int d, int rank, int j0, int j1, int lane) {
  using store_t = typename W::store_t;
  constexpr int kV = 16 / sizeof(store_t);  // elements per 16-byte chunk (8 bf16 / 4 fp32)
  float dot = 0.0f;
  // 16-byte chunks when no chunk straddles h and e and every row is aligned.
  const bool vec = (d % kV) == 0 &&
                   ((reinterpret_cast<uintptr_t>(hrow) | reinterpret_cast<uintptr_t>(erow) |
                     reinterpret_cast<uintptr_t>(w)) & 15u) == 0;
  if (vec) {
#pragma unroll 4
    for (int j = j0 + lane * kV; j < j1; j += 64 * kV) {
      const store_t* src = j < d ? hrow + j : erow + (j - d);
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src);
      const store_t* vs = reinterpret_cast<const store_t*>(&v);
#pragma unroll
      for (int i = 0; i < kV; i += 4) {
        const f32x4_t wv = *reinterpret_cast<const f32x4_t*>(w + j + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) dot = fmaf(wv[q], W::to_f32(vs[i + q]), dot);
      }
    }
  } else {
    for (int j = j0 + lane; j < j1; j += 64) {
      const float v = W::to_f32(j < d ? hrow[j] : erow[j - d]);
      dot = fmaf(w[j], v, dot);
    }
  }
  (void)rank;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
  return dot;
}

// All 256 threads of the workgroup must call it; every thread gets c.
// `red` is 4 floats of LDS.
template <class W>
__device__ __forceinline__ float conf_dot_wg(const typename W::store_t* hrow,
                                             const typename W::store_t* erow, const float* w,
                                             int d, int rank, float* red) {
  constexpr int kV = 16 / sizeof(typename W::store_t);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = d + rank;
  const int n4 = ((n + 3) / 4 + kV - 1) / kV * kV;
  const int j0 = min(n, wave * n4), j1 = min(n, j0 + n4);
  const float part = conf_dot_part<W>(hrow, erow, w, d, rank, j0, j1, lane);
  if (lane == 0) red[wave] = part;
  __syncthreads();
  const float dot = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();  // red may be reused
  return dot;
}

// conf_dot_part for bf16 rows in 16-byte chunks, split in two so that the loads
// can be issued long before the arithmetic: load() issues this lane's chunks
// (at most kConfChunks, i.e. d + rank up to 4 * 64 * 8 * kConfChunks), dot()
// then performs conf_dot_part's fused multiply-adds in its order and the same
// butterfly, so the result is bit-identical.
constexpr int kConfChunks = 3;
struct ConfPreload {
  u32x4_t v[kConfChunks];
  f32x4_t w0[kConfChunks], w1[kConfChunks];
  int n;  // chunks of this lane
  __device__ __forceinline__ void load(const uint16_t* hrow, const uint16_t* erow, const float* w,
                                       int d, int j0, int j1, int lane) {
    n = 0;
#pragma unroll
    for (int c = 0; c < kConfChunks; ++c) {
      const int j = j0 + lane * 8 + c * 64 * 8;
      const bool ok = j < j1;
      const int jj = ok ? j : 0;  // a valid address whose values are not used
      const uint16_t* src = jj < d ? hrow + jj : erow + (jj - d);
      v[c] = *reinterpret_cast<const u32x4_t*>(src);
      w0[c] = *reinterpret_cast<const f32x4_t*>(w + jj);
      w1[c] = *reinterpret_cast<const f32x4_t*>(w + jj + 4);
      n += ok ? 1 : 0;
    }
  }
  __device__ __forceinline__ float dot() const {
    float dot = 0.0f;
#pragma unroll
    for (int c = 0; c < kConfChunks; ++c) {
      if (c < n) {
        const uint16_t* vs = reinterpret_cast<const uint16_t*>(&v[c]);
#pragma unroll
        for (int q = 0; q < 4; ++q) dot = fmaf(w0[c][q], WBf16::to_f32(vs[q]), dot);
#pragma unroll
        for (int q = 0; q < 4; ++q) dot = fmaf(w1[c][q], WBf16::to_f32(vs[4 + q]), dot);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
    return dot;
  }
};

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

// A token id read from device memory, clamped into [0, V) so that the row
// gather it drives stays inside W1.  An id outside [0, V) (a corrupted anchor
// or block, or a step that found no winner) also sets the library's
// token-error word to 1 with a plain store (the host reads it back with
// dspark_token_errors); nothing traps.
__device__ __forceinline__ int checked_token(int x, int V, uint32_t* err) {
  if (x >= 0 && x < V) return x;
  if (err != nullptr) *err = 1u;
  return x < 0 ? 0 : V - 1;
}

// Winner words of the draft steps: one 64-bit word per (step, request), each
// alone in its 128-byte line.  Every workgroup of a step publishes into the
// words of all its requests with a device-scope atomic max, and atomics on one
// line are serialised; with 16 requests per line the step's atomics queued
// behind each other for several microseconds.
constexpr int kWinnerStride = 16;  // 64-bit words from one winner word to the next
__host__ __device__ inline size_t winner_index(int k_idx, int R, int r) {
  return ((size_t)k_idx * R + r) * kWinnerStride;
}

// Vocabulary id in a draft step's 64-bit winner word (-1: no winner).  The
// word packs an order-preserving key above the complemented id, so a 64-bit
// atomic max keeps the largest key and, on ties, the lowest id.
__device__ __forceinline__ int winner_id(unsigned long long w) {
  return w == 0ull ? -1 : (int)(~(uint32_t)(w & 0xFFFFFFFFull));
}

// Balanced split of T tiles over n slabs: the first n - T%n slabs get T/n
// tiles, the rest one more (so low slab ids carry the lighter share).
__host__ __device__ inline void slab_range(int s, int n, int T, int& b, int& e) {
  const int q = T / n, rem = T % n, lo = n - rem;
  b = s * q + (s > lo ? s - lo : 0);
  e = b + q + (s >= lo ? 1 : 0);
}

}  // namespace dspark

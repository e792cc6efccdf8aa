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
//   G2 transpose_w2     W2t [V][rank] -> w2, zero past V
//   G3 gather_et        E^T from W1 and x*, zero past n_rows
//      Both copies are chunk-major, [K / 64][rank][64]: the B operand of one
//      64-wide K chunk of a contraction is one contiguous 32 KB block.
//   G4 grad_e_partial   per (128-row group, vocabulary slab) partial dz . W2t
//   G5 grad_e_reduce    slab partials in slab order + dl w[d:]  -> dE
//   G6 grad_w2t         per 32-entry vocabulary tile, dz^T . E over all rows
//   G7 zero_floats / scatter_dw1   dW1 = 0, then per token the sum of its dE
//      rows in row order (written by the token's first row)
//   G8 grad_dh, grad_dw_part / grad_dw_final   dh; dw as fp64 sums over row
//      ranges, then over the ranges, each in a fixed order
#include "dspark_kernels.h"
#include "mfma_stream.h"

namespace dspark {

namespace {

constexpr int kGThreads = 256;  // 4 waves
constexpr int kChunk = 64;      // K per chunk of the contractions (4 MFMA K steps)

struct GradArgs {
  int V, rank, d, gamma, n_rows, n_pad, vp, e_slabs, e_groups;
  const uint16_t* W1;
  const uint16_t* W2t;
  const uint16_t* h;
  const float* w;
  const int32_t* x;  // x* [R][gamma + 1]
  uint32_t* err;     // token-error word (checked_token)
  const float* dz;   // [n_rows][V]
  const float* dl;   // [n_rows]
  uint16_t* w2;      // W2t transposed, chunk-major [vp / 64][rank][64]
  uint16_t* et;      // E^T, chunk-major [n_pad / 64][rank][64]
  float* dep;        // [e_slabs][n_pad][rank]
  float* de;         // [n_rows][rank]
  float* dW1;
  float* dW2t;
  float* dh;
  float* dw;
};

__device__ __forceinline__ int row_token(const GradArgs& g, int row) {
  const int r = row / g.gamma, k = row % g.gamma;  // position k+1 reads x*_k
  return checked_token(g.x[(size_t)r * (g.gamma + 1) + k], g.V, g.err);
}

// bf16 of an fp32 value, round to nearest even (values here are finite).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}


// ---------------------------------------------------------------------------
// G2 / G3: 64 x 64 tiles through LDS, read along rank and written along K
// into the chunk-major copy: element (n, k) at ((k / 64) rank + n) 64 + k % 64.
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
    if (n < g.rank && v < g.vp) g.w2[((size_t)(v >> 6) * g.rank + n) * 64 + (v & 63)] = tile[vv][nn];
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
    if (n < g.rank && row < g.n_pad)
      g.et[((size_t)(row >> 6) * g.rank + n) * 64 + (row & 63)] = tile[rr][nn];
  }
}

// ---------------------------------------------------------------------------
// The two contractions share one shape: a workgroup of 4 waves, each wave a
// 32 x (32 NC) fp32 output block in MFMA accumulators, K walked in chunks of
// 64.  The B operand of a chunk (32 NC rows of 64 K values, one contiguous
// block of the chunk-major copy) is common to the 4 waves: the workgroup
// copies it into LDS once (16 bytes per thread and piece, rows padded to 72 elements so
// that the lanes' 16-byte reads spread over all banks), loading chunk i+1 into
// registers while chunk i multiplies.  MFMA operands for K step s of a chunk:
//   A:  lane (m = l%32, half h) holds the 8 values k = 16 s + 8 h .. +7 of row m
//   B:  lane (n = l%32, half h) holds B-row n at the same 8 k.
// ---------------------------------------------------------------------------
constexpr int kLdsRow = kChunk + 8;

template <int NC>
struct BChunk {
  static constexpr int kPer = NC;  // 16-byte pieces per thread: NC * 32 rows * 8 pieces / 256
  u32x4_t reg[kPer];
  // chunk: the block of one K chunk, rows of 64 values
  __device__ __forceinline__ void load(const uint16_t* chunk) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = threadIdx.x + kGThreads * i;
      reg[i] = *reinterpret_cast<const u32x4_t*>(chunk + 8 * p);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = threadIdx.x + kGThreads * i, n = p >> 3, q = p & 7;
      *reinterpret_cast<u32x4_t*>(lds + n * kLdsRow + 8 * q) = reg[i];
    }
  }
};

template <int NC>
__device__ __forceinline__ void mma_chunk(f32x16_t (&acc)[NC], const bf16x8_t (&a)[4],
                                          const uint16_t* lds, int col, int half) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8_t af = a[s];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8_t bf =
          *reinterpret_cast<const bf16x8_t*>(lds + (c * 32 + col) * kLdsRow + 16 * s + 8 * half);
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[c], 0, 0, 0);
    }
  }
}

// Chunk loop over [c_begin, c_end) (at least one chunk), B from the
// chunk-major copy `bsrc`, the A operand staged like B: load_raw(ch) issues a
// wave's global loads of chunk ch (whole 128-byte lines), put_raw() rounds
// them to bf16 and writes them into the wave's A patch (32 rows of 64 K values,
// kLdsRow apart, the layout of the B chunk), from which every lane reads its
// MFMA operands.  In the lane layout itself a load instruction would touch 32
// different lines; the patch lets each instruction read whole lines.
template <int NC, class LoadRaw, class PutRaw>
__device__ __forceinline__ void contract_staged(f32x16_t (&acc)[NC], const uint16_t* bsrc,
                                                int c_begin, int c_end, uint16_t* lds,
                                                const uint16_t* apatch, LoadRaw load_raw,
                                                PutRaw put_raw) {
  constexpr size_t kChunkElems = (size_t)NC * 32 * kChunk;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  BChunk<NC> b;
  b.load(bsrc + c_begin * kChunkElems);
  load_raw(c_begin);
  b.store(lds);
  put_raw();
  lds_barrier();
  for (int ch = c_begin; ch < c_end; ++ch) {
    const int cn = ch + 1 < c_end ? ch + 1 : ch;
    b.load(bsrc + cn * kChunkElems);
    load_raw(cn);
    // keep the next chunk's loads ahead of this chunk's MFMAs (the scheduler
    // would otherwise sink them next to their use, leaving the latency bare)
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t cur[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      cur[s] = *reinterpret_cast<const bf16x8_t*>(apatch + col * kLdsRow + 16 * s + 8 * half);
    mma_chunk<NC>(acc, cur, lds, col, half);
    // and keep put_raw's selects on the loaded values (rows and entries past
    // the end become zeros) behind the MFMAs: hoisted above them, they made
    // the wave wait for the next chunk's loads before this chunk's MFMAs
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // every wave is past its reads of this chunk
    b.store(lds);
    put_raw();
    lds_barrier();
  }
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2((uint32_t)bf16_rne(a) | ((uint32_t)bf16_rne(b) << 16),
                    (uint32_t)bf16_rne(c) | ((uint32_t)bf16_rne(d) << 16));
}

// G4: wave q of workgroup (group, slab) owns rows 32 (4 group + q) .. +31;
// K = the vocabulary of the slab, B = w2.
template <int NC, bool kVec>
__global__ __launch_bounds__(kGThreads) void grad_e_partial(GradArgs g) {
  __shared__ __align__(16) uint16_t lds[NC * 32 * kLdsRow];
  __shared__ __align__(16) uint16_t apatch[4][32 * kLdsRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  // blockIdx -> (group, slab): workgroups are dealt to the 8 XCDs in turn, so
  // when the slabs divide evenly among them every group of a slab runs on one
  // XCD and the slab's w2 chunks are fetched into one L2 only.
  int grp, slab;
  if (g.e_slabs % 8 == 0) {
    const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    slab = xcd * (g.e_slabs / 8) + j / g.e_groups;
    grp = j % g.e_groups;
  } else {
    grp = blockIdx.x % g.e_groups;
    slab = blockIdx.x / g.e_groups;
  }
  const int rt = grp * 4 + wave;
  int c_begin, c_end;
  slab_range(slab, g.e_slabs, g.vp / kChunk, c_begin, c_end);

  // load instruction q of a chunk, lane l: the wave's row 4q + l/16 (rows past
  // n_rows read row n_rows - 1; their results are never used), entries
  // 4 (l%16) .. +3 of the chunk (zeros past V)
  const int lrow = lane >> 4, lk = 4 * (lane & 15);
  const float* zq[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = min(rt * 32 + 4 * q + lrow, g.n_rows - 1);
    zq[q] = g.dz + (size_t)row * g.V + lk;
  }
  // With V % 4 == 0 a lane's 4 entries are all inside V or all past it: the
  // loads go unconditionally to an in-bounds address and the entries past V
  // become zeros when they are written to the patch (a select right after a
  // load would make the wave wait for it).
  f32x4_t raw[8];
  bool kin = true;
  uint16_t* ap = apatch[wave];
  auto load_raw = [&](int ch) {
    const int vb = ch * kChunk + lk;
    if constexpr (kVec) {
      kin = vb < g.V;
      const int off = kin ? ch * kChunk : 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) raw[q] = *reinterpret_cast<const f32x4_t*>(zq[q] + off);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) raw[q][j] = vb + j < g.V ? zq[q][ch * kChunk + j] : 0.0f;
    }
  };
  auto put_raw = [&]() {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<uint2*>(ap + (4 * q + lrow) * kLdsRow + lk) =
          kin ? pack4_bf16(raw[q][0], raw[q][1], raw[q][2], raw[q][3]) : make_uint2(0u, 0u);
  };

  f32x16_t acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x16_t{};
  contract_staged<NC>(acc, g.w2, c_begin, c_end, lds, ap, load_raw, put_raw);
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

// G6: wave q of workgroup b owns vocabulary tile vt = 4 b + q (entries past V
// read as zero and are not written); K = all rows, B = et.  The wave's A patch
// holds the tile transposed, [entry][row]: lane l loads rows 32 g + 4 (l/8)
// + j (g = 0, 1; j = 0..3) at entries 4 (l%8) .. +3 of the tile, so each load
// instruction reads 8 whole 128-byte row segments, and writes, per entry, its
// 4 consecutive rows as one 8-byte piece.
template <int NC, bool kVec>
__global__ __launch_bounds__(kGThreads) void grad_w2t(GradArgs g) {
  __shared__ __align__(16) uint16_t lds[NC * 32 * kLdsRow];
  __shared__ __align__(16) uint16_t apatch[4][32 * kLdsRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int vt = blockIdx.x * 4 + wave;
  const int le = 4 * (lane & 7), lr = 4 * (lane >> 3);
  const int v0 = vt * 32 + le;  // this lane's first entry
  const bool vin = v0 < g.V;  // with V % 4 == 0: all 4 entries or none
  const float* zc = g.dz + (vin ? v0 : 0);
  // loads go unconditionally to in-bounds rows (row n_rows - 1 past the end);
  // rows past n_rows and entries past V become zeros in the patch
  f32x4_t raw[2][4];
  unsigned rin = 0u;  // bit 4 gg + j: row 32 gg + lr + j of the chunk exists
  uint16_t* ap = apatch[wave];
  auto load_raw = [&](int ch) {
    rin = 0u;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = ch * kChunk + 32 * gg + lr + j;
        rin |= (rr < g.n_rows ? 1u : 0u) << (4 * gg + j);
        if constexpr (kVec) {
          raw[gg][j] = *reinterpret_cast<const f32x4_t*>(zc + (size_t)min(rr, g.n_rows - 1) * g.V);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            raw[gg][j][e] = (rr < g.n_rows && v0 + e < g.V) ? zc[(size_t)rr * g.V + e] : 0.0f;
        }
      }
  };
  auto put_raw = [&]() {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      float v[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = (!kVec || vin) && ((rin >> (4 * gg + j)) & 1u);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][e] = ok ? raw[gg][j][e] : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint2*>(ap + (le + e) * kLdsRow + 32 * gg + lr) =
            pack4_bf16(v[0][e], v[1][e], v[2][e], v[3][e]);
    }
  };

  f32x16_t acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x16_t{};
  contract_staged<NC>(acc, g.et, 0, g.n_pad / kChunk, lds, ap, load_raw, put_raw);
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
// writes: the sum of that token's dE rows in row order.  The rows are scanned
// in windows of 256 (one per thread); a window's matches are compacted into
// LDS in row order (wave ballots, then wave offsets), and thread j adds their
// column j.
__global__ __launch_bounds__(kGThreads) void scatter_dw1(GradArgs g) {
  __shared__ int list[kGThreads];
  __shared__ int wcount[4];
  const int row = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int tok = row_token(g, row);
  int seen = 0;
  for (int r = t; r < row; r += kGThreads) seen |= row_token(g, r) == tok;
  if (__syncthreads_or(seen)) return;  // an earlier row owns this token
  float s = 0.0f;
  for (int base = row; base < g.n_rows; base += kGThreads) {
    const int r = base + t;
    const bool m = r < g.n_rows && row_token(g, r) == tok;
    const unsigned long long bal = __ballot(m);
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    int off = 0;
    for (int q = 0; q < wave; ++q) off += wcount[q];
    const int n = wcount[0] + wcount[1] + wcount[2] + wcount[3];
    if (m) list[off + __popcll(bal & ((1ull << lane) - 1ull))] = r;
    __syncthreads();
    if (t < g.rank)
      for (int i = 0; i < n; ++i) s += g.de[(size_t)list[i] * g.rank + t];
    __syncthreads();  // list and wcount are rewritten by the next window
  }
  if (t < g.rank) g.dW1[(size_t)tok * g.rank + t] = s;
}

// G8: dh = dl w[:d].
__global__ __launch_bounds__(kGThreads) void grad_dh(GradArgs g) {
  const size_t i = (size_t)blockIdx.x * kGThreads + threadIdx.x;
  if (i >= (size_t)g.n_rows * g.d) return;
  const int row = (int)(i / g.d), j = (int)(i % g.d);
  g.dh[i] = g.dl[row] * g.w[j];
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// dw[j] = sum over rows of dl [h; e]_j in a fixed order: workgroup (b, split)
// takes columns 64 b .. +63 and rows [split L, (split + 1) L); wave q adds
// rows q, q + 4, ... of that range in order (fp64), the 4 wave sums are added
// in wave order into partial[split][j]; grad_dw_final adds the splits in order.
constexpr int kDwSplits = 16;

__global__ __launch_bounds__(kGThreads) void grad_dw_part(GradArgs g, double* part) {
  __shared__ double red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const int split = blockIdx.y;
  const int L = (g.n_rows + kDwSplits - 1) / kDwSplits;
  const int r0 = split * L, r1 = min(g.n_rows, r0 + L);
  double s = 0.0;
  if (j < g.d + g.rank) {
#pragma unroll 4
    for (int row = r0 + wave; row < r1; row += 4) {
      const uint16_t v = j < g.d ? g.h[(size_t)row * g.d + j]
                                 : g.W1[(size_t)row_token(g, row) * g.rank + (j - g.d)];
      s += (double)g.dl[row] * (double)bf16_to_f32(v);
    }
  }
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && j < g.d + g.rank)
    part[(size_t)split * (g.d + g.rank) + j] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

__global__ __launch_bounds__(kGThreads) void grad_dw_final(GradArgs g, const double* part) {
  const int j = blockIdx.x * kGThreads + threadIdx.x;
  if (j >= g.d + g.rank) return;
  double s = 0.0;
  for (int sp = 0; sp < kDwSplits; ++sp) s += part[(size_t)sp * (g.d + g.rank) + j];
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
  if (vec)
    hipLaunchKernelGGL((grad_w2t<NC, true>), dim3((n_vt + 3) / 4), dim3(kGThreads), 0, stream, g);
  else
    hipLaunchKernelGGL((grad_w2t<NC, false>), dim3((n_vt + 3) / 4), dim3(kGThreads), 0, stream, g);
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
  g.err = a.err;
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
  double* part = reinterpret_cast<double*>(a.ws + tp.off_dwp);
  hipLaunchKernelGGL(grad_dw_part, dim3((g.d + g.rank + 63) / 64, kDwSplits), dim3(kGThreads), 0,
                     stream, g, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(grad_dw_final, dim3(blocks_for((size_t)(g.d + g.rank))), dim3(kGThreads), 0,
                     stream, g, static_cast<const double*>(part));
  return hipGetLastError();
}

}  // namespace dspark

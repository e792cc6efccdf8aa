// Vocabulary-tile streaming loops shared by the draft step and the verify pass.
//
// Both compute, for a tile of 32 vocabulary entries and a tile of 32 rows
// (requests, or (request, position) pairs), the 32x32 block of
//     bias[row][v] = E[row] . W2t[v]      (E = gathered W1 rows, K = rank)
// with MFMA, and hand the fp32 block to an epilogue that fuses everything else.
// Lane l owns row 32*tile + l%32 and vocabulary entries 16*(l/32) .. +15 of the
// tile (tile_perm), matching the accumulator layout of the 32x32 MFMAs.
//
// Epilogue interface (Epi), with a compile-time register slot S in {0, 1}
// (tiles alternate between two register buffers, so nothing is copied):
//   template <int S> void prefetch(int vt)   issue the loads of tile vt into slot S
//   template <int S> void consume(const f32x16_t& acc, int vt)   fold tile vt (slot S)
//
// kKs > 0 fixes the number of MFMA K-steps at compile time (rank = kKs * K
// per MFMA); kKs = 0 reads it at run time.
#pragma once

#include <type_traits>

#include "dspark_device.h"

namespace dspark {

constexpr int kVTile = 32;
constexpr int kStreamThreads = 256;
// Workgroups of kStreamThreads that the 256 CUs of an MI355X hold at once for
// the streaming kernels (two per CU at their register footprint).
constexpr int kResidentWgs = 512;

// E fragments (MFMA B operand) of this lane's row: W1[token], K split in steps.
template <class W, int kKs = 0>
__device__ __forceinline__ void load_e_frags(typename W::frag_t (&e)[W::kMaxKs], const void* W1,
                                             int token, int rank, int V, int half) {
  token = token < 0 ? 0 : (token >= V ? V - 1 : token);  // device ids are not validated
  const typename W::store_t* row = reinterpret_cast<const typename W::store_t*>(W1) +
                                   (size_t)token * rank;
  const int nks = kKs > 0 ? kKs : rank / W::kKStep;
#pragma unroll
  for (int ks = 0; ks < W::kMaxKs; ++ks) e[ks] = (ks < nks) ? W::load(row, ks, half) : W::zero();
}

// LDS bytes of one staged W2t tile (32 rows, row stride padded by 16 bytes).
template <class W>
__host__ __device__ inline size_t stream_lds_bytes(int rank) {
  return (size_t)kVTile * (rank * sizeof(typename W::store_t) + 16);
}

// Workgroup of 4 waves: each W2t tile is loaded from HBM once (256 threads x
// up to 4 x 16 bytes, prefetched one tile ahead in registers), staged in LDS and
// multiplied by every wave with its own E fragments.  The loop is unrolled by
// two so the epilogue's prefetch buffers alternate without copies.
template <class W, int kKs, class Epi>
__device__ __forceinline__ void shared_a_stream(const void* W2t, int V, int rank, int t_begin,
                                                int t_end,
                                                const typename W::frag_t (&e)[W::kMaxKs],
                                                unsigned char* lds, Epi& epi) {
  using store_t = typename W::store_t;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int nks = kKs > 0 ? kKs : rank / W::kKStep;
  const int row_bytes = rank * (int)sizeof(store_t);
  const int rs = row_bytes + 16;
  const int cpr = row_bytes / 16;
  const int nchunks = kVTile * cpr;

  u32x4_t pre[4];
  auto fetch = [&](int vt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + j * kStreamThreads;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (c < nchunks) {
        const int row = c / cpr, ch = c - row * cpr;
        const int vv = vt * kVTile + row;
        if (vv < V)
          v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const unsigned char*>(W2t) +
                                                (size_t)vv * row_bytes + (size_t)ch * 16);
      }
      pre[j] = v;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + j * kStreamThreads;
      if (c < nchunks) {
        const int row = c / cpr, ch = c - row * cpr;
        *reinterpret_cast<u32x4_t*>(lds + row * rs + ch * 16) = pre[j];
      }
    }
  };
  const store_t* arow = reinterpret_cast<const store_t*>(lds + tile_perm(lane & 31) * rs);
  auto mma = [&]() {
    f32x16_t acc = {};
    if constexpr (kKs > 0) {
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) acc = W::mma(W::load(arow, ks, half), e[ks], acc);
    } else {
#pragma unroll
      for (int ks = 0; ks < W::kMaxKs; ++ks)
        if (ks < nks) acc = W::mma(W::load(arow, ks, half), e[ks], acc);
    }
    return acc;
  };
  auto step = [&](auto slot, int vt) {
    constexpr int S = decltype(slot)::value;
    __syncthreads();  // previous tile's LDS reads are done
    stash();
    __syncthreads();  // this tile is visible
    if (vt + 1 < t_end) {
      fetch(vt + 1);
      epi.template prefetch<1 - S>(vt + 1);
    }
    const f32x16_t acc = mma();
    epi.template consume<S>(acc, vt);
  };
  if (t_begin >= t_end) return;
  fetch(t_begin);
  epi.template prefetch<0>(t_begin);
  for (int vt = t_begin; vt < t_end; vt += 2) {
    step(std::integral_constant<int, 0>{}, vt);
    if (vt + 1 >= t_end) break;
    step(std::integral_constant<int, 1>{}, vt + 1);
  }
}

// A single wave streams tiles t_begin, t_begin + t_stride, ... < t_end; the
// W2t fragment goes straight from global memory into VGPRs.
template <class W, int kKs, class Epi>
__device__ __forceinline__ void private_a_stream(const void* W2t, int V, int rank, int t_begin,
                                                 int t_end, int t_stride,
                                                 const typename W::frag_t (&e)[W::kMaxKs],
                                                 Epi& epi) {
  using store_t = typename W::store_t;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int nks = kKs > 0 ? kKs : rank / W::kKStep;
  const int prow = tile_perm(lane & 31);
  for (int vt = t_begin; vt < t_end; vt += t_stride) {
    epi.template prefetch<0>(vt);
    const int vv = vt * kVTile + prow;
    const store_t* wrow = reinterpret_cast<const store_t*>(W2t) + (size_t)(vv < V ? vv : V - 1) * rank;
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < W::kMaxKs; ++ks) {
      if (ks < nks) {
        typename W::frag_t af = (vv < V) ? W::load(wrow, ks, half) : W::zero();
        acc = W::mma(af, e[ks], acc);
      }
    }
    epi.template consume<0>(acc, vt);
  }
}

// Load 16 consecutive fp32 values row[vb .. vb+15]; entries >= V read as 0.
// `full` (uniform across the wave) says the whole 32-wide tile lies inside the
// row; with kVec (rows 16-byte aligned, V % 4 == 0) it is read with four
// 16-byte loads.
template <bool kVec>
__device__ __forceinline__ void load16(float (&u)[16], const float* row, int vb, int V, bool full) {
  if (kVec && full) {
    const f32x4_t* p = reinterpret_cast<const f32x4_t*>(row + vb);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4_t t = __builtin_nontemporal_load(p + q);
      u[4 * q + 0] = t[0];
      u[4 * q + 1] = t[1];
      u[4 * q + 2] = t[2];
      u[4 * q + 3] = t[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = (vb + i < V) ? row[vb + i] : 0.0f;
  }
}

}  // namespace dspark

// Vocabulary-tile streaming loops shared by the draft step and the verify pass.
//
// Both compute, for a tile of 32 vocabulary entries and a tile of 32 rows
// (requests, or (request, position) pairs), the 32x32 block of
//     bias[row][v] = E[row] . W2t[v]      (E = gathered W1 rows, K = rank)
// with MFMA, and hand the fp32 block to an epilogue that fuses everything else.
// Lane l owns row 32*tile + l%32 and vocabulary entries 16*(l/32) .. +15 of the
// tile (tile_perm), matching the accumulator layout of the 32x32 MFMAs.
//
// Epilogue interface (Epi), with a compile-time register slot S in
// {0 .. kDist} (kDist = the prefetch distance chosen by the kernel):
//   static constexpr int kLoads   load instructions one prefetch issues
//   template <int S> void prefetch(int vt)
//       issue the loads of full tile vt into slot S; vt < 0 asks for the same
//       loads from an address that is always valid and cached (the start of the
//       lane's row), whose values are never used.  Prefetches are therefore
//       never conditional, which keeps the compiler's load counting exact.
//   template <int S> void consume(const f32x16_t& acc, int vt)   fold full tile vt
//   void tail(const f32x16_t& acc, int vt)
//       load (masked) and fold the last, partial tile of the vocabulary.
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
// Largest prefetch distance of the shared stream (tile i is multiplied while
// tiles i+1 .. i+kDist are in flight); buffers rotate with period kDist + 1.
constexpr int kMaxDist = 2;

template <int S>
using slot_t = std::integral_constant<int, S>;

// Workgroup barrier for LDS hand-offs.  It waits only for this wave's LDS
// operations; a __syncthreads() would also wait for every outstanding global
// load of the wave and so drain the prefetch pipeline at each tile.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until every global load this wave has issued so far has returned.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's global loads are outstanding (vmcnt(N);
// expcnt and lgkmcnt left alone).  Stating the wait explicitly keeps the
// compiler from assuming, at a loop header, that older loads are still
// pending.
template <int N>
__device__ __forceinline__ void wait_loads_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

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
__host__ __device__ inline size_t stream_tile_bytes(int rank) {
  return (size_t)kVTile * (rank * sizeof(typename W::store_t) + 16);
}
template <class W>
__host__ __device__ inline size_t stream_lds_bytes(int rank, int dist) {
  return (size_t)(dist + 1) * stream_tile_bytes<W>(rank);
}

// Workgroup of 4 waves over tiles [t_begin, t_end) of the vocabulary.  Each
// W2t tile leaves HBM once per workgroup (256 threads x up to 4 x 16 bytes),
// is staged in LDS and multiplied by every wave with its own E fragments.
//
// Iteration i, with prefetch distance D = kDist and slot S = i mod (D + 1):
//   1. issue the loads of tile i+D: W2t into registers, the epilogue's rows;
//   2. MFMA tile i from LDS slot S;
//   3. epilogue of tile i (its rows were loaded during iteration i-D);
//   4. store W2t of tile i+1 (loaded during iteration i+1-D) into LDS slot S+1;
//   5. LDS barrier.
// D = 2 hides two iterations of load latency; epilogues that stream two rows
// per entry (verification) use D = 1 to stay within the register budget.
// Only full tiles go through the pipeline; a partial last tile of the
// vocabulary is handled after it without prefetching.
// load_e(e) fills the E fragments; it runs after the first tiles' loads are
// issued, so the row gather (which depends on a token id read from memory)
// overlaps them.
template <class W, int kKs, int kDist, int kThreads = kStreamThreads, class LoadE, class Epi>
__device__ __forceinline__ void shared_a_stream(const void* W2t, int V, int rank, int t_begin,
                                                int t_end, typename W::frag_t (&e)[W::kMaxKs],
                                                LoadE&& load_e, unsigned char* lds, Epi& epi) {
  using store_t = typename W::store_t;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int nks = kKs > 0 ? kKs : rank / W::kKStep;
  const int row_bytes = rank * (int)sizeof(store_t);
  const int rs = row_bytes + 16;
  const int cpr = row_bytes / 16;
  const int nchunks = kVTile * cpr;  // 16-byte chunks per tile
  const int tile_lds = kVTile * rs;
  const unsigned char* wbase = reinterpret_cast<const unsigned char*>(W2t);
  const int t_full = min(t_end, V / kVTile);

  // Chunk j of this thread: c = tid + kThreads j.  Threads past the tile's
  // chunk count load a duplicate of the last chunk (never stored), so the
  // loads are unconditional.
  constexpr int kPer = 1024 / kThreads;  // chunks of the largest tile (32 x 512 B)
  int coff[kPer], loff[kPer];
  bool cst[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = threadIdx.x + j * kThreads;
    cst[j] = c < nchunks;
    const int cc = cst[j] ? c : nchunks - 1;
    coff[j] = cc * 16;
    const int row = cc / cpr;
    loff[j] = row * rs + (cc - row * cpr) * 16;
  }

  static_assert(kDist >= 1 && kDist <= kMaxDist, "prefetch distance");
  constexpr int P = kDist + 1;
  u32x4_t wreg[P][kPer];
  auto fetch = [&](auto slot, int vt) {
    constexpr int S = decltype(slot)::value;
    const bool real = vt < t_full;
    const unsigned char* tile = wbase + (real ? (size_t)vt * nchunks * 16 : 0);
#pragma unroll
    for (int j = 0; j < kPer; ++j) wreg[S][j] = *reinterpret_cast<const u32x4_t*>(tile + coff[j]);
    epi.template prefetch<S>(real ? vt : -1);
  };
  auto stash = [&](auto slot) {
    constexpr int S = decltype(slot)::value;
    unsigned char* dst = lds + S * tile_lds;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (cst[j]) *reinterpret_cast<u32x4_t*>(dst + loff[j]) = wreg[S][j];
  };
  const int arow_off = tile_perm(lane & 31) * rs;
  auto mma = [&](const unsigned char* slot_base) {
    const store_t* arow = reinterpret_cast<const store_t*>(slot_base + arow_off);
    f32x16_t acc = {};
    if constexpr (kKs > 0) {
      // A fragments come from LDS in groups of kG, double-buffered, so each
      // group's reads are in flight while the previous group's MFMAs run
      // (one shared register set would expose an LDS round trip per MFMA).
      constexpr int kG = 4;
      constexpr int kGroups = (kKs + kG - 1) / kG;
      typename W::frag_t af[2][kG];
#pragma unroll
      for (int q = 0; q < kG; ++q)
        if (q < kKs) af[0][q] = W::load(arow, q, half);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        if (g + 1 < kGroups) {
#pragma unroll
          for (int q = 0; q < kG; ++q)
            if ((g + 1) * kG + q < kKs) af[(g + 1) & 1][q] = W::load(arow, (g + 1) * kG + q, half);
        }
#pragma unroll
        for (int q = 0; q < kG; ++q)
          if (g * kG + q < kKs) acc = W::mma(af[g & 1][q], e[g * kG + q], acc);
      }
      // Pin that order for the scheduler (it would otherwise sink each read
      // next to its MFMA to save registers): reads of group 0, then per group
      // the next group's reads followed by this group's MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, kG, 0);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        if (g + 1 < kGroups) __builtin_amdgcn_sched_group_barrier(0x100, kG, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, kG, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < W::kMaxKs; ++ks)
        if (ks < nks) acc = W::mma(W::load(arow, ks, half), e[ks], acc);
    }
    return acc;
  };
  auto body = [&](auto slot, int vt) {
    constexpr int S = decltype(slot)::value;
    fetch(slot_t<(S + kDist) % P>{}, vt + kDist);
    // the prefetch goes out before this tile's MFMAs (the scheduler would
    // otherwise spread its loads among them, later than they can be issued)
    __builtin_amdgcn_sched_barrier(0);
    const f32x16_t acc = mma(lds + S * tile_lds);
    epi.template consume<S>(acc, vt);
    stash(slot_t<(S + 1) % P>{});
    lds_barrier();
  };

  // Prologue: only the first tile is waited for (with the E fragments, which
  // then never stay pending into the loop); with distance 2 the second tile
  // is issued just before the loop, where the loop expects one tile in flight.
  if (t_begin < t_full) fetch(slot_t<0>{}, t_begin);
  load_e(e);
  wait_all_loads();
  if (t_begin < t_full) {
    stash(slot_t<0>{});
    if constexpr (kDist == 2) fetch(slot_t<1>{}, t_begin + 1);
    lds_barrier();
    int vt = t_begin;
    for (;;) {
      body(slot_t<0>{}, vt);
      if (++vt >= t_full) break;
      body(slot_t<1>{}, vt);
      if (++vt >= t_full) break;
      if constexpr (P > 2) {
        body(slot_t<2>{}, vt);
        if (++vt >= t_full) break;
      }
    }
  }
  if (t_end > t_full) {  // the partial last tile (rows >= V read as zero)
    const int vt = t_full;
    const int valid = (V - vt * kVTile) * cpr;
    unsigned char* dst = lds;  // slot 0: every wave is past its last read (barrier above)
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = threadIdx.x + j * kThreads;
      if (c < nchunks) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (c < valid) v = *reinterpret_cast<const u32x4_t*>(wbase + (size_t)vt * nchunks * 16 + c * 16);
        *reinterpret_cast<u32x4_t*>(dst + loff[j]) = v;
      }
    }
    lds_barrier();
    const f32x16_t acc = mma(lds);
    epi.tail(acc, vt);
  }
}

// Skewed variant of the shared stream for a compile-time rank (kKs > 0): the
// MFMAs of tile i+1 are issued interleaved with the epilogue of tile i, so
// the matrix core and the LDS reads that feed it work underneath the
// epilogue's VALU instead of in front of it.  Two accumulators, two LDS
// slots, two W2t register buffers and two epilogue slots (period 2).
//
// Iteration i (S = i mod 2):
//   a. store W2t of tile i+1 (loaded during iteration i-1) into LDS slot S^1;
//   b. LDS barrier;
//   c. issue the W2t loads of tile i+2 into register buffer S;
//   d. acc_next = MFMA of tile i+1 from LDS slot S^1   } interleaved by the
//   e. epilogue of tile i with acc_cur                 } scheduler groups below
//   f. issue the epilogue's loads of tile i+2 into slot S (tile i is folded).
// A partial last tile of the vocabulary is handled after the loop.
//
// With rev the full tiles are visited from the top of the range down (tile
// t_full - 1 - (i - t_begin) at iteration i).  A caller that alternates the
// direction from one launch to the next starts each launch on the W2t tiles
// the previous one read last.
//
// SkewStream holds the stream's per-thread offsets and W2t register buffers;
// shared_a_stream_skew is its plain use.
template <class W, int kKs, int kThreads = kStreamThreads>
struct SkewStream {
  static_assert(kKs > 0, "compile-time rank");
  using store_t = typename W::store_t;
  static constexpr int kRowBytes = kKs * W::kKStep * (int)sizeof(store_t);
  static constexpr int kRs = kRowBytes + 16;
  static constexpr int kCpr = kRowBytes / 16;
  static constexpr int kChunks = kVTile * kCpr;  // 16-byte chunks per tile
  static constexpr int kPer = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "whole chunks per thread");
  static constexpr int kTileLds = kVTile * kRs;

  const unsigned char* wbase;
  int V, t_full;
  int mrev = -1;  // rev: t_begin + t_full - 1
  int coff[kPer], loff[kPer];
  u32x4_t wreg[2][kPer];

  __device__ __forceinline__ SkewStream(const void* W2t, int V_, int t_end)
      : wbase(reinterpret_cast<const unsigned char*>(W2t)), V(V_), t_full(min(t_end, V_ / kVTile)) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = threadIdx.x + j * kThreads;
      coff[j] = c * 16;
      const int row = c / kCpr;
      loff[j] = row * kRs + (c - row * kCpr) * 16;
    }
  }
  // Tile visited at iteration i (i in [t_begin, t_full)).
  __device__ __forceinline__ int tile_at(int i) const { return mrev >= 0 ? mrev - i : i; }
  template <int S>
  __device__ __forceinline__ void fetch_w(int i) {
    const unsigned char* tile = wbase + (i < t_full ? (size_t)tile_at(i) * kChunks * 16 : 0);
#pragma unroll
    for (int j = 0; j < kPer; ++j) wreg[S][j] = *reinterpret_cast<const u32x4_t*>(tile + coff[j]);
  }
  template <int S>
  __device__ __forceinline__ void stash(unsigned char* dst) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) *reinterpret_cast<u32x4_t*>(dst + loff[j]) = wreg[S][j];
  }
  // 16 A-fragment reads and MFMAs; reads run up to kAhead fragments ahead.
  __device__ __forceinline__ f32x16_t mma(const unsigned char* slot_base,
                                          const typename W::frag_t (&e)[W::kMaxKs]) const {
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const store_t* arow =
        reinterpret_cast<const store_t*>(slot_base + tile_perm(lane & 31) * kRs);
    typename W::frag_t af[kKs];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) af[ks] = W::load(arow, ks, half);
    f32x16_t acc = {};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) acc = W::mma(af[ks], e[ks], acc);
    return acc;
  }
  // The stream over tiles [t_begin, t_end).  load_e(e) fills the E fragments;
  // it runs after the first tile's loads are issued, so the row gather (which
  // depends on a token id read from memory) overlaps them.
  template <class LoadE, class Epi>
  __device__ __forceinline__ void run(int t_begin, int t_end, typename W::frag_t (&e)[W::kMaxKs],
                                      LoadE&& load_e, unsigned char* lds, Epi& epi, bool rev) {
    if (rev) mrev = t_begin + t_full - 1;
    // Scheduler groups for one iteration body: the first kAhead A reads, then
    // per MFMA one more read and a share of the epilogue's VALU work.
    constexpr int kAhead = 4;
    constexpr int kValuPerMfma = 24;
    auto pin = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 1);
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (ks + kAhead < kKs) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 1);
      }
    };
    f32x16_t acc_cur = {};
    auto body = [&](auto slot, int vt) {
      constexpr int S = decltype(slot)::value;
      // Everything but the epilogue loads of tile i+1 has arrived: the W2t of
      // tile i+1 (stored next) and the epilogue rows of tile i.
      wait_loads_le<Epi::kLoads>();
      stash<S ^ 1>(lds + (S ^ 1) * kTileLds);
      lds_barrier();
      fetch_w<S>(vt + 2);
      const f32x16_t acc_next = mma(lds + (S ^ 1) * kTileLds, e);
      epi.template consume<S>(acc_cur, tile_at(vt));
      epi.template prefetch<S>(vt + 2 < t_full ? tile_at(vt + 2) : -1);
      pin();
      acc_cur = acc_next;
    };

    if (t_begin < t_full) {
      fetch_w<0>(t_begin);
      epi.template prefetch<0>(tile_at(t_begin));
    }
    load_e(e);
    wait_all_loads();  // the E fragments never stay pending into the loop
    if (t_begin < t_full) {
      stash<0>(lds);
      fetch_w<1>(t_begin + 1);
      epi.template prefetch<1>(t_begin + 1 < t_full ? tile_at(t_begin + 1) : -1);
      lds_barrier();
      acc_cur = mma(lds, e);
      int vt = t_begin;
      for (;;) {
        body(slot_t<0>{}, vt);
        if (++vt >= t_full) break;
        body(slot_t<1>{}, vt);
        if (++vt >= t_full) break;
      }
    }
    if (t_end > t_full) {  // the partial last tile (rows >= V read as zero)
      const int vt = t_full;
      const int valid = (V - vt * kVTile) * kCpr;
      lds_barrier();  // every wave is past its last LDS read
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int c = threadIdx.x + j * kThreads;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (c < valid) v = *reinterpret_cast<const u32x4_t*>(wbase + (size_t)vt * kChunks * 16 + c * 16);
        *reinterpret_cast<u32x4_t*>(lds + loff[j]) = v;
      }
      lds_barrier();
      const f32x16_t acc = mma(lds, e);
      epi.tail(acc, vt);
    }
  }
};

template <class W, int kKs, int kThreads = kStreamThreads, class LoadE, class Epi>
__device__ __forceinline__ void shared_a_stream_skew(const void* W2t, int V, int t_begin,
                                                     int t_end,
                                                     typename W::frag_t (&e)[W::kMaxKs],
                                                     LoadE&& load_e, unsigned char* lds,
                                                     Epi& epi, bool rev = false) {
  SkewStream<W, kKs, kThreads> ss(W2t, V, t_end);
  ss.run(t_begin, t_end, e, load_e, lds, epi, rev);
}

// ---------------------------------------------------------------------------
// Rows of a vocabulary tile in fp32 (one wave: 32 rows x 32 entries = 4 KB per
// array), read from global memory as whole 128-byte lines -- load instruction
// q, lane l: row 8q + l/8, entries 4 (l%8) .. +3 -- and handed to the MFMA lane
// layout (row l%32, entries 16 (l/32) .. +15) through a padded LDS patch of the
// wave (row stride 36 floats, so both the stores and the 16-byte reads are
// free of bank conflicts).  The lane layout would touch 32 lines per load
// instruction; whole lines are what the memory system serves best.
// kArrays row sets share the row offsets (e.g. U and the target logits).
// ---------------------------------------------------------------------------
constexpr int kPatchRowFloats = 36;
constexpr int kPatchFloats = kVTile * kPatchRowFloats;  // per wave (4.5 KB)

template <int kArrays, int kSlots>
struct RowTiles {
  const float* base[kArrays];  // vocabulary entry 0 of the row of offset 0
  size_t off[4];               // floats from base to this lane's (row, entry) of load q
  f32x4_t g[kSlots][kArrays][4];

  // row_off(j): offset in floats of the wave's row j (0..31) from base.
  template <class RowOff>
  __device__ __forceinline__ void init(RowOff&& row_off) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < 4; ++q) off[q] = row_off(8 * q + (l >> 3)) + 4 * (l & 7);
  }
  // Issue the loads of tile vt (vt < 0: the same loads from tile 0, unused).
  template <int S>
  __device__ __forceinline__ void load(int vt) {
    const int col = vt < 0 ? 0 : vt * kVTile;
#pragma unroll
    for (int a = 0; a < kArrays; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        g[S][a][q] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(base[a] + off[q] + col));
  }
  // Slot S to lane layout: out[a][i] = row l%32, entry 16 (l/32) + i.  The
  // arrays pass through the same patch one after another (a wave's LDS
  // operations complete in order, so a read returns before the next store).
  template <int S>
  __device__ __forceinline__ void to_lanes(float* patch, float (&out)[kArrays][16]) {
    const int l = threadIdx.x & 63;
    float* wr = patch + (l >> 3) * kPatchRowFloats + 4 * (l & 7);
    const float* rd = patch + (l & 31) * kPatchRowFloats + 16 * (l >> 5);
#pragma unroll
    for (int a = 0; a < kArrays; ++a) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t*>(wr + 8 * q * kPatchRowFloats) = g[S][a][q];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(rd + 4 * c);
        out[a][4 * c + 0] = v[0];
        out[a][4 * c + 1] = v[1];
        out[a][4 * c + 2] = v[2];
        out[a][4 * c + 3] = v[3];
      }
    }
  }
};

// E fragments (bf16, rank = 16 kKs with kKs a multiple of 4) of the wave's 32
// rows, gathered as whole lines.  The fragment layout reads 16 bytes from 32
// different rows per load instruction; instead each 128-byte quarter Q of the
// rows is loaded with 8 lanes per row (instruction p: row 8p + l/8, chunk
// l%8), stored into the wave's LDS patch and read back in fragment order
// (lane l: row l%32, chunks 2 ks + l/32 for the four ks of the quarter).
// `token` is this lane's row id (already clamped to [0, V)); the patch must be
// free (it is used in turn by the quarters, in order within the wave).
template <int kKs>
__device__ __forceinline__ void load_e_frags_lines(bf16x8_t (&e)[WBf16::kMaxKs],
                                                   const uint16_t* W1, int token, float* patch) {
  static_assert(kKs % 4 == 0 && kKs <= WBf16::kMaxKs, "whole 128-byte quarters");
  constexpr int kRank = kKs * WBf16::kKStep;
  constexpr int kQuarters = kKs / 4;
  constexpr int kStride = kPatchRowFloats * 4;  // bytes per patch row
  const int l = threadIdx.x & 63, h = l >> 5;
  int tq[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) tq[p] = __shfl(token, 8 * p + (l >> 3));
  u32x4_t raw[kQuarters][4];
#pragma unroll
  for (int Q = 0; Q < kQuarters; ++Q)
#pragma unroll
    for (int p = 0; p < 4; ++p)
      raw[Q][p] = *reinterpret_cast<const u32x4_t*>(W1 + (size_t)tq[p] * kRank +
                                                    (8 * Q + (l & 7)) * 8);
  unsigned char* pb = reinterpret_cast<unsigned char*>(patch);
#pragma unroll
  for (int Q = 0; Q < kQuarters; ++Q) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      *reinterpret_cast<u32x4_t*>(pb + (8 * p + (l >> 3)) * kStride + (l & 7) * 16) = raw[Q][p];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      e[4 * Q + i] =
          *reinterpret_cast<const bf16x8_t*>(pb + (l & 31) * kStride + (2 * i + h) * 16);
  }
#pragma unroll
  for (int ks = kKs; ks < WBf16::kMaxKs; ++ks) e[ks] = WBf16::zero();
}

// Load 16 consecutive fp32 values row[vb .. vb+15] of a full tile; with kVec
// (rows 16-byte aligned) as four 16-byte non-temporal loads.
template <bool kVec>
__device__ __forceinline__ void load16(float (&u)[16], const float* row, int vb) {
  if constexpr (kVec) {
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
    for (int i = 0; i < 16; ++i) u[i] = row[vb + i];
  }
}

// Masked variant for the partial last tile: entries >= V read as `fill`.
__device__ __forceinline__ void load16_masked(float (&u)[16], const float* row, int vb, int V,
                                              float fill) {
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = (vb + i < V) ? row[vb + i] : fill;
}

}  // namespace dspark

// Internal interface between the C-ABI host layer (dspark_api.hip) and the
// kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "draft_step.h"

namespace dspark {

// RNN head (rnn_head.hip); bf16 weights, rank % 32 == 0, d % 16 == 0.
constexpr int kProjSplit = 4;  // K quarters of the input projection (partial sums in P)
struct RnnArgs {
  int R, V, rank, d, gamma;
  const uint16_t* W1;
  const uint16_t* W_ih;   // [3 rank][rank + d]
  const uint16_t* W_hh;   // [3 rank][rank]
  const float* b_ih;      // [3 rank]
  const float* b_hh;
  const uint16_t* h;      // [R][gamma][d]
  const int32_t* x;       // [R][gamma + 1] (column 0: the anchor)
  const unsigned long long* best;  // draft steps' winner words [gamma][R]
  float* P;               // input projections, kProjSplit partials [kProjSplit][R * gamma][3 rank]
  float* Pk;              // their sums, step-major [gamma][R][3 rank]
  uint16_t* rows_out;     // optional: bf16(s_k) of every position [R][gamma][rank]
  uint16_t* E;            // bf16(s_k) [R][rank], the step's bias rows
  uint32_t* err;  // token-error word (checked_token)
};
hipError_t launch_rnn_input_proj(const RnnArgs& a, hipStream_t stream);
hipError_t launch_rnn_state_step(const RnnArgs& a, int k, const float* s_prev, float* s_next,
                                 hipStream_t stream);

struct ConfArgs {
  int R, gamma, d, rank, V;
  bool bf16;
  const void* h;
  const void* W1;
  const int32_t* x;
  const float* w;
  float* c;
  float* a;
  uint32_t* err;  // token-error word (checked_token)
};
hipError_t launch_confidence(const ConfArgs& a, hipStream_t stream);

// Prefix scheduler (see schedule.hip): one launch over the grid; the last
// workgroup to finish applies the early stop.  The workspace carries, by
// sorted position, the prefix sums G and the candidates' requests, and the
// finishing counters (zero before the first call; every call leaves them zero).
struct SchedRankArgs {
  int R, gamma, N;      // N = R * gamma
  bool async;           // asynchronous variant: a = a_lag (budget), a_cur (selection)
  const float* a;
  const float* a_cur;
  const double* sps;
  int32_t* ell;
  int32_t* budget;
  double* theta;
  // workspace (sched_ws_layout)
  int n_wgs;            // workgroups per key array
  unsigned* done;       // finishing counters
  int32_t* req;         // [N] request of the candidate at each sorted position (a_cur when async)
  double* gpos;         // [N + 1] G_b, the exact sum of q over the first b candidates
                        // (of a_lag when async)
};
size_t sched_ws_bytes(int N);
void sched_ws_layout(SchedRankArgs& a, void* ws);
hipError_t launch_schedule_ranked(const SchedRankArgs& a, hipStream_t stream);

// Verification (see verify.hip).
struct VerifyPlan {
  int n_rows;       // R * gamma
  int n_rtiles;     // ceil(n_rows / 32)
  int n_groups;     // c* pass: groups of 4 row tiles
  int n_slabs;      // c* pass: vocabulary slabs per group
  int s_groups;     // sampling pass: groups of 128 requests
  int s_slabs;      // sampling pass: vocabulary slabs per group
  int n_vtiles;
  int lse_chunks;   // vocabulary chunks per row in the target normaliser pass
  int fuse_sample;  // 1: the c* pass also runs the sampling race (no row tile meets > 2 requests)
  size_t off_lse_t, off_tv, off_best, off_srow, off_skind, off_lsepart, ws_bytes;
};

struct VerifyArgs {
  int R, V, rank, gamma;
  bool bf16, greedy;
  const void* W1;
  const void* W2t;
  const float* U;
  const float* target;
  const int32_t* x;
  const void* E_rows;      // RNN head: bias rows per (request, position) [R][gamma][rank]; null: W1[x]
  const float* lse_d;
  const float* p_d_x;
  const int32_t* ell;
  float kscale;
  uint64_t seed;
  float* c_star;
  int32_t* n_accept;
  int32_t* next_token;
  int32_t* tau;
  float* tau_mean;
  unsigned char* ws;
  uint32_t* err;  // token-error word (checked_token)
};

VerifyPlan plan_verify(int R, int V, int gamma);
hipError_t launch_verify(const VerifyArgs& a, const VerifyPlan& plan, hipStream_t stream);

// Training losses (verify.hip): the verification workspace followed by these.
struct TrainPlan {
  size_t off_dlse;  // draft-normaliser records [n_slabs][3][n_rows]
  size_t off_lse_d; // draft log-normalisers (natural log) [n_rows]
  size_t off_ce;    // -log p_d(x*) [n_rows]
  size_t off_c;     // confidence c_k [n_rows]
  size_t off_surv;  // survival products of the confidence head (unused) [n_rows]
  size_t off_mu;    // sum_v sign(p_d - p_t) p_d, signed 2^-40 fixed point [n_rows] (u64)
  size_t off_dl;    // dL / d(confidence logit) [n_rows]
  size_t ws_bytes;  // end of the forward workspace
  // gradients (train_grad.hip), after the forward workspace
  int n_pad;        // rows rounded up to 128
  int vp;           // vocabulary rounded up to 64
  int e_groups;     // 128-row groups of the dE contraction
  int e_slabs;      // vocabulary slabs of the dE contraction
  size_t off_w2;    // W2t transposed, bf16, chunk-major [vp / 64][rank][64]
  size_t off_et;    // gathered W1 rows transposed, bf16, chunk-major [n_pad / 64][rank][64]
  size_t off_dep;   // dE slab partials [e_slabs][n_pad][rank]
  size_t off_de;    // dE [n_rows][rank]
  size_t off_dwp;   // dw partial sums over row ranges, fp64 [16][d + rank]
  size_t ws_grad_bytes;
};

struct TrainArgs {
  float lambda, alpha_ce, alpha_tv, alpha_conf;
  float inv_t;     // 1 / T
  const float* c;  // confidence c_k [n_rows], computed before the assembly
  float* terms;    // [n_rows][4]: ce, tv, conf, c
  double* sums;    // [4]: sum_k w_k ce, sum w_k tv, sum w_k conf, total
  // gradients (all null for the losses alone); bf16 weights and h only
  int d;
  const void* h;
  const float* w;
  float* dU;       // [n_rows][V]
  float* dW1;      // [V][rank]
  float* dW2t;     // [V][rank]
  float* dh;       // [n_rows][d]
  float* dw;       // [d + rank]
};

TrainPlan plan_train(int R, int V, int rank, int d, int gamma);
// Losses; with ta.dU set also every gradient (then ws holds ws_grad_bytes).
hipError_t launch_train(const VerifyArgs& a, const TrainArgs& ta, const VerifyPlan& plan,
                        const TrainPlan& tp, hipStream_t stream);
// The gradients behind the logits, after dU and dl are in place (train_grad.hip).
hipError_t launch_train_grad_rest(const VerifyArgs& a, const TrainArgs& ta, const VerifyPlan& plan,
                                  const TrainPlan& tp, hipStream_t stream);

}  // namespace dspark

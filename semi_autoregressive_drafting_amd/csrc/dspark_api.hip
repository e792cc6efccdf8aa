// C ABI of the DSpark drafting hot path (declared in include/dspark.h).
//
// Every entry point validates its arguments on the host before touching HIP,
// so each error status can be produced on a machine without a GPU.  The
// library never allocates, frees or synchronises; it only enqueues kernels on
// the caller's stream.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "dspark.h"
#include "dspark_kernels.h"

using namespace dspark;

// The workspace of dspark_draft_block_noalloc: one copy per GPU in the code
// object, held until the process ends.  22 MiB holds the draft workspace of
// every shape the ABI accepts (the largest, R = 512 and gamma = 16, needs
// 22,020,096 bytes).  In host code the name stands for a host-side symbol, not
// a device address: the device address comes from hipGetSymbolAddress, once
// per device (scratch_address below), and only that address is passed on.
constexpr size_t kNoAllocScratchBytes = (size_t)22 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The token-error word of this GPU: every kernel that gathers a W1 row by a
// token id read from device memory stores 1 here when the id lies outside
// [0, V).  Kernels receive its device address (token_error_address); the host
// reads and clears it through dspark_token_errors.
static __device__ __align__(256) uint32_t token_error[64];

namespace {

constexpr int kMaxR = 512;
constexpr int kMaxGamma = 16;
constexpr int kMaxV = 1 << 24;
constexpr int kMaxD = 65536;
constexpr int kMaxSched = 8192;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

dspark_status check_rank(int dt, int rank) {
  if (dt == DSPARK_BF16) {
    if (rank < 16 || rank > 256 || rank % 16 != 0) return DSPARK_ERR_SHAPE;
  } else if (dt == DSPARK_F32) {
    if (rank < 4 || rank > 128 || rank % 4 != 0) return DSPARK_ERR_SHAPE;
  } else {
    return DSPARK_ERR_DTYPE;
  }
  return DSPARK_OK;
}

bool bad_temperature(float T) { return !(T >= 0.0f) || isinf(T); }

float kscale_of(float T) { return T > 0.0f ? (float)(1.4426950408889634 / (double)T) : 1.0f; }

// RNN head workspace after the draft step's: input-projection partials and
// their step-major sums, the two state buffers and the bf16 state rows.
struct RnnPlan {
  size_t off_P, off_Pk, off_S0, off_S1, off_E, ws_bytes;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

RnnPlan plan_rnn(int R, int V, int rank, int gamma) {
  RnnPlan q{};
  size_t off = al256(plan_draft_step(R, V, gamma).ws_bytes);
  q.off_P = off;
  off = al256(off + (size_t)kProjSplit * R * gamma * 3 * rank * 4);
  q.off_Pk = off;
  off = al256(off + (size_t)R * gamma * 3 * rank * 4);
  q.off_S0 = off;
  off = al256(off + (size_t)R * rank * 4);
  q.off_S1 = off;
  off = al256(off + (size_t)R * rank * 4);
  q.off_E = off;
  off = al256(off + (size_t)R * rank * 2);
  q.ws_bytes = off;
  return q;
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept per device afterwards.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

dspark_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSPARK_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return DSPARK_ERR_LAUNCH;
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return DSPARK_OK;
}

std::mutex g_err_mu;
uint32_t* g_err_addr[kMaxDevices] = {};

// Device address of the token-error word on the current device (looked up
// once per device).
dspark_status token_error_address(uint32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSPARK_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_err_mu);
  if (g_err_addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(token_error)) != hipSuccess || ptr == nullptr)
      return DSPARK_ERR_LAUNCH;
    g_err_addr[dev] = static_cast<uint32_t*>(ptr);
  }
  *out = g_err_addr[dev];
  return DSPARK_OK;
}

}  // namespace

extern "C" {

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_NULL: return "required pointer is NULL";
    case DSPARK_ERR_SHAPE: return "size out of range, inconsistent or misaligned";
    case DSPARK_ERR_DTYPE: return "unknown element type";
    case DSPARK_ERR_VALUE: return "bad scalar argument";
    case DSPARK_ERR_WORKSPACE: return "workspace missing or too small";
    case DSPARK_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t dspark_workspace_bytes(int op, int R, int V, int rank, int gamma) {
  if (R < 1 || R > kMaxR || V < 2 || V > kMaxV || gamma < 1 || gamma > kMaxGamma) return 0;
  switch (op) {
    case DSPARK_OP_DRAFT_STEP: return plan_draft_step(R, V, gamma).ws_bytes;
    case DSPARK_OP_SCHEDULE:
      if (R * gamma > kMaxSched) return 0;
      return sched_ws_bytes(R * gamma);
    case DSPARK_OP_VERIFY: return plan_verify(R, V, gamma).ws_bytes;
    case DSPARK_OP_TRAIN_LOSS: return plan_train(R, V, rank < 1 ? 1 : rank, 1, gamma).ws_bytes;
    case DSPARK_OP_DRAFT_RNN:
      if (rank < 32 || rank > 256 || rank % 32 != 0) return 0;
      return plan_rnn(R, V, rank, gamma).ws_bytes;
    case DSPARK_OP_TRAIN_GRAD:
      if (rank < 32 || rank > 256 || rank % 32 != 0) return 0;
      // sized for the largest d (the dw partials sit at the end of the layout)
      return plan_train(R, V, rank, kMaxD, gamma).ws_grad_bytes;
    default: return 0;
  }
}

}  // extern "C"

namespace {

// Validation shared by dspark_draft_step and dspark_draft_block (k = 0 means
// "any step"); fills `args` for step 1 on success.
dspark_status check_draft(int R, int V, int rank, int d, int gamma, int k, int dt, const void* W1,
                          const void* W2t, const float* U, const void* h, const float* w,
                          float temperature, uint64_t seed, int32_t* x, float* p, float* lse,
                          float* c, float* a, float* z_debug, void* ws, size_t ws_bytes,
                          StepArgs& args, StepPlan& plan) {
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (!W1 || !W2t || !U || !x || !p || !lse) return DSPARK_ERR_NULL;
  if ((h == nullptr) != (w == nullptr)) return DSPARK_ERR_NULL;
  if (h && (!c || !a)) return DSPARK_ERR_NULL;
  if (R < 1 || R > kMaxR || V < 2 || V > kMaxV || gamma < 1 || gamma > kMaxGamma)
    return DSPARK_ERR_SHAPE;
  dspark_status s = check_rank(dt, rank);
  if (s != DSPARK_OK) return s;
  if (h && (d < 1 || d > kMaxD)) return DSPARK_ERR_SHAPE;
  if (!aligned16(W1) || !aligned16(W2t) || ((V % 4) == 0 && !aligned16(U)))
    return DSPARK_ERR_SHAPE;
  if (k < 0 || k > gamma || bad_temperature(temperature)) return DSPARK_ERR_VALUE;
  plan = plan_draft_step(R, V, gamma);
  if (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws)) return DSPARK_ERR_WORKSPACE;

  args = StepArgs{};
  args.R = R;
  args.V = V;
  args.rank = rank;
  args.d = d;
  args.gamma = gamma;
  args.k = k < 1 ? 1 : k;
  args.bf16 = dt == DSPARK_BF16;
  args.greedy = temperature == 0.0f;
  args.W1 = W1;
  args.W2t = W2t;
  args.U = U;
  args.h = h;
  args.w = w;
  args.kscale = kscale_of(temperature);
  args.seed = seed;
  args.x = x;
  args.p = p;
  args.lse = lse;
  args.c = c;
  args.a = a;
  args.z_debug = z_debug;
  args.rec = static_cast<float*>(ws);
  args.rec_step_f = plan.rec_step / sizeof(float);
  args.best = reinterpret_cast<unsigned long long*>(static_cast<unsigned char*>(ws) + plan.off_best);
  args.prev_from_best = false;
  args.n_vtiles = plan.n_vtiles;
  args.n_slabs = plan.n_slabs;
  args.n_groups = plan.n_groups;
  return DSPARK_OK;
}

dspark_status verify_common(int R, int V, int rank, int gamma, int dt, const void* W1,
                                   const void* W2t, const float* U, const float* target,
                                   const int32_t* x, const void* rows, const float* lse_d,
                                   const float* p_d_x, const int32_t* ell, float temperature,
                                   uint64_t seed, float* c_star, int32_t* n_accept,
                                   int32_t* next_token, int32_t* tau, float* tau_mean, void* ws,
                                   size_t ws_bytes, dspark_stream_t stream) {
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (!W1 || !W2t || !U || !target || !x || !lse_d || !p_d_x || !ell || !c_star || !n_accept ||
      !next_token || !tau || !tau_mean)
    return DSPARK_ERR_NULL;
  if (R < 1 || R > kMaxR || V < 2 || V > kMaxV || gamma < 1 || gamma > kMaxGamma)
    return DSPARK_ERR_SHAPE;
  dspark_status s = check_rank(dt, rank);
  if (s != DSPARK_OK) return s;
  if (!aligned16(W1) || !aligned16(W2t) || (rows && !aligned16(rows)) ||
      ((V % 4) == 0 && (!aligned16(U) || !aligned16(target))))
    return DSPARK_ERR_SHAPE;
  if (bad_temperature(temperature)) return DSPARK_ERR_VALUE;
  const VerifyPlan plan = plan_verify(R, V, gamma);
  if (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws)) return DSPARK_ERR_WORKSPACE;

  VerifyArgs args{};
  args.R = R;
  args.V = V;
  args.rank = rank;
  args.gamma = gamma;
  args.bf16 = dt == DSPARK_BF16;
  args.greedy = temperature == 0.0f;
  args.W1 = W1;
  args.W2t = W2t;
  args.U = U;
  args.target = target;
  args.x = x;
  args.E_rows = rows;
  args.lse_d = lse_d;
  args.p_d_x = p_d_x;
  args.ell = ell;
  args.kscale = kscale_of(temperature);
  args.seed = seed;
  args.c_star = c_star;
  args.n_accept = n_accept;
  args.next_token = next_token;
  args.tau = tau;
  args.tau_mean = tau_mean;
  args.ws = static_cast<unsigned char*>(ws);
  if (token_error_address(&args.err) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  if (launch_verify(args, plan, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

// Validation shared by the two schedulers (pointers were checked by the caller).
dspark_status check_schedule(int R, int gamma, int sps_len, const void* ws, size_t ws_bytes) {
  if (R < 1 || R > kMaxR || gamma < 1 || gamma > kMaxGamma || R * gamma > kMaxSched)
    return DSPARK_ERR_SHAPE;
  if (sps_len < R * (1 + gamma) + 1) return DSPARK_ERR_SHAPE;
  if (!ws || ws_bytes < sched_ws_bytes(R * gamma) || (reinterpret_cast<uintptr_t>(ws) & 15u))
    return DSPARK_ERR_WORKSPACE;
  return DSPARK_OK;
}

}  // namespace

extern "C" {

dspark_status dspark_draft_step(int R, int V, int rank, int d, int gamma, int k, int dt,
                                const void* W1, const void* W2t, const float* U,
                                const void* h, const float* w, float temperature,
                                uint64_t seed, int32_t* x, float* p, float* lse, float* c,
                                float* a, float* z_debug, void* ws, size_t ws_bytes,
                                dspark_stream_t stream) {
  if (k < 1) return DSPARK_ERR_VALUE;
  StepArgs args;
  StepPlan plan;
  const dspark_status s = check_draft(R, V, rank, d, gamma, k, dt, W1, W2t, U, h, w, temperature,
                                      seed, x, p, lse, c, a, z_debug, ws, ws_bytes, args, plan);
  if (s != DSPARK_OK) return s;
  if (token_error_address(&args.err) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (launch_draft_step(args, plan, st) != hipSuccess ||
      launch_draft_finalize(args, plan, k, 1, st) != hipSuccess)
    return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_draft_block_phases(int R, int V, int rank, int d, int gamma, int dt,
                                        const void* W1, const void* W2t, const float* U,
                                        const void* h, const float* w, float temperature,
                                        uint64_t seed, int32_t* x, float* p, float* lse,
                                        float* c, float* a, void* ws, size_t ws_bytes,
                                        int phases, dspark_stream_t stream) {
  if (phases < 1 || phases > (DSPARK_PHASE_STEPS | DSPARK_PHASE_MERGE)) return DSPARK_ERR_VALUE;
  StepArgs args;
  StepPlan plan;
  const dspark_status s = check_draft(R, V, rank, d, gamma, 0, dt, W1, W2t, U, h, w, temperature,
                                      seed, x, p, lse, c, a, nullptr, ws, ws_bytes, args, plan);
  if (s != DSPARK_OK) return s;
  if (token_error_address(&args.err) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (phases & DSPARK_PHASE_STEPS) {
    if (launch_draft_steps(args, plan, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  }
  if (phases & DSPARK_PHASE_MERGE) {
    args.k = 1;
    args.prev_from_best = true;  // x_{k-1} of positions 2..gamma from the winner words
    if (launch_draft_finalize(args, plan, 1, gamma, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  }
  return DSPARK_OK;
}

dspark_status dspark_draft_block_noalloc(int R, int V, int rank, int d, int gamma, int dt,
                                         const void* W1, const void* W2t, const float* U,
                                         const void* h, const float* w, float temperature,
                                         uint64_t seed, int32_t* x, float* p, float* lse,
                                         float* c, float* a, dspark_stream_t stream) {
  // validate first (no HIP call yet): the workspace stand-in is only checked
  // for its size, which must fit the static scratch
  StepArgs args;
  StepPlan plan;
  void* const stand_in = reinterpret_cast<void*>((uintptr_t)256);
  const dspark_status s = check_draft(R, V, rank, d, gamma, 0, dt, W1, W2t, U, h, w, temperature,
                                      seed, x, p, lse, c, a, nullptr, stand_in,
                                      kNoAllocScratchBytes, args, plan);
  if (s != DSPARK_OK) return s;
  void* ws = nullptr;
  const dspark_status t = scratch_address(&ws);
  if (t != DSPARK_OK) return t;
  if (token_error_address(&args.err) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  args.rec = static_cast<float*>(ws);
  args.best =
      reinterpret_cast<unsigned long long*>(static_cast<unsigned char*>(ws) + plan.off_best);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the scratch keeps whatever the previous call on this GPU left there
  if (launch_clear_winners(args, plan, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  if (launch_draft_steps(args, plan, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  args.k = 1;
  args.prev_from_best = true;
  if (launch_draft_finalize(args, plan, 1, gamma, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_draft_block(int R, int V, int rank, int d, int gamma, int dt,
                                 const void* W1, const void* W2t, const float* U,
                                 const void* h, const float* w, float temperature,
                                 uint64_t seed, int32_t* x, float* p, float* lse, float* c,
                                 float* a, void* ws, size_t ws_bytes, dspark_stream_t stream) {
  return dspark_draft_block_phases(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, temperature, seed,
                                   x, p, lse, c, a, ws, ws_bytes,
                                   DSPARK_PHASE_STEPS | DSPARK_PHASE_MERGE, stream);
}

dspark_status dspark_draft_block_rnn(int R, int V, int rank, int d, int gamma, int dt,
                                     const void* W1, const void* W2t, const float* U,
                                     const void* h, const float* w, const void* W_ih,
                                     const void* W_hh, const float* b_ih, const float* b_hh,
                                     float temperature, uint64_t seed, int32_t* x, float* p,
                                     float* lse, float* c, float* a, float* state, void* rows,
                                     void* ws, size_t ws_bytes, dspark_stream_t stream) {
  if (!h || !w || !W_ih || !W_hh || !b_ih || !b_hh || !state) return DSPARK_ERR_NULL;
  if (dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;  // the state rows are bf16 like W1
  if (rank % 32 != 0 || d % 16 != 0) return DSPARK_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(W_ih) || !aligned16(W_hh) || !aligned16(state))
    return DSPARK_ERR_SHAPE;
  StepArgs args;
  StepPlan plan;
  const dspark_status s = check_draft(R, V, rank, d, gamma, 0, dt, W1, W2t, U, h, w, temperature,
                                      seed, x, p, lse, c, a, nullptr, ws, ws_bytes, args, plan);
  if (s != DSPARK_OK) return s;
  const RnnPlan rp = plan_rnn(R, V, rank, gamma);
  if (ws_bytes < rp.ws_bytes) return DSPARK_ERR_WORKSPACE;
  if (token_error_address(&args.err) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  RnnArgs ra{};
  ra.R = R;
  ra.V = V;
  ra.rank = rank;
  ra.d = d;
  ra.gamma = gamma;
  ra.W1 = static_cast<const uint16_t*>(W1);
  ra.W_ih = static_cast<const uint16_t*>(W_ih);
  ra.W_hh = static_cast<const uint16_t*>(W_hh);
  ra.b_ih = b_ih;
  ra.b_hh = b_hh;
  ra.h = static_cast<const uint16_t*>(h);
  ra.x = x;
  ra.err = args.err;
  ra.best = args.best;
  ra.P = reinterpret_cast<float*>(wsb + rp.off_P);
  ra.Pk = reinterpret_cast<float*>(wsb + rp.off_Pk);
  ra.E = reinterpret_cast<uint16_t*>(wsb + rp.off_E);
  ra.rows_out = static_cast<uint16_t*>(rows);
  float* S[2] = {reinterpret_cast<float*>(wsb + rp.off_S0), reinterpret_cast<float*>(wsb + rp.off_S1)};
  if (launch_rnn_input_proj(ra, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  args.E_rows = ra.E;
  for (int k = 1; k <= gamma; ++k) {
    float* next = k == gamma ? state : S[k & 1];
    if (launch_rnn_state_step(ra, k, S[(k - 1) & 1], next, st) != hipSuccess)
      return DSPARK_ERR_LAUNCH;
    args.k = k;
    args.prev_from_best = k > 1;
    if (launch_draft_step(args, plan, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  }
  args.k = 1;
  args.prev_from_best = true;
  if (launch_draft_finalize(args, plan, 1, gamma, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_confidence(int R, int gamma, int d, int rank, int V, int dt,
                                const void* h, const void* W1, const int32_t* x,
                                const float* w, float* c, float* a, dspark_stream_t stream) {
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (!h || !W1 || !x || !w || !c || !a) return DSPARK_ERR_NULL;
  if (R < 1 || R > kMaxR || gamma < 1 || gamma > kMaxGamma || d < 1 || d > kMaxD || V < 2 ||
      V > kMaxV)
    return DSPARK_ERR_SHAPE;
  dspark_status s = check_rank(dt, rank);
  if (s != DSPARK_OK) return s;
  ConfArgs args{R, gamma, d, rank, V, dt == DSPARK_BF16, h, W1, x, w, c, a, nullptr};
  if (token_error_address(&args.err) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  if (launch_confidence(args, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_schedule(int R, int gamma, const float* a, const double* sps, int sps_len,
                              int32_t* ell, int32_t* budget, double* theta, void* ws,
                              size_t ws_bytes, dspark_stream_t stream) {
  if (!a || !sps || !ell || !budget) return DSPARK_ERR_NULL;
  const dspark_status s = check_schedule(R, gamma, sps_len, ws, ws_bytes);
  if (s != DSPARK_OK) return s;
  SchedRankArgs args{};
  args.R = R;
  args.gamma = gamma;
  args.N = R * gamma;
  args.async = false;
  args.a = a;
  args.sps = sps;
  args.ell = ell;
  args.budget = budget;
  args.theta = theta;
  sched_ws_layout(args, ws);
  if (launch_schedule_ranked(args, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_schedule_async(int R, int gamma, const float* a_lag, const float* a_cur,
                                    const double* sps, int sps_len, int32_t* ell,
                                    int32_t* budget, double* theta, void* ws, size_t ws_bytes,
                                    dspark_stream_t stream) {
  if (!a_lag || !a_cur || !sps || !ell || !budget) return DSPARK_ERR_NULL;
  const dspark_status s = check_schedule(R, gamma, sps_len, ws, ws_bytes);
  if (s != DSPARK_OK) return s;
  SchedRankArgs args{};
  args.R = R;
  args.gamma = gamma;
  args.N = R * gamma;
  args.async = true;
  args.a = a_lag;
  args.a_cur = a_cur;
  args.sps = sps;
  args.ell = ell;
  args.budget = budget;
  args.theta = theta;
  sched_ws_layout(args, ws);
  if (launch_schedule_ranked(args, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

dspark_status dspark_verify(int R, int V, int rank, int gamma, int dt, const void* W1,
                            const void* W2t, const float* U, const float* target,
                            const int32_t* x, const float* lse_d, const float* p_d_x,
                            const int32_t* ell, float temperature, uint64_t seed,
                            float* c_star, int32_t* n_accept, int32_t* next_token,
                            int32_t* tau, float* tau_mean, void* ws, size_t ws_bytes,
                            dspark_stream_t stream) {
  return verify_common(R, V, rank, gamma, dt, W1, W2t, U, target, x, nullptr, lse_d, p_d_x, ell,
                       temperature, seed, c_star, n_accept, next_token, tau, tau_mean, ws,
                       ws_bytes, stream);
}

dspark_status dspark_verify_rnn(int R, int V, int rank, int gamma, int dt, const void* W1,
                                const void* W2t, const float* U, const float* target,
                                const int32_t* x, const void* rows, const float* lse_d,
                                const float* p_d_x, const int32_t* ell, float temperature,
                                uint64_t seed, float* c_star, int32_t* n_accept,
                                int32_t* next_token, int32_t* tau, float* tau_mean, void* ws,
                                size_t ws_bytes, dspark_stream_t stream) {
  if (!rows) return DSPARK_ERR_NULL;
  return verify_common(R, V, rank, gamma, dt, W1, W2t, U, target, x, rows, lse_d, p_d_x, ell,
                       temperature, seed, c_star, n_accept, next_token, tau, tau_mean, ws,
                       ws_bytes, stream);
}

}  // extern "C"

namespace {

// Losses, and with g (non-null) every gradient.
struct GradOut {
  float *dU, *dW1, *dW2t, *dh, *dw;
};

dspark_status train_common(int R, int V, int rank, int d, int gamma, int dt, const void* W1,
                           const void* W2t, const float* U, const void* h, const float* w,
                           const float* target, const int32_t* x_star, float temperature,
                           float lambda, float alpha_ce, float alpha_tv, float alpha_conf,
                           float* terms, double* sums, const GradOut* g, void* ws,
                           size_t ws_bytes, dspark_stream_t stream) {
  if (dt != DSPARK_F32 && dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (!W1 || !W2t || !U || !h || !w || !target || !x_star || !terms || !sums)
    return DSPARK_ERR_NULL;
  if (g && (!g->dU || !g->dW1 || !g->dW2t || !g->dh || !g->dw)) return DSPARK_ERR_NULL;
  if (R < 1 || R > kMaxR || V < 2 || V > kMaxV || gamma < 1 || gamma > kMaxGamma || d < 1 ||
      d > kMaxD)
    return DSPARK_ERR_SHAPE;
  dspark_status s = check_rank(dt, rank);
  if (s != DSPARK_OK) return s;
  if (g && dt != DSPARK_BF16) return DSPARK_ERR_DTYPE;  // gradients: bf16 weights only
  if (g && rank % 32 != 0) return DSPARK_ERR_SHAPE;
  if (!aligned16(W1) || !aligned16(W2t) ||
      ((V % 4) == 0 && (!aligned16(U) || !aligned16(target))) ||
      (g && (V % 4) == 0 && !aligned16(g->dU)))
    return DSPARK_ERR_SHAPE;
  if (!(temperature > 0.0f) || isinf(temperature) || !(lambda > 0.0f) || isinf(lambda) ||
      !isfinite(alpha_ce) || !isfinite(alpha_tv) || !isfinite(alpha_conf))
    return DSPARK_ERR_VALUE;
  const VerifyPlan plan = plan_verify(R, V, gamma);
  const TrainPlan tplan = plan_train(R, V, rank, d, gamma);
  const size_t need = g ? tplan.ws_grad_bytes : tplan.ws_bytes;
  if (!ws || ws_bytes < need || !aligned16(ws)) return DSPARK_ERR_WORKSPACE;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  float* c = reinterpret_cast<float*>(wsb + tplan.off_c);
  float* surv = reinterpret_cast<float*>(wsb + tplan.off_surv);
  // c_k = sigma(w . [h_k; W1[x*_{k-1}]]) with the target block as the Markov input
  ConfArgs cargs{R, gamma, d, rank, V, dt == DSPARK_BF16, h, W1, x_star, w, c, surv, nullptr};
  if (token_error_address(&cargs.err) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  if (launch_confidence(cargs, st) != hipSuccess) return DSPARK_ERR_LAUNCH;

  VerifyArgs args{};
  args.R = R;
  args.V = V;
  args.rank = rank;
  args.gamma = gamma;
  args.bf16 = dt == DSPARK_BF16;
  args.greedy = false;
  args.W1 = W1;
  args.W2t = W2t;
  args.U = U;
  args.target = target;
  args.x = x_star;
  args.err = cargs.err;
  args.kscale = kscale_of(temperature);
  args.ws = wsb;
  TrainArgs targs{};
  targs.lambda = lambda;
  targs.alpha_ce = alpha_ce;
  targs.alpha_tv = alpha_tv;
  targs.alpha_conf = alpha_conf;
  targs.inv_t = 1.0f / temperature;
  targs.c = c;
  targs.terms = terms;
  targs.sums = sums;
  targs.d = d;
  targs.h = h;
  targs.w = w;
  if (g) {
    targs.dU = g->dU;
    targs.dW1 = g->dW1;
    targs.dW2t = g->dW2t;
    targs.dh = g->dh;
    targs.dw = g->dw;
  }
  if (launch_train(args, targs, plan, tplan, st) != hipSuccess) return DSPARK_ERR_LAUNCH;
  return DSPARK_OK;
}

}  // namespace

extern "C" {

dspark_status dspark_train_loss(int R, int V, int rank, int d, int gamma, int dt, const void* W1,
                                const void* W2t, const float* U, const void* h, const float* w,
                                const float* target, const int32_t* x_star, float temperature,
                                float lambda, float alpha_ce, float alpha_tv, float alpha_conf,
                                float* terms, double* sums, void* ws, size_t ws_bytes,
                                dspark_stream_t stream) {
  return train_common(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, target, x_star, temperature,
                      lambda, alpha_ce, alpha_tv, alpha_conf, terms, sums, nullptr, ws, ws_bytes,
                      stream);
}

dspark_status dspark_train_loss_grad(int R, int V, int rank, int d, int gamma, int dt,
                                     const void* W1, const void* W2t, const float* U,
                                     const void* h, const float* w, const float* target,
                                     const int32_t* x_star, float temperature, float lambda,
                                     float alpha_ce, float alpha_tv, float alpha_conf,
                                     float* terms, double* sums, float* dU, float* dW1,
                                     float* dW2t, float* dh, float* dw, void* ws,
                                     size_t ws_bytes, dspark_stream_t stream) {
  const GradOut g{dU, dW1, dW2t, dh, dw};
  return train_common(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, target, x_star, temperature,
                      lambda, alpha_ce, alpha_tv, alpha_conf, terms, sums, &g, ws, ws_bytes,
                      stream);
}

dspark_status dspark_token_errors(uint32_t* flag, int clear) {
  if (!flag) return DSPARK_ERR_NULL;
  if (clear != 0 && clear != 1) return DSPARK_ERR_VALUE;
  uint32_t* word = nullptr;
  if (token_error_address(&word) != DSPARK_OK) return DSPARK_ERR_LAUNCH;
  if (hipMemcpy(flag, word, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return DSPARK_ERR_LAUNCH;
  if (clear) {
    const uint32_t zero = 0u;
    if (hipMemcpy(word, &zero, sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess)
      return DSPARK_ERR_LAUNCH;
  }
  return DSPARK_OK;
}

}  // extern "C"

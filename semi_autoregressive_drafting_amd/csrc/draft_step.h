// Internal interface of the draft step (markov_step.hip): its launch plan,
// arguments and launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

// Launch shape of one draft step (see markov_step.hip).
struct StepPlan {
  int grid_x, grid_y;
  int n_slabs;        // vocabulary slabs (workgroups) per request group
  int n_groups;       // request groups of 128 (4 waves = 4 request tiles sharing
                      // an LDS W2t tile)
  int n_vtiles;       // 32-wide vocabulary tiles
  size_t rec_step;    // workspace: per-step record planes [gamma][n_slabs][5][R]
  size_t off_best;    //   then the winner words [gamma][R] (u64, kWinnerStride apart)
  size_t ws_bytes;
};

struct StepArgs {
  int R, V, rank, d, gamma, k;
  bool bf16, greedy;
  bool prev_from_best;  // x_{k-1} comes from step k-1's winner word (inside a block)
  const void* W1;
  const void* W2t;
  const float* U;
  const void* h;
  const float* w;
  const void* E_rows;   // RNN head: row r of the bias input per request [R][rank]; null: W1[x_{k-1}]
  float kscale;  // log2(e) / T
  uint64_t seed;
  int32_t* x;
  float* p;
  float* lse;
  float* c;
  float* a;
  float* z_debug;
  float* rec;                // records of step 1; step k at rec + (k-1) * rec_step_f
  size_t rec_step_f;         // floats per step plane
  unsigned long long* best;  // winner words [gamma][R], kWinnerStride apart
  int n_vtiles, n_slabs, n_groups;
  uint32_t* err;  // token-error word (checked_token)
};

StepPlan plan_draft_step(int R, int V, int gamma);
hipError_t launch_draft_step(const StepArgs& a, const StepPlan& plan, hipStream_t stream);
// The gamma steps of a block, in order (a.k and a.prev_from_best are set here).
hipError_t launch_draft_steps(StepArgs a, const StepPlan& plan, hipStream_t stream);
// Zero the winner words of the workspace (its region from plan.off_best on).
hipError_t launch_clear_winners(const StepArgs& a, const StepPlan& plan, hipStream_t stream);
// Merge the records of steps k0 .. k0+nk-1 and write x, p and lse (c and a are
// written by the step kernels themselves).
hipError_t launch_draft_finalize(const StepArgs& a, const StepPlan& plan, int k0, int nk,
                                 hipStream_t stream);

}  // namespace dspark

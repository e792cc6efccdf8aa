/*
 * dspark.h -- C ABI of the DSpark semi-autoregressive drafting hot path for
 * AMD MI355X (gfx950).  Library: libdspark.so (hand-written HIP kernels).
 *
 * Sources (cited by page title and section):
 *   [P1] "DSpark" (rainlin-net.pages.dev/llm-inference/dspark)
 *   [P2] "投机解码的新做法：整块草稿、按负载验证与 PD 分离" (anrans.github.io
 *        ai-infra-handbooks, serving/frontier/spec-next)
 *   [P3] "DSpark: Speculative decodingを活用したLLM推論の高速化" (ja.news.hada.io)
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise.  Every buffer is
 *     owned by the caller; the library never allocates, frees or
 *     synchronises.  Each call only enqueues kernels on `stream` (0 = the
 *     default stream) and returns.
 *   - Arguments are validated on the host before any HIP call; a failed check
 *     returns an error status and enqueues nothing.  Launch failures return
 *     DSPARK_ERR_LAUNCH.  Faults inside kernels surface at the caller's next
 *     synchronisation.  Device data is not validated on the host: a token id
 *     outside [0, V) that a kernel uses to gather a W1 row is clamped into
 *     range (so the gather stays in bounds) and recorded in the GPU's
 *     token-error word (see dspark_token_errors); NaNs are not checked.
 *   - Outputs are overwritten; outputs must not alias inputs.
 *   - Layouts are row-major and dense:
 *       W1   [V][rank]       Markov embedding table (P1 §2.3, W1 in R^{V x r})
 *       W2t  [V][rank]       the Markov projection W2 in R^{r x V} (P1 §2.3)
 *                            stored vocabulary-major, i.e. W2t[v][i] = W2[i][v]
 *                            (the weight layout of a rank->vocab linear layer)
 *       U    [R][gamma][V]   backbone base logits U_1..U_gamma, fp32 (P1 §2.1)
 *       h    [R][gamma][d]   backbone hidden states h_1..h_gamma (P1 §2.1)
 *       w    [d + rank]      confidence weights, fp32: w[0:d] for h_k,
 *                            w[d:] for W1[x_{k-1}] (P1 §3.1, eq. c_k)
 *       x    [R][gamma+1]    int32 token block; x[r][0] is the anchor x_0,
 *                            x[r][k] the token drafted at position k
 *       p, lse, c, a  [R][gamma] fp32, position k stored at column k-1
 *   - W1, W2t and h share one element type `dt`: DSPARK_BF16 (raw bf16 bits)
 *     or DSPARK_F32.
 *   - Random numbers come from a counter-based generator (the PCG hash of
 *     Jarzynski & Olano, JCGT 2020): for stream s, request r, position k and
 *     vocabulary entry v, key = pcg folded over (seed low word, seed high
 *     word, s, r, k); bits = pcg(key + v); u = ((bits >> 9) + 0.5) * 2^-23.
 *     Streams: 1 draft sampling, 2 acceptance tests, 3 residual resampling,
 *     4 bonus sampling.  Outputs are therefore a deterministic function of
 *     (inputs, seed), and repeated calls give bit-identical results.
 *
 * Limits: 1 <= R <= 512; 1 <= gamma <= 16; 2 <= V <= 2^24;
 *         bf16: rank multiple of 16, 16 <= rank <= 256;
 *         fp32: rank multiple of 4, 4 <= rank <= 128;  1 <= d <= 65536;
 *         W1, W2t, ws (and U, target when V % 4 == 0) 16-byte aligned;
 *         R * gamma <= 8192 for dspark_schedule.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dspark_stream_t; /* a hipStream_t */

typedef enum {
  DSPARK_OK = 0,
  DSPARK_ERR_NULL = 1,      /* a required pointer is NULL */
  DSPARK_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
  DSPARK_ERR_DTYPE = 3,     /* unknown element type */
  DSPARK_ERR_VALUE = 4,     /* bad scalar (temperature < 0 or NaN, k out of range) */
  DSPARK_ERR_WORKSPACE = 5, /* workspace NULL or smaller than dspark_workspace_bytes() */
  DSPARK_ERR_LAUNCH = 6     /* a kernel launch failed */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

typedef enum {
  DSPARK_OP_DRAFT_STEP = 0,
  DSPARK_OP_SCHEDULE = 1,
  DSPARK_OP_VERIFY = 2,
  DSPARK_OP_TRAIN_LOSS = 3,
  DSPARK_OP_TRAIN_GRAD = 4, /* rank must be a multiple of 32 (<= 256), else 0 */
  DSPARK_OP_DRAFT_RNN = 5   /* rank must be a multiple of 32 (<= 256), else 0 */
} dspark_op;

/* Bytes of device workspace entry point `op` needs for these sizes (0 if the
 * sizes are invalid).  Host-only; makes no HIP call. */
size_t dspark_workspace_bytes(int op, int R, int V, int rank, int gamma);

/* Human-readable name of a status code (static string). Host-only. */
const char* dspark_status_string(int status);

/*
 * The token-error word of the current device (not a method step: a guard
 * for corrupted device data).  Every kernel that gathers a W1 row by a token
 * id read from device memory -- the anchor and drafted columns of x in the
 * draft step, the confidence head and verification, x* in training, the
 * winner of the previous step inside a block -- stores 1 into the word when
 * the id lies outside [0, V), clamps the id into range and carries on.  The
 * word is shared by all calls on the device and stays set until cleared.
 * *flag (HOST pointer) receives the word; clear = 1 then resets it to 0,
 * clear = 0 leaves it.  Synchronous (blocking copies): call it after the
 * streams that ran the kernels have been synchronised.  flag NULL ->
 * DSPARK_ERR_NULL; clear outside {0, 1} -> DSPARK_ERR_VALUE; no device or a
 * failed copy -> DSPARK_ERR_LAUNCH.
 */
dspark_status dspark_token_errors(uint32_t* flag, int clear);

/*
 * One sequential draft step k (1 <= k <= gamma) for all R requests
 * [P1 §2.2 eq. p_k; §2.3 eq. B; P1 §6.2 loop; P3 アーキテクチャ]:
 *   e_r   = W1[x[r][k-1]]                         gather (one lookup)
 *   z_r,v = U[r][k-1][v] + e_r . W2t[v]           bias + base logits
 *   T > 0: s = z / T, lse = log sum_v exp(s_v),
 *          x[r][k] = lowest v maximising s_v + G_v, G_v = -ln(-ln u_v) from
 *          stream 1 at (r, k, v); p[r][k-1] = exp(s_x - lse).
 *   T = 0: x[r][k] = lowest argmax_v z; p = 1; lse := max_v z.
 * If h and w are both non-NULL, also the confidence head and survival
 * product [P1 §3.1 eq. c_k; §1.1 eq. a_j]:
 *   c[r][k-1] = sigma(w[0:d] . h[r][k-1] + w[d:] . e_r)       (fp32)
 *   a[r][k-1] = (k == 1 ? 1 : a[r][k-2]) * c[r][k-1]           (one fp32 multiply)
 * (c and a must then be non-NULL; with h == w == NULL they are not touched.)
 * z_debug, if non-NULL, receives z as fp32 [R][V] (testing only).
 * Reads x[:, k-1]; writes x[:, k], p, lse (and c, a) at column k-1.
 * ws: dspark_workspace_bytes(DSPARK_OP_DRAFT_STEP, ...) bytes of device memory
 * (per-workgroup partial records for gamma steps, then gamma x R 64-bit winner
 * words, each alone in a 128-byte line), ZERO-FILLED before its first use: the
 * winner words are atomic-max targets that every call leaves at zero again.
 * Calls that may run concurrently need separate workspaces.
 * Enqueues two kernels: the streaming step, which also computes c and a of
 * step k (they are valid once it has run), and the finalisation (the record
 * merge, which writes x[:, k], p and lse).
 */
dspark_status dspark_draft_step(int R, int V, int rank, int d, int gamma, int k, int dt,
                                const void* W1, const void* W2t, const float* U,
                                const void* h, const float* w, float temperature,
                                uint64_t seed, int32_t* x, float* p, float* lse, float* c,
                                float* a, float* z_debug, void* ws, size_t ws_bytes,
                                dspark_stream_t stream);

/*
 * The whole draft block: dspark_draft_step for k = 1..gamma in order on
 * `stream` (x[:, 0] must hold the anchors), without z_debug.  Same arguments,
 * results and workspace as the single step.  Step k takes x_{k-1} straight
 * from step k-1's winner word, and one finalisation for all gamma positions
 * runs after the last step (gamma + 1 kernels).
 */
dspark_status dspark_draft_block(int R, int V, int rank, int d, int gamma, int dt,
                                 const void* W1, const void* W2t, const float* U,
                                 const void* h, const float* w, float temperature,
                                 uint64_t seed, int32_t* x, float* p, float* lse, float* c,
                                 float* a, void* ws, size_t ws_bytes, dspark_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * dspark_draft_block without the workspace arguments.  Same arguments
 * otherwise, same kernels, and the same results bit for bit as
 * dspark_draft_block with a zero-filled workspace.
 *
 * The workspace is a static device array inside the library, 22 MiB per GPU,
 * held from the library's first use on that GPU until the process ends.  It
 * fits the draft workspace of every shape this ABI accepts; a shape whose
 * workspace did not fit would return DSPARK_ERR_WORKSPACE before any HIP
 * call.  Nothing is allocated or freed: the call only enqueues kernels
 * (a small fill kernel clears the winner words, then the gamma steps and
 * the merge).  Every call on a GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * wrong results; serialise them.  Errors: as dspark_draft_block, plus
 * DSPARK_ERR_LAUNCH if the array's device address cannot be obtained.
 */
dspark_status dspark_draft_block_noalloc(int R, int V, int rank, int d, int gamma, int dt,
                                         const void* W1, const void* W2t, const float* U,
                                         const void* h, const float* w, float temperature,
                                         uint64_t seed, int32_t* x, float* p, float* lse,
                                         float* c, float* a, dspark_stream_t stream);

/*
 * dspark_draft_block split into its two phases, so that a caller can place
 * events between them: DSPARK_PHASE_STEPS enqueues the gamma streaming steps
 * (winner words and partial records in ws), DSPARK_PHASE_MERGE the record
 * merge that writes x[:, 1..gamma], p and lse [P1 §2.2 eq. p_k: the exact
 * draft probability of each sampled token].  Calling STEPS then MERGE on one
 * stream equals dspark_draft_block (both together: phases = 3); MERGE must
 * follow the STEPS of the same block with the same arguments and workspace.
 * phases outside 1..3 -> DSPARK_ERR_VALUE.
 */
enum { DSPARK_PHASE_STEPS = 1, DSPARK_PHASE_MERGE = 2 };
dspark_status dspark_draft_block_phases(int R, int V, int rank, int d, int gamma, int dt,
                                        const void* W1, const void* W2t, const float* U,
                                        const void* h, const float* w, float temperature,
                                        uint64_t seed, int32_t* x, float* p, float* lse,
                                        float* c, float* a, void* ws, size_t ws_bytes,
                                        int phases, dspark_stream_t stream);

/*
 * A draft block with the RNN head [P1 §2.4 RNN Head; P3 アーキテクチャ]: the
 * pages describe a block-internal state s_k updated by a gate over the
 * previous state (the longer prefix), the previous token's embedding and the
 * backbone state h_k, and give no equations.  This entry point reads it as a
 * GRU cell (gate order reset, update, new; s_0 = 0), with e_k = W1[x[r][k-1]]:
 *   r   = sigma(W_ih[0:H] [e; h_k] + b_ih[0:H] + W_hh[0:H] s + b_hh[0:H])
 *   z   = sigma(W_ih[H:2H] [e; h_k] + b_ih[H:2H] + W_hh[H:2H] s + b_hh[H:2H])
 *   n   = tanh(W_ih[2H:] [e; h_k] + b_ih[2H:] + r * (W_hh[2H:] s + b_hh[2H:]))
 *   s_k = (1 - z) n + z s_{k-1}                          (H = rank)
 * and bf16(s_k) replaces W1[x_{k-1}] in the bias of the draft step
 * (dspark_draft_step's formula otherwise: same sampling, RNG streams,
 * confidence c_k = sigma(w . [h_k; W1[x_{k-1}]]) and survival a_k).
 * Inputs as dspark_draft_block (dt must be DSPARK_BF16, else
 * DSPARK_ERR_DTYPE; h and w required), plus W_ih bf16 [3 rank][rank + d],
 * W_hh bf16 [3 rank][rank], b_ih, b_hh fp32 [3 rank].  rank must be a
 * multiple of 32 and d of 16 (DSPARK_ERR_SHAPE).  Outputs as
 * dspark_draft_block, plus state fp32 [R][rank] = s_gamma (16-byte aligned)
 * and, unless rows is NULL, rows bf16 [R][gamma][rank] = bf16(s_k) of every
 * position: the bias rows that dspark_verify_rnn needs.
 * ws: dspark_workspace_bytes(DSPARK_OP_DRAFT_RNN, ...) bytes, zero-filled
 * once before first use (the draft step's part is left zeroed by each call).
 */
dspark_status dspark_draft_block_rnn(int R, int V, int rank, int d, int gamma, int dt,
                                     const void* W1, const void* W2t, const float* U,
                                     const void* h, const float* w, const void* W_ih,
                                     const void* W_hh, const float* b_ih, const float* b_hh,
                                     float temperature, uint64_t seed, int32_t* x, float* p,
                                     float* lse, float* c, float* a, float* state, void* rows,
                                     void* ws, size_t ws_bytes, dspark_stream_t stream);

/*
 * Confidence head and survival for a whole drafted block
 * [P1 §3.1 eq. c_k; P1 §1.1 eq. a_j; §4.1 eq. tau]:
 *   c[r][k-1] = sigma(w[0:d] . h[r][k-1] + w[d:] . W1[x[r][k-1]]),  k = 1..gamma
 *   a[r][j]   = fp32 running product c[r][0] * ... * c[r][j], left to right.
 * Same arithmetic as the fused path of dspark_draft_step.
 */
dspark_status dspark_confidence(int R, int gamma, int d, int rank, int V, int dt,
                                const void* h, const void* W1, const int32_t* x,
                                const float* w, float* c, float* a, dspark_stream_t stream);

/*
 * Hardware-aware prefix scheduler [P1 §4.1 eqs. B, tau, Theta and the global
 * sort; P1 §4.2 early stop; P3 スケジューラ; P2 "按负载决定验证多少"]:
 *   sort all N = R*gamma candidates (r, j) by key (a[r][j] descending, flat
 *   index r*gamma + j ascending); q_i = round-half-even(a_i * 2^32) (int64);
 *   G_b = q_1 + ... + q_b; tau_fix(b) = R*2^32 + G_b;
 *   Theta_fix(b) = (double)tau_fix(b) * sps[R + b];
 *   admit b+1 while Theta_fix(b+1) > Theta_fix(b) (strictly); stop at the first
 *   non-increase.  Outputs (device): ell[R] = admitted positions of request r
 *   (always a prefix), *budget = b*, *theta = Theta_fix(b*) * 2^-32 (tokens/s;
 *   may be NULL).
 * sps: fp64 [sps_len], steps/s at B verified tokens, B = 0..R*(1+gamma)
 * (sps_len >= R*(1+gamma)+1).  a: fp32 [R][gamma], values in [0, 1].
 * R*gamma <= 8192.  ws: dspark_workspace_bytes(DSPARK_OP_SCHEDULE, R, V, rank,
 * gamma) bytes (V and rank are ignored), 16-byte aligned, ZERO-FILLED before
 * its first use: it holds the prefix sums and requests by sorted position and
 * the counters of finished workgroups, which every call leaves at zero again.
 * Calls that overlap in time need workspaces of their own; a workspace sized
 * for one R*gamma serves every smaller call.
 */
dspark_status dspark_schedule(int R, int gamma, const float* a, const double* sps, int sps_len,
                              int32_t* ell, int32_t* budget, double* theta, void* ws,
                              size_t ws_bytes, dspark_stream_t stream);

/*
 * Asynchronous (production) scheduler [P1 §4.3 生产异步调度; P3
 * スケジューラの実運用適用]: the budget comes from survival probabilities two
 * steps old, the selection from the current ones.
 *   K = the b in 0..N (N = R*gamma) with the largest
 *       Theta_fix(b) = (double)(R*2^32 + G_b) * sps[R + b], where G_b sums
 *       q_i = round-half-even(a_lag_i * 2^32) over the first b candidates of
 *       a_lag in the dspark_schedule key order; every b is examined (no early
 *       stop) and the smallest b wins a tie.
 *   Then the first K candidates of a_cur in the same key order (a_cur
 *   descending, flat index ascending) are admitted.
 * Outputs (device): ell[R] = admitted positions of request r (a prefix when
 * the rows of a_cur are non-increasing), *budget = K, *theta =
 * Theta_fix(K) * 2^-32 (the lagged estimate; may be NULL).
 * a_lag, a_cur: fp32 [R][gamma], values in [0, 1]; sps and ws as for
 * dspark_schedule; R*gamma <= 8192.  ell depends on a_lag only through K.
 */
dspark_status dspark_schedule_async(int R, int gamma, const float* a_lag, const float* a_cur,
                                    const double* sps, int sps_len, int32_t* ell,
                                    int32_t* budget, double* theta, void* ws, size_t ws_bytes,
                                    dspark_stream_t stream);

/*
 * Verification of drafted blocks against target logits [P1 §3.1 eq. c*;
 * standard rejection sampling: P1 opening and §2.2, P3 問題定義]:
 *   for every (r, k): p_d = softmax((U[r][k-1] + W1[x[r][k-1]] . W2) / T),
 *   p_t = softmax(target[r][k-1] / T);  c_star[r][k-1] = 1 - 1/2 |p_d - p_t|_1.
 *   for j = 1..ell[r]: accept x[r][j] iff u(stream 2, r, j, v=0) <
 *   p_t(x_j) / p_d_x[r][j-1]  (p_d_x = the draft probabilities kept by
 *   dspark_draft_step).  At the first rejection next_token[r] = Gumbel-argmax of
 *   log(p_t - p_d) over {v : p_t(v) > p_d(v)} (stream 3 at (r, j)); if all are
 *   accepted, next_token[r] = Gumbel sample of p_t at row ell[r]+1 (stream 4),
 *   or -1 when ell[r] = gamma.  n_accept[r] = accepted count; tau[r] =
 *   n_accept[r] + 1; *tau_mean = mean of tau over requests (fp32).
 *   T = 0: both laws are point masses (draft: on x_j; target: lowest argmax).
 * lse_d: [R][gamma] fp32 draft log-normalisers from dspark_draft_step.
 * target: fp32 [R][gamma][V].  ws: dspark_workspace_bytes(DSPARK_OP_VERIFY,...).
 */
dspark_status dspark_verify(int R, int V, int rank, int gamma, int dt, const void* W1,
                            const void* W2t, const float* U, const float* target,
                            const int32_t* x, const float* lse_d, const float* p_d_x,
                            const int32_t* ell, float temperature, uint64_t seed,
                            float* c_star, int32_t* n_accept, int32_t* next_token,
                            int32_t* tau, float* tau_mean, void* ws, size_t ws_bytes,
                            dspark_stream_t stream);

/*
 * dspark_verify for blocks drafted by the RNN head [P1 §2.4]: p_d at
 * position k is recomputed from rows[r][k-1] ([R][gamma][rank] in dt, 16-byte
 * aligned; dspark_draft_block_rnn writes them in bf16) in place of W1[x[r][k-1]];
 * everything else, arguments, outputs, workspace and errors included, is
 * dspark_verify's.  rows NULL -> DSPARK_ERR_NULL.
 */
dspark_status dspark_verify_rnn(int R, int V, int rank, int gamma, int dt, const void* W1,
                                const void* W2t, const float* U, const float* target,
                                const int32_t* x, const void* rows, const float* lse_d,
                                const float* p_d_x, const int32_t* ell, float temperature,
                                uint64_t seed, float* c_star, int32_t* n_accept,
                                int32_t* next_token, int32_t* tau, float* tau_mean, void* ws,
                                size_t ws_bytes, dspark_stream_t stream);

/*
 * Training losses of the sequential and confidence heads [P1 §5 训练目标; P3
 * アーキテクチャ (default weights)] over R drafted blocks of gamma positions,
 * with the target block as the Markov input (teacher forcing):
 *   e_{r,k}  = W1[x*[r][k-1]]  (x*[r][0] is the anchor)
 *   p_d      = softmax((U[r][k-1] + e . W2) / T),  p_t = softmax(target[r][k-1] / T)
 *   ce       = -ln p_d(x*[r][k])
 *   tv       = ||p_d - p_t||_1,  c* = 1 - tv / 2 (a constant target)
 *   c        = sigma(w . [h[r][k-1]; e])
 *   conf     = -(c* ln c + (1 - c*) ln(1 - c))
 *   w_k      = exp(-(k-1) / lambda)  (P3 uses lambda = gamma)
 * Outputs (device): terms fp32 [R][gamma][4] = (ce, tv, conf, c) per position;
 * sums fp64 [4] = (sum w_k ce, sum w_k tv, sum w_k conf,
 * alpha_ce*.. + alpha_tv*.. + alpha_conf*..), summed over the batch in a fixed
 * order (bit-reproducible).  The P1 defaults are alpha = 0.1, 0.9, 1.0.
 * Inputs as for dspark_verify (U, target fp32 [R][gamma][V]; W1, W2t, h in dt;
 * w fp32 [d + rank]); x_star int32 [R][gamma+1].  T > 0 and lambda > 0 (else
 * DSPARK_ERR_VALUE).  ws: dspark_workspace_bytes(DSPARK_OP_TRAIN_LOSS, ...)
 * bytes; its contents need no initialisation.  Forward only: the gradients
 * come from dspark_train_loss_grad.
 */
dspark_status dspark_train_loss(int R, int V, int rank, int d, int gamma, int dt, const void* W1,
                                const void* W2t, const float* U, const void* h, const float* w,
                                const float* target, const int32_t* x_star, float temperature,
                                float lambda, float alpha_ce, float alpha_tv, float alpha_conf,
                                float* terms, double* sums, void* ws, size_t ws_bytes,
                                dspark_stream_t stream);

/*
 * dspark_train_loss plus the gradients of the weighted total
 * L = alpha_ce sum w_k ce + alpha_tv sum w_k tv + alpha_conf sum w_k conf
 * [P1 §5 训练目标], c* held constant (it is a label).  With z = U + e . W2,
 * s_v = sign(p_d(v) - p_t(v)) (0 where equal) and mu = sum_v s_v p_d(v):
 *   dU[r][k-1][v] = dL/dz = (w_k / T) (alpha_ce (p_d(v) - [v = x*_k])
 *                                      + alpha_tv p_d(v) (s_v - mu))
 *   dl            = w_k alpha_conf (c - c*)       (confidence logit)
 *   dE            = dU . W2t + dl w[d:]           (gathered rows e)
 *   dW1[t]        = sum of the dE rows whose Markov input x*[r][k-1] is t
 *                   (0 for tokens that do not occur)
 *   dW2t          = dU^T . E                     fp32 [V][rank]
 *   dh            = dl w[:d]                      fp32 [R][gamma][d]
 *   dw            = sum over positions of dl [h; e]  fp32 [d + rank]
 * Outputs (device, fp32, overwritten): dU [R][gamma][V] (16-byte aligned when
 * V % 4 == 0), dW1 [V][rank], dW2t [V][rank], dh, dw.  The two contractions
 * round dU to bf16 as an MFMA operand and accumulate in fp32; every other
 * step is fp32 or fp64.  All sums run in a fixed order (bit-reproducible).
 * Requires dt = DSPARK_BF16 (else DSPARK_ERR_DTYPE) and rank a multiple of 32
 * (else DSPARK_ERR_SHAPE).  ws: dspark_workspace_bytes(DSPARK_OP_TRAIN_GRAD,
 * ...) bytes (it holds a transposed copy of W2t; sized for any d up to 65536); no
 * initialisation needed.
 */
dspark_status dspark_train_loss_grad(int R, int V, int rank, int d, int gamma, int dt,
                                     const void* W1, const void* W2t, const float* U,
                                     const void* h, const float* w, const float* target,
                                     const int32_t* x_star, float temperature, float lambda,
                                     float alpha_ce, float alpha_tv, float alpha_conf,
                                     float* terms, double* sums, float* dU, float* dW1,
                                     float* dW2t, float* dh, float* dw, void* ws,
                                     size_t ws_bytes, dspark_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */

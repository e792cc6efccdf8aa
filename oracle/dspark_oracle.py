"""CPU oracle for the DSpark semi-autoregressive drafting hot path.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The product path
never does, and this module shares no code with it (no kernels, headers,
helpers, tables or constants): it is a plain, slow, obviously correct fp64
restatement of what the pages define, used to check the HIP path.

Sources, cited by page title and section (no other source defines the method):
  [P1] "DSpark" -- rainlin-net.pages.dev/llm-inference/dspark (sections 1-9).
  [P2] "投机解码的新做法：整块草稿、按负载验证与 PD 分离" -- anrans.github.io
       ai-infra-handbooks, serving/frontier/spec-next (headings "负载越高，K 越要小",
       "一次前向给出一整块草稿", "按负载决定验证多少", "练习").
  [P3] "DSpark: Speculative decodingを活用したLLM推論の高速化" -- ja.news.hada.io
       topic 30902 (headings アーキテクチャ, 実験分析, 実サービス配備).

What each function follows, and what pins it (tests/test_oracle_pins.py):
  markov_bias / draft_logits   P1 §2.3 eq. B, P1 §2.2 eq. p_k.  Pinned by the
        identity-W1 special case, the full-matrix B = W1 W2 row, the P2 Markov
        toy printout (0.62 / 0.81) and a two-token closed form.
  draft_distribution           P1 §2.2 eq. p_k and eq. P(X|x0).  Pinned by
        brute-force enumeration (sum over all blocks = 1) and closed forms.
  draft_step (two-level Gumbel-argmax)   sampling of p_k.  Pinned by a
        chi-square test of sampled blocks against the enumerated P(X|x0) (V = 8:
        one vocabulary block), chi-square tests of single steps at V = 40 and
        V = 100 (several blocks, a ragged last block) against softmax, the
        reduction to the textbook Gumbel-max for V <= 16 and for one-hot blocks,
        and T=0 -> argmax.
  confidence                   P1 §3.1 eq. c_k.  Pinned by closed forms.
  survival / expected_tau      P1 §1.1 eq. a_j and eq. tau.  Pinned by the P2
        Markov toy printout and closed forms.
  theta_of_ell / schedule      P1 §4.1 eqs. B, tau, Theta and the global sort;
        P1 §4.2 early stop.  Pinned by the P2 cost-model and plan() printouts,
        exhaustive search over ell vectors, prefix contiguity and closed forms.
  schedule_async               P1 §4.3; P3 スケジューラの実運用適用.  Pinned by
        brute force over budgets (exact rational Theta), an explicit top-K
        count, agreement with `schedule` on unimodal curves, a hand-built cliff
        curve where the early stop and the global maximum differ, and causal
        isolation (ell changes with a_lag only through K).
  train_losses                 P1 §5 (L_CE, L_TV, L_conf, w_k; P3 defaults).
        Pinned by the two-token closed form, identical-law special cases,
        invariance to a constant logit shift, and the default weights.
  train_loss_grads             derivatives of train_losses.  Pinned by central
        finite differences of train_losses in every input it differentiates.
  gru_cell, rnn_draft_round    P1 §2.4 (RNN head; a GRU reading, the pages give
        no equations).  Pinned by torch.nn.GRUCell (CPU, fp64) on the same
        weights, by the saturated update gate (z = 1: the state stays 0 and the
        head reduces to the Markov head with W2 = 0), by the saturated new gate
        path (z = 0, identity input weights, no recurrence: the Markov head with
        bias rows bf16(tanh W1[x])), and by the block law summing to 1 at V = 8.
  verify                       P1 §3.1 eq. c*, standard rejection sampling (P1
        intro and §2.2; P3 問題定義).  Pinned by the c* = overlap identity,
        special cases, losslessness (output law = p_t) and acceptance-rate = c*.

Parity unpinned: the bits of the counter-based random number generator.  The
pages do not fix a generator; the one used here (and, written separately, on
the GPU) is the PCG hash of Jarzynski & Olano, "Hash Functions for GPU
Rendering", JCGT 9(3), 2020, keyed as described at `stream_key`.  Only its
statistical behaviour is pinned (uniformity of u and the sampler tests above).

Readings taken where the pages are silent:
  * draft sampling is the Gumbel-max trick applied at two levels: the
    vocabulary is cut into aligned blocks of 16 ids; a block is drawn by
    Gumbel-argmax of the block log-masses (noise from the DRAFT stream at
    counter = block index), then an id inside it by Gumbel-argmax of the logits
    (noise from the DRAFT_ENTRY stream at counter = id).  The law of the result
    is exactly softmax(s); ties -> lowest block, then lowest id.  Verification's
    residual and bonus draws are one-level Gumbel-argmax over the vocabulary;
  * s = (U_k + bias) / T; p_d and p_t use the same T; T = 0 means argmax
    (point mass, p = 1, lse reported as max z);
  * the confidence head has no bias term; w = [w_h (d); w_e (rank)]; c_1 uses
    W1[x_0] (the anchor);
  * a is an fp32 running product of fp32 c (left to right); tau in the
    scheduler is fixed point with unit 2^-32, Theta = float64(tau_fix) * SPS;
  * the global sort key is (a descending, flat index req*gamma+j ascending);
    the early stop admits candidate b+1 only if Theta strictly increases;
    Theta(0) = R * SPS(R);
  * verification: accept iff u < p_t(x)/p_d(x); under greedy drafting (T = 0)
    the draft law at position k is the point mass on the drafted x_k (so
    p_d(x) = 1 and c*_k = p_t(x_k)); the first rejection resamples
    from max(0, p_t - p_d) by Gumbel-argmax of log(p_t - p_d); all accepted ->
    bonus sampled from p_t at position ell+1 (none when ell = gamma, id -1);
    realised tau per request = accepted + 1.
"""
from __future__ import annotations

import itertools

import numpy as np

# ----------------------------------------------------------------------------
# Counter-based random numbers (written from the JCGT 2020 definition).
# ----------------------------------------------------------------------------
STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESID, STREAM_BONUS, STREAM_DRAFT_ENTRY = 1, 2, 3, 4, 5

_U32 = np.uint32


def pcg_hash(x):
    """pcg(v): state = v*747796405 + 2891336453; word = ((state >> ((state >> 28) + 4))
    ^ state) * 277803737; return (word >> 22) ^ word  -- all mod 2^32."""
    x = np.asarray(x, dtype=np.uint32)
    with np.errstate(over="ignore"):
        state = x * _U32(747796405) + _U32(2891336453)
        word = ((state >> ((state >> _U32(28)) + _U32(4))) ^ state) * _U32(277803737)
    return (word >> _U32(22)) ^ word


def stream_key(seed, stream, req, k):
    """32-bit key of one (seed, stream, request, position) row: the seed's low and
    high words, the stream id, the request index and the position are folded in,
    one pcg round each, in that order."""
    seed = np.asarray(seed, dtype=np.uint64)
    lo = (seed & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    hi = (seed >> np.uint64(32)).astype(np.uint32)
    h = pcg_hash(lo)
    h = pcg_hash(h ^ hi)
    h = pcg_hash(h ^ _U32(stream))
    h = pcg_hash(h ^ np.asarray(req, dtype=np.uint32))
    h = pcg_hash(h ^ np.asarray(k, dtype=np.uint32))
    return h


def uniforms(seed, stream, req, k, v):
    """u in (0,1) for element v of a row: bits = pcg(key + v mod 2^32);
    u = ((bits >> 9) + 0.5) * 2^-23, an odd multiple of 2^-24 with at most 24
    significant bits, hence exact in fp32 as well as fp64."""
    key = stream_key(seed, stream, req, k)
    with np.errstate(over="ignore"):
        bits = pcg_hash(key + np.asarray(v, dtype=np.uint32))
    return ((bits >> _U32(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel(u):
    """Standard Gumbel variate from a uniform: G = -ln(-ln u)."""
    return -np.log(-np.log(u))


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns: (bits << 16) reinterpreted as fp32."""
    return (np.asarray(bits, dtype=np.uint32) << _U32(16)).view(np.float32).astype(np.float64)


def as_f64(store):
    """Weights/hidden states as stored (uint16 bf16 bits or float32) -> exact fp64."""
    store = np.asarray(store)
    return bf16_to_f64(store) if store.dtype == np.uint16 else store.astype(np.float64)


# ----------------------------------------------------------------------------
# Sequential head: Markov bias, logits, distribution, sampling   [P1 §2.2-2.3]
# ----------------------------------------------------------------------------
def markov_bias(W1, W2t, x_prev):
    """B(x_{k-1}, .) = W1[x_{k-1}] W2  [P1 §2.3, eq. B], with W2 (rank x V) stored
    as its transpose W2t (V x rank).  One embedding lookup, then one rank->vocab
    projection per request."""
    E = W1[np.asarray(x_prev)]            # [n, rank]
    return E @ W2t.T                      # [n, V]


def draft_logits(U_k, W1, W2t, x_prev):
    """Exponent of p_k: U_k(v) + B_k(x_{k-1}, v)  [P1 §2.2, eq. p_k]."""
    return np.asarray(U_k, dtype=np.float64) + markov_bias(W1, W2t, x_prev)


def log_softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(s - m).sum(axis=-1, keepdims=True))
    return s - lse, lse[..., 0]


def draft_distribution(z, T):
    """p_k(. | x0, x<k) = softmax(z / T) over the vocabulary  [P1 §2.2, eq. p_k].
    T = 0: point mass on the lowest-id maximiser of z."""
    z = np.asarray(z, dtype=np.float64)
    if T > 0:
        logp, _ = log_softmax_rows(z / T)
        return np.exp(logp)
    p = np.zeros_like(z)
    idx = np.argmax(z, axis=-1)
    np.put_along_axis(p, idx[..., None], 1.0, axis=-1)
    return p


def _top2(keys):
    """(argmax with lowest index on ties, top1 - top2 gap) per row of a 2-D
    array.  With a single column, or a single finite entry, the gap is +inf."""
    x = np.argmax(keys, axis=-1)
    top1 = np.take_along_axis(keys, x[:, None], axis=-1)[:, 0]
    rest = keys.copy()
    np.put_along_axis(rest, x[:, None], -np.inf, axis=-1)
    top2 = rest.max(axis=-1)
    return x, top1 - top2


DRAFT_BLOCK = 16   # vocabulary ids per block of the two-level draft sampler


def block_log_mass(s):
    """log sum_{v in b} exp(s_v) for the aligned blocks b = [16j, 16j + 16) of the
    vocabulary (the last one ragged when V % 16 != 0); s [n, V] -> [n, nb]."""
    s = np.asarray(s, dtype=np.float64)
    n, V = s.shape
    nb = -(-V // DRAFT_BLOCK)
    pad = np.full((n, nb * DRAFT_BLOCK), -np.inf)
    pad[:, :V] = s
    blk = pad.reshape(n, nb, DRAFT_BLOCK)
    mb = blk.max(axis=2)
    return mb + np.log(np.exp(blk - mb[..., None]).sum(axis=2))


def draft_block_keys(s, seed, k, req_ids):
    """Perturbed block scores: block log-mass + G, G from the DRAFT stream at
    counter = block index."""
    lb = block_log_mass(s)
    nb = lb.shape[1]
    u = uniforms(np.asarray(seed)[..., None] if np.ndim(seed) else seed, STREAM_DRAFT,
                 np.asarray(req_ids)[:, None], k, np.arange(nb, dtype=np.uint32)[None, :])
    return lb + gumbel(u)


def draft_entry_keys(s_row, block, seed, k, req):
    """Perturbed scores s_v + G_v of the ids of one block of one row, G from the
    DRAFT_ENTRY stream at counter = v.  Returns (ids, keys)."""
    V = len(s_row)
    ids = np.arange(block * DRAFT_BLOCK, min(V, (block + 1) * DRAFT_BLOCK))
    u = uniforms(seed, STREAM_DRAFT_ENTRY, req, k, ids.astype(np.uint32))
    return ids, np.asarray(s_row, dtype=np.float64)[ids] + gumbel(u)


def draft_step(U_k, W1, W2t, x_prev, T, seed, k, req_ids, E=None):
    """One sequential step k for a set of requests (rows of U_k).

    z = U_k + W1[x_{k-1}] W2; for T > 0: s = z/T, lse = log sum_v exp(s_v),
    p_k(v) = exp(s_v - lse), and x_k is drawn from p_k by the two-level
    Gumbel-max trick: the block b* maximising block_log_mass(s)_b + G_b (lowest
    b on ties), then the id maximising s_v + G'_v inside b* (lowest id on
    ties).  P(b*) = sum_{v in b*} p_k(v) and P(v | b*) = p_k(v) / P(b*), so
    x_k ~ p_k exactly.  T = 0: x_k = argmax z, p = 1, lse := max z.

    Returned near-tie diagnostics (natural-log units of s): block_keys [n, nb]
    and gap = min(top-two gap of the block keys, top-two gap of the entry keys
    inside b*); at T = 0 the top-two gap of z.  E, if given, replaces the
    gathered rows W1[x_{k-1}] (the RNN head's state rows).
    """
    if E is None:
        z = draft_logits(U_k, W1, W2t, x_prev)
    else:
        z = np.asarray(U_k, dtype=np.float64) + np.asarray(E, dtype=np.float64) @ W2t.T
    n, V = z.shape
    req_ids = np.asarray(req_ids)
    if T > 0:
        s = z / T
        m = s.max(axis=1)
        lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        bkeys = draft_block_keys(s, seed, k, req_ids)
        bstar, gap_b = _top2(bkeys)
        # the ids of each row's drawn block, their noise and perturbed scores
        ids = bstar[:, None] * DRAFT_BLOCK + np.arange(DRAFT_BLOCK)[None, :]
        valid = ids < V
        idc = np.minimum(ids, V - 1)
        u = uniforms(np.asarray(seed)[..., None] if np.ndim(seed) else seed, STREAM_DRAFT_ENTRY,
                     req_ids[:, None], k, idc.astype(np.uint32))
        ekeys = np.where(valid, np.take_along_axis(s, idc, axis=1) + gumbel(u), -np.inf)
        xi, gap_e = _top2(ekeys)
        x = ids[np.arange(n), xi].astype(np.int64)
        gap = np.minimum(gap_b, gap_e)
        p = np.exp(s[np.arange(n), x] - lse)
        return {"z": z, "x": x, "p": p, "lse": lse, "gap": gap, "block_keys": bkeys}
    x, gap = _top2(z)
    return {"z": z, "x": x.astype(np.int64), "p": np.ones(n), "lse": z.max(axis=1), "gap": gap}


def draft_token_deficit(st, i, x_other, T, seed, k, req):
    """How far another token x_other of row i of a draft_step result falls short
    of being the sampler's choice, in natural-log units of s: T > 0 -> the larger
    of (max block key - key of x_other's block) and (max entry key inside that
    block - entry key of x_other); T = 0 -> max z - z[x_other].  0 for the
    sampler's own token; a differing token is a near-tie flip iff this is small."""
    if T == 0:
        return float(st["z"][i].max() - st["z"][i, x_other])
    bk = st["block_keys"][i]
    b = int(x_other) // DRAFT_BLOCK
    ids, ekeys = draft_entry_keys(st["z"][i] / T, b, seed, k, req)
    return float(max(bk.max() - bk[b], ekeys.max() - ekeys[ids == x_other][0]))


# ----------------------------------------------------------------------------
# Confidence head and survival                               [P1 §1.1, §3.1]
# ----------------------------------------------------------------------------
def sigmoid(t):
    return 1.0 / (1.0 + np.exp(-t))


def confidence(h_k, w, W1, x_prev):
    """c_k = sigma(w^T [h_k ; W1[x_{k-1}]])  [P1 §3.1, eq. c_k]; no bias term,
    w[:d] weights h_k and w[d:] weights the Markov embedding."""
    h_k = np.asarray(h_k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    d = h_k.shape[-1]
    e = W1[np.asarray(x_prev)]
    return sigmoid(h_k @ w[:d] + e @ w[d:])


def survival(c32):
    """a_{r,j} = prod_{i<=j} c_{r,i}  [P1 §1.1 eq. a_j; §4.1 eq. tau], as an fp32
    running product of fp32 c taken left to right (one rounding per factor)."""
    c32 = np.asarray(c32, dtype=np.float32)
    a = np.empty_like(c32)
    run = np.ones(c32.shape[:-1], dtype=np.float32)
    for j in range(c32.shape[-1]):
        run = (run * c32[..., j]).astype(np.float32)
        a[..., j] = run
    return a


def expected_tau(a, ell=None):
    """tau = 1 + sum_{j<=ell} a_j per request (bonus token included)
    [P1 §1.1 eq. tau; §4.1 eq. tau].  ell=None means the whole block."""
    a = np.asarray(a, dtype=np.float64)
    if ell is None:
        return 1.0 + a.sum(axis=-1)
    j = np.arange(a.shape[-1])
    return 1.0 + np.where(j[None, :] < np.asarray(ell)[:, None], a, 0.0).sum(axis=-1)


# ----------------------------------------------------------------------------
# Hardware-aware prefix scheduler                                  [P1 §4]
# ----------------------------------------------------------------------------
TAU_ONE = 2 ** 32   # fixed-point unit of tau


def tau_fixed_units(a):
    """q(a) = round-half-even(a * 2^32) as int64 (exact scaling in fp64)."""
    return np.rint(np.asarray(a, dtype=np.float32).astype(np.float64) * TAU_ONE).astype(np.int64)


def theta_of_ell(a, ell, sps):
    """Theta = tau * SPS(B) for a vector of verify lengths  [P1 §4.1, eqs. B, tau,
    Theta]: B = sum_r (1 + ell_r), tau = sum_r (1 + sum_{j<=ell_r} a_{r,j}).
    tau is accumulated in fixed point (unit 2^-32); returns Theta in tokens/s."""
    a = np.asarray(a, dtype=np.float32)
    R, g = a.shape
    ell = np.asarray(ell, dtype=np.int64)
    q = tau_fixed_units(a)
    mask = np.arange(g)[None, :] < ell[:, None]
    tau_fix = R * TAU_ONE + int(q[mask].sum())
    B = R + int(ell.sum())
    return float(np.float64(tau_fix) * np.float64(sps[B])) * 2.0 ** -32


def schedule(a, sps):
    """Global sort of all (request, position) candidates by survival, then admit
    them one by one while Theta strictly increases  [P1 §4.1 global sort, §4.2
    early stop; P3 スケジューラ].

    Returns (ell[R], budget b*, Theta(b*) in tokens/s, sorted flat order,
    Theta_fixed[0..N] before the 2^-32 scaling)."""
    a = np.asarray(a, dtype=np.float32)
    R, g = a.shape
    N = R * g
    flat = a.reshape(-1)
    order = np.argsort(-flat.astype(np.float64), kind="stable")      # a desc, index asc
    q = tau_fixed_units(flat[order])
    G = np.concatenate([[0], np.cumsum(q)]).astype(np.int64)
    tau_fix = np.int64(R) * TAU_ONE + G
    theta_fix = tau_fix.astype(np.float64) * np.asarray(sps, dtype=np.float64)[R + np.arange(N + 1)]
    b = 0
    while b < N and theta_fix[b + 1] > theta_fix[b]:
        b += 1
    ell = np.bincount(order[:b] // g, minlength=R).astype(np.int64)
    return ell, b, float(theta_fix[b]) * 2.0 ** -32, order, theta_fix


def schedule_async(a_lag, a_cur, sps):
    """Production asynchronous scheduling  [P1 §4.3 生产异步调度; P3
    スケジューラの実運用適用]: the total budget K is chosen from survival
    probabilities two steps old (a_lag) by the global maximum of Theta over
    every budget b = 0..N (early stop removed; the smallest b on a tie); the
    current step then admits the K candidates with the largest current
    survival a_cur (same order as `schedule`: a descending, index ascending).

    Returns (ell[R], K, Theta_lag(K) in tokens/s, Theta_fixed_lag[0..N])."""
    a_lag = np.asarray(a_lag, dtype=np.float32)
    a_cur = np.asarray(a_cur, dtype=np.float32)
    R, g = a_cur.shape
    N = R * g
    order_lag = np.argsort(-a_lag.reshape(-1).astype(np.float64), kind="stable")
    q = tau_fixed_units(a_lag.reshape(-1)[order_lag])
    G = np.concatenate([[0], np.cumsum(q)]).astype(np.int64)
    theta_fix = (np.int64(R) * TAU_ONE + G).astype(np.float64) * \
        np.asarray(sps, dtype=np.float64)[R + np.arange(N + 1)]
    K = int(np.argmax(theta_fix))                  # first (smallest) b of the maximum
    order_cur = np.argsort(-a_cur.reshape(-1).astype(np.float64), kind="stable")
    ell = np.bincount(order_cur[:K] // g, minlength=R).astype(np.int64)
    return ell, K, float(theta_fix[K]) * 2.0 ** -32, theta_fix


# ----------------------------------------------------------------------------
# Training objective                                       [P1 §5; P3 アーキテクチャ]
# ----------------------------------------------------------------------------
LOSS_ALPHAS = (0.1, 0.9, 1.0)   # alpha_CE, alpha_TV, alpha_conf (P1 §5 and P3 defaults)


def position_weights(gamma, lam):
    """w_k = exp(-(k-1)/lambda), k = 1..gamma  [P1 §5]; P3 writes the same
    weight with lambda = gamma."""
    return np.exp(-np.arange(gamma, dtype=np.float64) / float(lam))


def train_losses(U, target, W1, W2t, h, w, x_star, T=1.0, lam=None, alphas=LOSS_ALPHAS):
    """The three training losses of one batch of drafted blocks  [P1 §5]:

        L_CE   = -sum_k w_k log p_k^d(x*_k)
        L_TV   =  sum_k w_k ||p_k^d - p_k^t||_1
        L_conf = -sum_k w_k [c*_k log c_k + (1 - c*_k) log(1 - c_k)]
        L      = a_CE L_CE + a_TV L_TV + a_conf L_conf,

    with c*_k = 1 - 1/2 ||p_k^d - p_k^t||_1 (the acceptance probability, a
    constant target here) and c_k the confidence head.  The Markov head and the
    confidence head see the target block x* (teacher forcing): position k uses
    x*_{k-1}, x*_0 being the anchor.  U, target: [n, gamma, V]; h: [n, gamma, d];
    x_star: [n, gamma + 1]; lam defaults to gamma.

    Returns a dict of per-position terms [n, gamma] (ce, tv, conf, c, c_star),
    the weights w [gamma], the per-loss sums over the batch and the total L."""
    U = np.asarray(U, dtype=np.float64)
    n, g, V = U.shape
    lam = g if lam is None else lam
    wk = position_weights(g, lam)
    x_star = np.asarray(x_star, dtype=np.int64)
    ce = np.zeros((n, g)); tv = np.zeros((n, g)); cf = np.zeros((n, g))
    c = np.zeros((n, g)); cs = np.zeros((n, g))
    for i in range(n):
        z_d = draft_logits(U[i], W1, W2t, x_star[i, :g])             # rows k = 1..g
        logp_d, _ = log_softmax_rows(z_d / T)
        logp_t, _ = log_softmax_rows(np.asarray(target[i], dtype=np.float64) / T)
        p_d, p_t = np.exp(logp_d), np.exp(logp_t)
        ce[i] = -logp_d[np.arange(g), x_star[i, 1:]]
        tv[i] = np.abs(p_d - p_t).sum(axis=-1)
        cs[i] = 1.0 - 0.5 * tv[i]
        c[i] = confidence(as_f64(h[i]), w, W1, x_star[i, :g])
        cf[i] = -(cs[i] * np.log(c[i]) + (1.0 - cs[i]) * np.log1p(-c[i]))
    sums = {"ce": float((ce * wk).sum()), "tv": float((tv * wk).sum()),
            "conf": float((cf * wk).sum())}
    total = alphas[0] * sums["ce"] + alphas[1] * sums["tv"] + alphas[2] * sums["conf"]
    return {"ce": ce, "tv": tv, "conf": cf, "c": c, "c_star": cs, "w": wk, "sums": sums,
            "total": total}


def train_loss_grads(U, target, W1, W2t, h, w, x_star, T=1.0, lam=None, alphas=LOSS_ALPHAS):
    """Gradients of L = a_CE L_CE + a_TV L_TV + a_conf L_conf  [P1 §5] (c* held
    constant, as a target), written out from the definitions:

      dL/dz_v  = (w_k / T) [a_CE (p_d(v) - 1[v = x*_k]) + a_TV p_d(v) (s_v - mu)],
                 s_v = sign(p_d(v) - p_t(v)) (0 on equality), mu = sum_u s_u p_d(u);
                 z = U + e.W2, so dL/dU = dL/dz and dL/dbias = dL/dz;
      dL/dl    = w_k a_conf (c - c*) for the confidence logit l = w.[h; e];
      dL/dW2t  = sum_rows dL/dz (outer) e;   dL/de = dL/dz . W2t + dL/dl w[d:];
      dL/dh    = dL/dl w[:d];                dL/dw = sum_rows dL/dl [h; e].

    Returns dU [n, gamma, V], dW2t [V, rank], dE [n, gamma, rank] (with respect
    to the gathered rows e = W1[x*_{k-1}]; dW1 is their scatter-add), dh
    [n, gamma, d], dw [d + rank] and dl [n, gamma]; and, for checking a
    computation that decides the signs s_v in another precision, p_d, p_t
    [n, gamma, V], mu [n, gamma] and the factors w_k a_CE / T, w_k a_TV / T
    [gamma] of the two terms of dU."""
    U = np.asarray(U, dtype=np.float64)
    n, g, V = U.shape
    lam = g if lam is None else lam
    wk = position_weights(g, lam)
    x_star = np.asarray(x_star, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    d = np.asarray(h).shape[-1]
    rank = W1.shape[1]
    dU = np.zeros((n, g, V)); dW2t = np.zeros((V, rank)); dE = np.zeros((n, g, rank))
    dh = np.zeros((n, g, d)); dw = np.zeros(d + rank); dl = np.zeros((n, g))
    P_d = np.zeros((n, g, V)); P_t = np.zeros((n, g, V)); MU = np.zeros((n, g))
    a_ce, a_tv, a_cf = alphas
    for i in range(n):
        e = W1[x_star[i, :g]]                                       # [g, rank]
        z_d = np.asarray(U[i]) + e @ W2t.T
        p_d = np.exp(log_softmax_rows(z_d / T)[0])
        p_t = np.exp(log_softmax_rows(np.asarray(target[i], dtype=np.float64) / T)[0])
        sgn = np.sign(p_d - p_t)
        mu = (sgn * p_d).sum(axis=-1, keepdims=True)
        P_d[i], P_t[i], MU[i] = p_d, p_t, mu[:, 0]
        onehot = np.zeros_like(p_d)
        onehot[np.arange(g), x_star[i, 1:]] = 1.0
        gz = (wk[:, None] / T) * (a_ce * (p_d - onehot) + a_tv * p_d * (sgn - mu))
        dU[i] = gz
        dW2t += gz.T @ e
        hi = as_f64(h[i])
        c = sigmoid(hi @ w[:d] + e @ w[d:])
        cs = 1.0 - 0.5 * np.abs(p_d - p_t).sum(axis=-1)
        dl[i] = wk * a_cf * (c - cs)
        dE[i] = gz @ W2t + dl[i][:, None] * w[d:]
        dh[i] = dl[i][:, None] * w[:d]
        dw[:d] += dl[i] @ hi
        dw[d:] += dl[i] @ e
    return {"dU": dU, "dW2t": dW2t, "dE": dE, "dh": dh, "dw": dw, "dl": dl,
            "p_d": P_d, "p_t": P_t, "mu": MU,
            "f_ce": wk * a_ce / T, "f_tv": wk * a_tv / T}


def schedule_exhaustive(a, sps):
    """max over all ell in {0..gamma}^R of Theta(ell) (tiny R, gamma only)."""
    a = np.asarray(a, dtype=np.float32)
    R, g = a.shape
    best, arg = -np.inf, None
    for ell in itertools.product(range(g + 1), repeat=R):
        th = theta_of_ell(a, ell, sps)
        if th > best:
            best, arg = th, np.array(ell)
    return best, arg


# ----------------------------------------------------------------------------
# Verification: c* and lossless rejection sampling      [P1 §3.1, §2.2; P3]
# ----------------------------------------------------------------------------
def tv_acceptance(p_d, p_t):
    """c* = 1 - 1/2 ||p_d - p_t||_1  [P1 §3.1, eq. c*]."""
    return 1.0 - 0.5 * np.abs(np.asarray(p_d) - np.asarray(p_t)).sum(axis=-1)


def verify(U, Tl, W1, W2t, x, ell, T, seed, req_ids, E=None):
    """Per-position c* for all gamma positions, then standard rejection sampling
    over each request's admitted prefix (positions 1..ell_r).

    U, Tl: [n, gamma, V] draft base logits and target logits; x: [n, gamma+1]
    token block (x[:,0] = anchor); ell: [n].  Returns a dict with c_star
    [n,gamma], overlap [n,gamma] (= sum min(p_d, p_t)), n_accept [n],
    next_token [n], tau [n] and per-request diagnostics for near-tie counting.
    E [n, gamma, rank], if given, holds the bias rows of each position in place
    of W1[x_{k-1}] (blocks drafted by the RNN head).
    """
    U = np.asarray(U)
    n, g, V = U.shape
    x = np.asarray(x, dtype=np.int64)
    ell = np.asarray(ell, dtype=np.int64)
    v = np.arange(V, dtype=np.uint32)
    out = {k: [] for k in ("c_star", "overlap", "n_accept", "next_token", "tau",
                           "accept_margin", "sample_gap", "p_d_x", "p_t_x")}
    for i in range(n):
        req = int(req_ids[i])
        if E is None:
            z_d = draft_logits(U[i], W1, W2t, x[i, :g])          # rows k = 1..gamma
        else:
            z_d = np.asarray(U[i], dtype=np.float64) + np.asarray(E[i], dtype=np.float64) @ W2t.T
        z_t = np.asarray(Tl[i], dtype=np.float64)
        # greedy drafting's law at position k is the point mass on its drafted token
        if T > 0:
            p_d = draft_distribution(z_d, T)
        else:
            p_d = np.zeros((g, V))
            p_d[np.arange(g), x[i, 1:]] = 1.0
        p_t = draft_distribution(z_t, T)
        out["c_star"].append(tv_acceptance(p_d, p_t))
        out["overlap"].append(np.minimum(p_d, p_t).sum(axis=-1))
        rows = np.arange(g)
        # the kept draft probability of each drafted token; under greedy drafting
        # the draft law at position j is the point mass on the drafted x_j itself
        pdx = p_d[rows, x[i, 1:]]
        ptx = p_t[rows, x[i, 1:]]
        out["p_d_x"].append(pdx)
        out["p_t_x"].append(ptx)
        n_acc, nxt, margin, gap = 0, None, [], np.inf
        for j in range(1, ell[i] + 1):
            ratio = np.inf if pdx[j - 1] == 0 else ptx[j - 1] / pdx[j - 1]
            u = float(uniforms(seed, STREAM_ACCEPT, req, j, 0))
            margin.append(abs(u - ratio) if np.isfinite(ratio) else np.inf)
            if u < ratio:
                n_acc += 1
                continue
            r = np.maximum(p_t[j - 1] - p_d[j - 1], 0.0)
            G = gumbel(uniforms(seed, STREAM_RESID, req, j, v))
            if np.any(r > 0):
                with np.errstate(divide="ignore"):
                    keys = np.where(r > 0, np.log(r), -np.inf) + G
            else:
                keys = (z_t[j - 1] / T if T > 0 else np.where(p_t[j - 1] > 0, 0.0, -np.inf)) + G
            xs, gp = _top2(keys[None, :])
            nxt, gap = int(xs[0]), float(gp[0])
            break
        if nxt is None:
            if ell[i] < g:
                row = ell[i]
                if T > 0:
                    keys = z_t[row] / T + gumbel(uniforms(seed, STREAM_BONUS, req, row + 1, v))
                else:
                    keys = z_t[row]
                xs, gp = _top2(keys[None, :])
                nxt, gap = int(xs[0]), float(gp[0])
            else:
                nxt = -1
        out["n_accept"].append(n_acc)
        out["next_token"].append(nxt)
        out["tau"].append(n_acc + 1)
        out["accept_margin"].append(min(margin) if margin else np.inf)
        out["sample_gap"].append(gap)
    res = {k: np.array(vv) for k, vv in out.items()}
    res["tau_mean"] = float(np.mean(res["tau"])) if n else 0.0
    return res


# ----------------------------------------------------------------------------
# RNN head  [P1 §2.4; P3 アーキテクチャ]: a block-internal state s_k, updated
# by a gate from the previous state (the longer prefix), the previous token's
# embedding and the backbone state h_k.  The pages give no equations; the
# reading here is a GRU cell in the convention of torch.nn.GRUCell over the
# input [e_k; h_k], e_k = W1[x_{k-1}], hidden size rank, s_0 = 0, and the
# state takes the place of e_k in the bias: B_k = bf16(s_k) W2 (the state
# enters the rank -> vocabulary projection in the weights' precision).
# ----------------------------------------------------------------------------
def bf16_round(x):
    """Round-to-nearest-even to bf16, returned as fp64 (finite inputs)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return bf16_to_f64(r)


def gru_cell(x_in, s, W_ih, W_hh, b_ih, b_hh):
    """One GRU update, gate order (reset, update, new):
       r = sigma(W_ir x + b_ir + W_hr s + b_hr)
       z = sigma(W_iz x + b_iz + W_hz s + b_hz)
       n = tanh(W_in x + b_in + r * (W_hn s + b_hn))
       s' = (1 - z) n + z s
    x_in [n, rank + d], s [n, rank]; W_ih [3 rank, rank + d], W_hh [3 rank, rank]."""
    H = s.shape[-1]
    gi = np.asarray(x_in, dtype=np.float64) @ W_ih.T + b_ih
    gh = np.asarray(s, dtype=np.float64) @ W_hh.T + b_hh
    r = sigmoid(gi[:, :H] + gh[:, :H])
    z = sigmoid(gi[:, H:2 * H] + gh[:, H:2 * H])
    n = np.tanh(gi[:, 2 * H:] + r * gh[:, 2 * H:])
    return (1.0 - z) * n + z * s


def rnn_draft_round(U, h, w, W1, W2t, gru, anchor, T, seed, req_ids):
    """gamma steps of the RNN head: s_k = gru(s_{k-1}, [W1[x_{k-1}]; h_k]), then the
    step of draft_step with bf16(s_k) as its rows; confidence and survival as
    for the Markov head (c_k from h_k and W1[x_{k-1}]).  gru = (W_ih, W_hh,
    b_ih, b_hh) in fp64.  Also returns the final state s_gamma and the bias rows
    bf16(s_k) of every position (what verification needs in place of W1[x])."""
    W_ih, W_hh, b_ih, b_hh = gru
    n, g, V = U.shape
    rank = W1.shape[1]
    x = np.empty((n, g + 1), dtype=np.int64)
    x[:, 0] = anchor
    p = np.empty((n, g)); lse = np.empty((n, g)); c = np.empty((n, g)); gap = np.empty((n, g))
    rows = np.empty((n, g, rank))
    st_ = np.zeros((n, rank))
    for k in range(1, g + 1):
        e = W1[x[:, k - 1]]
        hk = np.asarray(h[:, k - 1], dtype=np.float64)
        st_ = gru_cell(np.concatenate([e, hk], axis=1), st_, W_ih, W_hh, b_ih, b_hh)
        rows[:, k - 1] = bf16_round(st_)
        step = draft_step(U[:, k - 1], W1, W2t, x[:, k - 1], T, seed, k, req_ids, E=rows[:, k - 1])
        c[:, k - 1] = confidence(hk, w, W1, x[:, k - 1])
        x[:, k], p[:, k - 1], lse[:, k - 1], gap[:, k - 1] = step["x"], step["p"], step["lse"], step["gap"]
    return {"x": x, "p": p, "lse": lse, "c": c, "a": survival(c.astype(np.float32)),
            "state": st_, "gap": gap, "rows": rows}


# ----------------------------------------------------------------------------
# A whole draft round (free running), for the smoke check and the CPU baseline
# ----------------------------------------------------------------------------
def draft_round(U, h, w, W1, W2t, anchor, T, seed, req_ids):
    """gamma sequential steps [P1 §6.2 loop semantics: prev = sampled token],
    confidence and survival for each position.  Inputs in fp64/fp32 arrays:
    U [n,gamma,V], h [n,gamma,d], W1/W2t [V,rank]."""
    n, g, V = U.shape
    x = np.empty((n, g + 1), dtype=np.int64)
    x[:, 0] = anchor
    p = np.empty((n, g))
    lse = np.empty((n, g))
    c = np.empty((n, g))
    for k in range(1, g + 1):
        st = draft_step(U[:, k - 1], W1, W2t, x[:, k - 1], T, seed, k, req_ids)
        c[:, k - 1] = confidence(h[:, k - 1], w, W1, x[:, k - 1])
        x[:, k], p[:, k - 1], lse[:, k - 1] = st["x"], st["p"], st["lse"]
    c32 = c.astype(np.float32)
    return {"x": x, "p": p, "lse": lse, "c": c, "a": survival(c32)}

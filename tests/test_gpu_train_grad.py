"""GPU parity of the training gradients (dspark_train_loss_grad) against the
CPU oracle's train_loss_grads, through the C ABI [P1 §5; P1 §2.3, §3.1].

Tolerances, from the arithmetic of the two sides:
  dU    per element, 1e-3 of the magnitude of its two terms,
        (w_k/T) (a_CE (p_d + [v = x*]) + 2 a_TV p_d): the GPU's p_d and p_t
        carry fp32 normalisers and an fp32 MFMA bias.  Where the oracle's
        |p_d - p_t| is within 1e-5 of max(p_d, p_t), the sign s_v is decided
        by rounding, and every s_v in {-1, 0, 1} is a valid (sub)gradient of the
        L1 norm: there the GPU value must match one of the three.
  dE, dW1, dW2t   the contractions round dU to bf16 (relative error <= 2^-9)
        and accumulate in fp32: |error| <= 2^-7 sum |dU| |other operand|
        (twice the rounding bound, covering dU's own error), plus 1e-3 of
        |dl| |w| for the confidence term of dE.
  dh, dw   fp32 / fp64 sums of dl times bf16 inputs, dl = w_k a_conf (c - c*):
        1e-3 of w_k a_conf (|c| + |c*|) per position (c as in the loss tests).
"""
import numpy as np
import pytest
import torch

from oracle import dspark_oracle as O
from semi_autoregressive_drafting_amd import dspark as D, runner, synth
from tests.gpu_parity import say

pytestmark = pytest.mark.gpu

# ragged rows (111 = 3.5 row tiles) and a vocabulary tail with V % 4 != 0 at
# the smallest rank; a three-chunk rank with V % 4 == 0 and 200 rows
synth.custom("grad_v997_r37_g3", V=997, rank=32, d=40, gamma=3, R=37, dtype="bf16", peak="three")
synth.custom("grad_v1000_r100_g2", V=1000, rank=96, d=33, gamma=2, R=100, dtype="bf16",
             peak="three")
synth.custom("grad_v4099_r8_g5", V=4099, rank=64, d=72, gamma=5, R=8, dtype="bf16", peak="three")
# one request and one position: a single row in every tile and contraction
synth.custom("grad_v64_r1_g1", V=64, rank=32, d=16, gamma=1, R=1, dtype="bf16", peak="three")
# V % 8 == 4: the last vector load of a row holds 4 entries
synth.custom("grad_v1004_r20_g3", V=1004, rank=64, d=32, gamma=3, R=20, dtype="bf16", peak="three")
# the largest row count (R = 512, gamma = 16: 8192 rows, 64 row groups of the contractions)
synth.custom("grad_v1031_r512_g16", V=1031, rank=64, d=24, gamma=16, R=512, dtype="bf16",
             peak="three")


def _x_star(inp, seed, repeat=False):
    rng = np.random.default_rng(seed)
    wl = inp.wl
    hi = 7 if repeat else wl.V  # repeat: few distinct tokens, so dW1 rows collect many dE rows
    x = rng.integers(0, hi, (wl.R, wl.gamma + 1)).astype(np.int32)
    x[:, 0] = inp.anchor
    return x


def _run(inp, xs, T, lam, alphas=O.LOSS_ALPHAS):
    di = runner.DeviceInputs.upload(inp)
    out = runner.train_loss_grad(di, torch.from_numpy(xs).cuda(), T, lam, alphas)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}


def _check_dU(got_dU, G, xs, reqs):
    """dU of requests `reqs` against the oracle (G computed on those requests)."""
    pd, pt, mu = G["p_d"], G["p_t"], G["mu"][..., None]
    fce, ftv = G["f_ce"][None, :, None], G["f_tv"][None, :, None]
    afce, aftv = np.abs(fce), np.abs(ftv)  # term magnitudes (a weight may be negative)
    n, g, V = pd.shape
    hot = np.zeros_like(pd)
    for i in range(n):
        hot[i, np.arange(g), xs[reqs[i], 1:]] = 1.0
    scale = afce * (pd + hot) + 2.0 * aftv * pd
    tol = 1e-3 * scale + 1e-12
    err = np.abs(got_dU - G["dU"])
    bad = err > tol
    if bad.any():
        # sign decided by rounding: accept any s in {-1, 0, 1}
        tie = np.abs(pd - pt) <= 1e-5 * np.maximum(pd, pt)
        s_or = np.sign(pd - pt)
        ok_alt = np.zeros_like(bad)
        for s_alt in (-1.0, 0.0, 1.0):
            alt = G["dU"] + ftv * pd * (s_alt - s_or)
            ok_alt |= np.abs(got_dU - alt) <= tol
        still = bad & ~(tie & ok_alt)
        assert not still.any(), (
            f"dU: {int(still.sum())} of {still.size} off; worst "
            f"{float((err / tol)[still].max()):.3g} x tol at {np.argwhere(still)[0].tolist()}")
        say(f"  dU: {int(bad.sum())} near-tie signs decided by rounding")


def _dl_scale(got_terms, wk, a_conf):
    """w_k a_conf (|c| + |c*|) per position from the GPU's (checked) terms."""
    c = got_terms[..., 3]
    cs = 1.0 - 0.5 * got_terms[..., 1]
    return wk[None, :] * abs(a_conf) * (np.abs(c) + np.abs(cs))


def _check_all(name, T, lam, seed=5, repeat=False, alphas=O.LOSS_ALPHAS, inp=None, w64=None):
    """inp / w64: prebuilt inputs and their exact fp64 (W1, W2t), else the
    workload's generated ones."""
    say(f"[grad] {name} T={T} lambda={lam} repeat={repeat} alphas={alphas}")
    inp = synth.generate(name, seed=0, target=True) if inp is None else inp
    wl = inp.wl
    xs = _x_star(inp, seed, repeat)
    got = _run(inp, xs, T, lam, alphas)
    W1, W2t = (O.as_f64(inp.W1_store), O.as_f64(inp.W2t_store)) if w64 is None else w64
    h = O.as_f64(inp.h_store)
    # the library takes the weights in fp32
    alphas = tuple(float(np.float32(x)) for x in alphas)
    G = O.train_loss_grads(inp.U, inp.target, W1, W2t, inp.h_store, inp.w, xs, T=T, lam=lam,
                           alphas=alphas)
    reqs = np.arange(wl.R)
    _check_dU(got["dU"], G, xs, reqs)

    # dE through dW1 (scatter of the oracle's dE rows onto their tokens)
    aU = np.abs(G["dU"])
    E = W1[xs[:, :wl.gamma]]                                    # [R, g, rank]
    wd = np.asarray(inp.w, dtype=np.float64)
    lam_ = wl.gamma if lam is None else lam
    wk = O.position_weights(wl.gamma, lam_)
    dls = _dl_scale(got["terms"], wk, alphas[2])
    tol_dE = 2.0 ** -7 * (aU @ np.abs(W2t)) + 1e-3 * dls[..., None] * np.abs(wd[wl.d:]) + 1e-7
    dW1_ref = np.zeros_like(W1)
    dW1_tol = np.zeros_like(W1)
    np.add.at(dW1_ref, xs[:, :wl.gamma].reshape(-1), G["dE"].reshape(-1, wl.rank))
    np.add.at(dW1_tol, xs[:, :wl.gamma].reshape(-1), tol_dE.reshape(-1, wl.rank))
    err = np.abs(got["dW1"] - dW1_ref)
    assert (err <= dW1_tol + 1e-7).all(), f"dW1 worst {float((err / (dW1_tol + 1e-7)).max()):.3g} x tol"
    unused = np.setdiff1d(np.arange(wl.V), xs[:, :wl.gamma])
    assert (got["dW1"][unused] == 0).all()

    # dW2t = dU^T E
    tol_w2 = 2.0 ** -7 * np.einsum("rkv,rkj->vj", aU, np.abs(E)) + 1e-7
    err = np.abs(got["dW2t"] - G["dW2t"])
    assert (err <= tol_w2).all(), f"dW2t worst {float((err / tol_w2).max()):.3g} x tol"

    # confidence head
    tol_dh = 1e-3 * dls[..., None] * np.abs(wd[None, None, :wl.d]) + 1e-9
    assert (np.abs(got["dh"] - G["dh"]) <= tol_dh).all(), "dh"
    feat = np.concatenate([h, E], axis=-1)                      # [R, g, d + rank]
    tol_dw = 1e-3 * np.einsum("rk,rkj->j", dls, np.abs(feat)) + 1e-7
    assert (np.abs(got["dw"] - G["dw"]) <= tol_dw).all(), "dw"

    # the losses themselves match the forward entry point's
    o = O.train_losses(inp.U, inp.target, W1, W2t, inp.h_store, inp.w, xs, T=T, lam=lam,
                       alphas=alphas)
    np.testing.assert_allclose(got["terms"][..., 1], o["tv"], rtol=1e-3, atol=1e-5)
    assert got["sums"][3] == pytest.approx(o["total"], rel=1e-3)
    say("  ok")
    return got


@pytest.mark.parametrize("name,T,lam,repeat", [
    ("grad_v997_r37_g3", 1.0, None, False),
    ("grad_v997_r37_g3", 0.7, 2.0, True),
    ("grad_v1000_r100_g2", 1.3, 5.0, False),
    ("grad_v4099_r8_g5", 1.0, None, True),
    ("grad_v64_r1_g1", 1.0, None, False),
    ("grad_v1004_r20_g3", 1.0, None, True),
    ("grad_v1031_r512_g16", 1.0, None, True),
])
def test_train_grads_small(name, T, lam, repeat):
    _check_all(name, T, lam, repeat=repeat)


def test_train_grads_other_weights_and_temperature():
    """Non-default loss weights (a negative one included) and a low temperature."""
    _check_all("grad_v1000_r100_g2", 0.5, 1.5, alphas=(0.3, -0.25, 2.0))


def test_train_grads_deterministic():
    inp = synth.generate("grad_v1000_r100_g2", seed=0, target=True)
    xs = _x_star(inp, 9, repeat=True)
    a = _run(inp, xs, 1.0, None)
    b = _run(inp, xs, 1.0, None)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_train_grads_full_size():
    """Full vocabulary, rank 256, R = 128, gamma = 7 (896 rows: 7 groups of
    128, 32-entry vocabulary tiles over 151936 entries).  dU against the
    oracle on a spread sample of 8 requests; the contractions against fp64
    sums of the GPU's own dU on sampled rows / vocabulary entries (the
    property dE = dU . W2t + dl w[d:], dW2t = dU^T E at any size)."""
    name = "round_4b_r128_g7"
    say(f"[grad] {name} full size")
    inp = synth.generate(name, seed=0, target=True)
    wl = inp.wl
    xs = _x_star(inp, 11)
    got = _run(inp, xs, 1.0, None)
    W1, W2t = O.as_f64(inp.W1_store), O.as_f64(inp.W2t_store)
    reqs = np.linspace(0, wl.R - 1, 8).round().astype(int)
    G = O.train_loss_grads(inp.U[reqs], inp.target[reqs], W1, W2t, inp.h_store[reqs], inp.w,
                           xs[reqs], T=1.0)
    _check_dU(got["dU"][reqs], G, xs, reqs)
    # dW2t on sampled vocabulary entries against the GPU's dU
    dU = got["dU"].reshape(-1, wl.V)
    E = W1[xs[:, :wl.gamma]].reshape(-1, wl.rank)
    rng = np.random.default_rng(4)
    vs = np.concatenate([rng.choice(wl.V, 60, replace=False), [0, wl.V - 1]])
    for v in vs:
        ref = dU[:, v] @ E
        tol = 2.0 ** -7 * (np.abs(dU[:, v]) @ np.abs(E)) + 1e-7
        assert (np.abs(got["dW2t"][v] - ref) <= tol).all(), f"dW2t row {v}"
    # dW1 on the tokens of sampled rows: scatter of dE = dU . W2t + dl w[d:]
    wk = O.position_weights(wl.gamma, wl.gamma)
    c = got["terms"][..., 3].reshape(-1)
    cs = 1.0 - 0.5 * got["terms"][..., 1].reshape(-1)
    wkr = np.tile(wk, wl.R)
    dl = wkr * O.LOSS_ALPHAS[2] * (c - cs)
    wd = np.asarray(inp.w, dtype=np.float64)
    toks = xs[:, :wl.gamma].reshape(-1)
    for t in np.unique(toks[rng.choice(len(toks), 6, replace=False)]):
        rows = np.nonzero(toks == t)[0]
        ref = sum(dU[r] @ W2t + dl[r] * wd[wl.d:] for r in rows)
        tol = sum(2.0 ** -7 * (np.abs(dU[r]) @ np.abs(W2t))
                  + 1e-3 * wkr[r] * (abs(c[r]) + abs(cs[r])) * np.abs(wd[wl.d:]) for r in rows) + 1e-7
        assert (np.abs(got["dW1"][t] - ref) <= tol).all(), f"dW1 row {t}"
    say("  ok")


def test_train_grad_rejects_fp32_weights():
    """The gradient entry point takes bf16 weights only."""
    inp = synth.generate("tiny_v1024_r4_g4", seed=0, target=True)
    xs = _x_star(inp, 1)
    with pytest.raises(D.DsparkError):
        _run(inp, xs, 1.0, None)


def test_train_grads_max_vocabulary():
    """Two rows (one request, gamma = 2) at the largest vocabulary, V = 2^24;
    the weights are a random 4096-row block tiled down the vocabulary."""
    import dataclasses
    V = 1 << 24
    small = synth.custom("grad_block_v4096_r1_g2", V=4096, rank=32, d=16, gamma=2, R=1,
                         dtype="bf16", peak="three", target=True)
    wl = synth.custom("grad_v16777216_r1_g2", V=V, rank=32, d=16, gamma=2, R=1, dtype="bf16",
                      peak="three", target=True)
    base = synth.generate(small.name, seed=0)
    rng = np.random.default_rng(2025)
    U = rng.standard_normal((1, 2, V), dtype=np.float32) * np.float32(2.0)
    target = U + rng.standard_normal((1, 2, V), dtype=np.float32)
    inp = dataclasses.replace(base, wl=wl, U=U, target=target,
                              W1_store=np.tile(base.W1_store, (V // 4096, 1)),
                              W2t_store=np.tile(base.W2t_store, (V // 4096, 1)),
                              anchor=np.array([V - 1], dtype=np.int32))
    w64 = (np.tile(O.as_f64(base.W1_store), (V // 4096, 1)),
           np.tile(O.as_f64(base.W2t_store), (V // 4096, 1)))
    _check_all(wl.name, 1.0, None, inp=inp, w64=w64)

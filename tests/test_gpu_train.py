"""GPU parity of the training losses (L_CE, L_TV, L_conf with position weights,
P1 §5) against the CPU oracle, through the C ABI.  The Markov and confidence
heads see the target block x* (teacher forcing).

Tolerances: ce 2e-3 absolute (a difference of two log-normalisers, as the
logits' 2e-3); tv and c* 1e-3 relative with a 1e-5 absolute floor (as c* in
verification); c 1e-3 relative (as c_k); conf 2e-3 absolute; weighted sums
1e-3 relative."""
import numpy as np
import pytest
import torch

from oracle import dspark_oracle as O
from semi_autoregressive_drafting_amd import runner, synth
from tests.gpu_parity import say

pytestmark = pytest.mark.gpu

# a vocabulary tail with V % 4 != 0 and the smallest rank; a shared-shape rank
# without the compile-time MFMA loop
synth.custom("train_v997_r37_g3", V=997, rank=16, d=40, gamma=3, R=37, dtype="bf16", peak="three")
synth.custom("train_v1000_r100_g2", V=1000, rank=48, d=33, gamma=2, R=100, dtype="bf16",
             peak="three")


def _x_star(inp, seed):
    rng = np.random.default_rng(seed)
    wl = inp.wl
    x = rng.integers(0, wl.V, (wl.R, wl.gamma + 1)).astype(np.int32)
    x[:, 0] = inp.anchor
    return x


def _check(name, T, lam, reqs=None, seed=3):
    say(f"[train] {name} T={T} lambda={lam}")
    inp = synth.generate(name, seed=0, target=True)
    wl = inp.wl
    di = runner.DeviceInputs.upload(inp)
    xs = _x_star(inp, seed)
    terms, sums = runner.train_loss(di, torch.from_numpy(xs).cuda(), T, lam)
    torch.cuda.synchronize()
    terms = terms.cpu().numpy().astype(np.float64)
    sums = sums.cpu().numpy()
    reqs = np.arange(wl.R) if reqs is None else np.asarray(reqs)
    W1, W2t = O.as_f64(inp.W1_store), O.as_f64(inp.W2t_store)
    o = O.train_losses(inp.U[reqs], inp.target[reqs], W1, W2t, inp.h_store[reqs], inp.w, xs[reqs],
                       T=T, lam=lam)
    g = terms[reqs]
    np.testing.assert_allclose(g[..., 0], o["ce"], rtol=0, atol=2e-3, err_msg="ce")
    np.testing.assert_allclose(g[..., 1], o["tv"], rtol=1e-3, atol=1e-5, err_msg="tv")
    np.testing.assert_allclose(g[..., 3], o["c"], rtol=1e-3, atol=0, err_msg="c")
    np.testing.assert_allclose(g[..., 2], o["conf"], rtol=0, atol=2e-3, err_msg="conf")
    # the weighted sums: against the oracle on the full batch, and always
    # against the GPU's own terms with the oracle's weights
    wk = O.position_weights(wl.gamma, wl.gamma if lam is None else lam)
    own = [(terms[..., j] * wk).sum() for j in range(3)]
    np.testing.assert_allclose(sums[:3], own, rtol=1e-5)
    a = [float(np.float32(x)) for x in O.LOSS_ALPHAS]  # the library takes fp32 weights
    assert sums[3] == pytest.approx(a[0] * sums[0] + a[1] * sums[1] + a[2] * sums[2], rel=1e-12)
    if len(reqs) == wl.R:
        np.testing.assert_allclose(sums[:3], [o["sums"]["ce"], o["sums"]["tv"], o["sums"]["conf"]],
                                   rtol=1e-3)
        assert sums[3] == pytest.approx(o["total"], rel=1e-3)
    say(f"  ok: sums {np.round(sums, 4).tolist()}")
    return terms, sums


@pytest.mark.parametrize("name,T,lam", [
    ("tiny_v1024_r4_g4", 1.0, None), ("tiny_v1024_r4_g4", 0.6, 2.0),
    ("train_v997_r37_g3", 1.0, None), ("train_v1000_r100_g2", 1.3, 5.0),
])
def test_train_losses_small(name, T, lam):
    _check(name, T, lam)


def test_train_losses_full_size():
    """Full vocabulary, rank 256, R = 128, gamma = 7 (the production c* pass
    and the line-coalesced draft-normaliser pass); the oracle checks a spread
    sample of 12 requests."""
    _check("round_4b_r128_g7", 1.0, None, reqs=np.linspace(0, 127, 12).round().astype(int))


def test_train_losses_deterministic():
    inp = synth.generate("round_4b_r128_g7", seed=0, target=True)
    di = runner.DeviceInputs.upload(inp)
    xs = torch.from_numpy(_x_star(inp, 9)).cuda()
    t1, s1 = runner.train_loss(di, xs)
    t2, s2 = runner.train_loss(di, xs)
    torch.cuda.synchronize()
    assert torch.equal(t1, t2) and torch.equal(s1, s2)

"""GPU parity of the RNN head's draft block (dspark_draft_block_rnn) against the
CPU oracle's GRU reading of P1 §2.4, through the C ABI.

Teacher-forced per step, as for the Markov head: the oracle's state is driven
by the GPU's tokens, so a near-tie flip at one step does not cascade.  Same
tolerances as the Markov head (tokens may differ only where the GPU's token
is within 1e-3 of the oracle's top perturbed score at both levels of the
sampler, 0.1% at most; p_k and c_k 1e-3 relative; lse
1e-4; survival bit-exact) plus the final state s_gamma within 1e-4 absolute
(fp32 gates and a two-term bf16 split of the state in the recurrent product,
against fp64).  The state enters the bias rounded to bf16 on both sides; the
two roundings can differ by one bf16 step where the fp32 and fp64 states
straddle a rounding boundary, which moves a logit by far less than the 2e-3
logit tolerance that the near-tie rule is built on."""
import numpy as np
import pytest
import torch

from oracle import dspark_oracle as O
from semi_autoregressive_drafting_amd import dspark as D, runner, synth
from tests.gpu_parity import LSE_ATOL, NEAR_TIE, P_RTOL, Z_TOL, say

pytestmark = pytest.mark.gpu

# ragged vocabulary (V % 4 != 0) and request counts that leave part of a
# request tile padded, with the smallest ranks
synth.custom("rnn_v997_r37_g3", V=997, rank=32, d=48, gamma=3, R=37, dtype="bf16", peak="three")
synth.custom("rnn_v4099_r20_g5", V=4099, rank=64, d=80, gamma=5, R=20, dtype="bf16", peak="three")
# one request, a vocabulary below one MFMA tile pair, the smallest d
synth.custom("rnn_v50_r1_g2", V=50, rank=32, d=16, gamma=2, R=1, dtype="bf16", peak="three")
# the largest batch and block (R = 512, gamma = 16) at the largest rank
synth.custom("rnn_v1031_r512_g16", V=1031, rank=256, d=32, gamma=16, R=512, dtype="bf16",
             peak="three")

STATE_ATOL = 1e-4


def _run(name, T, seed):
    inp = synth.generate(name, seed=0)
    wl = inp.wl
    di = runner.DeviceInputs.upload(inp)
    buf = runner.RoundBuffers.allocate(di)
    gru = synth.gru_weights(wl, 0)
    rw = runner.RnnWeights.upload(gru)
    state = torch.empty((wl.R, wl.rank), dtype=torch.float32, device="cuda")
    nb = D.dspark_workspace_bytes(D.DSPARK_OP_DRAFT_RNN, wl.R, wl.V, wl.rank, wl.gamma)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    runner.draft_rnn(di, buf, rw, T, seed, state, ws)
    torch.cuda.synchronize()
    host = {n: getattr(buf, n).cpu().numpy() for n in ("x", "p", "lse", "c", "a")}
    host["state"] = state.cpu().numpy()
    return inp, gru, host, (di, buf, rw, state, ws)


def _check(inp, gru, host, T, seed, reqs=None):
    wl = inp.wl
    reqs = np.arange(wl.R) if reqs is None else np.asarray(reqs)
    W1, W2t = O.as_f64(inp.W1_store), O.as_f64(inp.W2t_store)
    g64 = (O.as_f64(gru[0]), O.as_f64(gru[1]), gru[2].astype(np.float64), gru[3].astype(np.float64))
    h = O.as_f64(inp.h_store)
    x = host["x"].astype(np.int64)
    s = np.zeros((len(reqs), wl.rank))
    flips = 0
    for k in range(1, wl.gamma + 1):
        s = O.gru_cell(np.concatenate([W1[x[reqs, k - 1]], h[reqs, k - 1]], axis=1), s, *g64)
        st = O.draft_step(inp.U[reqs, k - 1].astype(np.float64), W1, W2t, x[reqs, k - 1], T, seed, k,
                          reqs, E=O.bf16_round(s))
        xg = x[reqs, k]
        assert np.all((xg >= 0) & (xg < wl.V)), f"step {k}: token id out of range"
        flip = xg != st["x"]
        for i in np.nonzero(flip)[0]:
            dfc = O.draft_token_deficit(st, i, int(xg[i]), T, seed, k, int(reqs[i]))
            assert dfc < NEAR_TIE, f"step {k} req {reqs[i]}: token mismatch away from a near tie ({dfc})"
        flips += int(flip.sum())
        if T > 0:
            p_or = np.exp(st["z"][np.arange(len(reqs)), xg] / T - st["lse"])
            lse_err = np.abs(host["lse"][reqs, k - 1] - st["lse"])
            assert lse_err.max() < LSE_ATOL * max(1.0, np.abs(st["lse"]).max()), lse_err.max()
        else:
            p_or = np.ones(len(reqs))
            assert np.abs(host["lse"][reqs, k - 1] - st["lse"]).max() < Z_TOL
        p_rel = np.abs(host["p"][reqs, k - 1] - p_or) / p_or
        assert p_rel.max() < P_RTOL, f"step {k}: p rel err {p_rel.max()}"
        c_or = O.confidence(h[reqs, k - 1], inp.w, W1, x[reqs, k - 1])
        assert (np.abs(host["c"][reqs, k - 1] - c_or) / c_or).max() < P_RTOL
    np.testing.assert_array_equal(host["a"], O.survival(host["c"]))
    err = np.abs(host["state"][reqs] - s).max()
    assert err < STATE_ATOL, f"final state abs err {err}"
    samples = len(reqs) * wl.gamma
    assert flips <= max(0, int(1e-3 * samples)) or (samples < 1000 and flips == 0), flips
    say(f"  ok: {samples} samples, {flips} near-tie flips, state err {err:.2e}")


@pytest.mark.parametrize("name,T", [
    ("rnn_v997_r37_g3", 1.0), ("rnn_v997_r37_g3", 0.0), ("rnn_v4099_r20_g5", 0.7),
    ("rnn_v50_r1_g2", 1.0), ("rnn_v1031_r512_g16", 1.0),
])
def test_rnn_draft_block_small(name, T):
    say(f"[rnn] {name} T={T}")
    inp, gru, host, _ = _run(name, T, 21)
    _check(inp, gru, host, T, 21)


def test_rnn_draft_block_full_size_greedy():
    """Greedy drafting with the RNN head at R = 32, gamma = 7 (one request group
    with three padded request tiles), full vocabulary, rank 256."""
    name = "qwen3_4b_r32_g7"
    say(f"[rnn] {name} T=0")
    inp, gru, host, _ = _run(name, 0.0, 3)
    _check(inp, gru, host, 0.0, 3, np.linspace(0, inp.wl.R - 1, 6).round().astype(int))


def test_rnn_draft_block_full_size_and_repeatable():
    """The headline shape (R = 128, gamma = 16, V = 151936, rank 256, d 4096):
    a spread sample of 6 requests against the oracle; a second call on the
    same workspace gives identical bits."""
    name = "qwen3_8b_r128_g16"
    say(f"[rnn] {name}")
    inp, gru, host, (di, buf, rw, state, ws) = _run(name, 1.0, 5)
    reqs = np.linspace(0, inp.wl.R - 1, 6).round().astype(int)
    _check(inp, gru, host, 1.0, 5, reqs)
    runner.draft_rnn(di, buf, rw, 1.0, 5, state, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(buf.x.cpu().numpy(), host["x"])
    np.testing.assert_array_equal(buf.p.cpu().numpy(), host["p"])
    np.testing.assert_array_equal(state.cpu().numpy(), host["state"])


@pytest.mark.parametrize("name,V,R,gamma", [
    ("rnn_round_v4099_r40_g4", 4099, 40, 4),
    # gamma = 16: the c* pass also runs the sampling race, here with bias rows
    ("rnn_round_v3001_r6_g16", 3001, 6, 16),
])
def test_rnn_round_verifies_against_its_own_rows(name, V, R, gamma):
    """Draft with the RNN head (bias rows written out), schedule, verify with
    those rows.  The oracle rebuilds the rows from the GPU's tokens through its
    own GRU and verifies with them: c* within 1e-3, accept decisions and
    next tokens exact away from near ties; the GPU's rows equal the oracle's up
    to one bf16 step plus the state tolerance."""
    from tests.test_gpu_verify import ACCEPT_NEAR_TIE, CSTAR_ATOL, CSTAR_RTOL
    synth.custom(name, V=V, rank=64, d=48, gamma=gamma, R=R, dtype="bf16", peak="three",
                 target=True)
    inp = synth.generate(name, seed=0, target=True)
    wl = inp.wl
    di = runner.DeviceInputs.upload(inp)
    buf = runner.RoundBuffers.allocate(di)
    gru = synth.gru_weights(wl, 0)
    rw = runner.RnnWeights.upload(gru)
    state = torch.empty((wl.R, wl.rank), dtype=torch.float32, device="cuda")
    rows = torch.empty((wl.R, wl.gamma, wl.rank), dtype=torch.int16, device="cuda")
    nb = D.dspark_workspace_bytes(D.DSPARK_OP_DRAFT_RNN, wl.R, wl.V, wl.rank, wl.gamma)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    T, seed = 1.0, 41
    runner.draft_rnn(di, buf, rw, T, seed, state, ws, rows)
    runner.schedule(di, buf)
    runner.verify_rnn(di, buf, rows, T, seed)
    torch.cuda.synchronize()
    g = {n: getattr(buf, n).cpu().numpy() for n in ("x", "ell", "c_star", "n_accept", "next_token",
                                                    "tau")}
    rows_g = O.bf16_to_f64(rows.cpu().numpy().view(np.uint16))
    # oracle rows from the GPU's tokens
    W1, W2t = O.as_f64(inp.W1_store), O.as_f64(inp.W2t_store)
    g64 = (O.as_f64(gru[0]), O.as_f64(gru[1]), gru[2].astype(np.float64), gru[3].astype(np.float64))
    h = O.as_f64(inp.h_store)
    x = g["x"].astype(np.int64)
    s = np.zeros((wl.R, wl.rank))
    rows_o = np.empty((wl.R, wl.gamma, wl.rank))
    for k in range(1, wl.gamma + 1):
        s = O.gru_cell(np.concatenate([W1[x[:, k - 1]], h[:, k - 1]], axis=1), s, *g64)
        rows_o[:, k - 1] = O.bf16_round(s)
    # one bf16 step of the value, plus the state's own absolute error
    row_err = np.abs(rows_g - rows_o) - (2.0 ** -7 * np.abs(rows_o) + STATE_ATOL)
    assert (row_err <= 0).all(), f"rows: worst excess {row_err.max():.3g} at {np.unravel_index(row_err.argmax(), row_err.shape)}"
    res = O.verify(inp.U, inp.target, W1, W2t, x, g["ell"], T, seed, np.arange(wl.R), E=rows_o)
    cs_o = res["c_star"]
    assert np.all(np.abs(g["c_star"] - cs_o) <= np.maximum(CSTAR_ATOL, CSTAR_RTOL * np.abs(cs_o)))
    near = (res["accept_margin"] < ACCEPT_NEAR_TIE) | (res["sample_gap"] < NEAR_TIE)
    ok = ((g["n_accept"] == res["n_accept"]) & (g["next_token"] == res["next_token"])
          & (g["tau"] == res["tau"]))
    assert np.all(ok | near), np.nonzero(~ok & ~near)
    # with the Markov rows the acceptance outcome would differ: the rows matter
    res_m = O.verify(inp.U, inp.target, W1, W2t, x, g["ell"], T, seed, np.arange(wl.R))
    assert np.abs(res_m["c_star"] - cs_o).max() > 1e-3
    say(f"  ok: budget {g['ell'].sum()}, tau mean {g['tau'].mean():.3f}")

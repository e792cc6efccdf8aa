"""GPU parity of verification (per-position c*, acceptance chain, residual /
bonus resampling, realised tau) against the oracle, fed the GPU's own drafted
block and admitted lengths."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import dspark_oracle as O
from semi_autoregressive_drafting_amd import runner, synth
from tests.gpu_parity import Case, NEAR_TIE, say

pytestmark = pytest.mark.gpu

CSTAR_RTOL, CSTAR_ATOL = 1e-3, 1e-5
ACCEPT_NEAR_TIE = 1e-5


def run_and_check(case, T, seed, ell_override=None, reqs=None):
    di = case.di
    buf, host, _ = case.run_draft(T, seed)
    runner.schedule(di, buf)
    if ell_override is not None:
        buf.ell.copy_(torch.as_tensor(ell_override, dtype=torch.int32))
    runner.verify(di, buf, T, seed)
    torch.cuda.synchronize()
    g = {n: getattr(buf, n).cpu().numpy() for n in ("ell", "c_star", "n_accept", "next_token",
                                                    "tau", "tau_mean")}
    R = case.wl.R
    reqs = np.arange(R) if reqs is None else np.asarray(reqs)
    x = host["x"].astype(np.int64)
    res = O.verify(case.inp.U[reqs], case.inp.target[reqs], case.W1, case.W2t, x[reqs],
                   g["ell"][reqs], T, seed, reqs)
    # c* for every position
    cs_g, cs_o = g["c_star"][reqs], res["c_star"]
    assert np.all(np.abs(cs_g - cs_o) <= np.maximum(CSTAR_ATOL, CSTAR_RTOL * np.abs(cs_o))), \
        np.abs(cs_g - cs_o).max()
    # accept decisions / tokens: exact unless the oracle saw a near tie
    near = (res["accept_margin"] < ACCEPT_NEAR_TIE) | (res["sample_gap"] < NEAR_TIE)
    ok = ((g["n_accept"][reqs] == res["n_accept"]) & (g["next_token"][reqs] == res["next_token"])
          & (g["tau"][reqs] == res["tau"]))
    assert np.all(ok | near), np.nonzero(~ok & ~near)
    assert (~ok).sum() <= 1e-3 * len(reqs)
    if len(reqs) == R:
        assert abs(float(g["tau_mean"][0]) - res["tau_mean"]) <= 1e-6 * res["tau_mean"]
    return g, res


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_verify_tiny(T):
    case = Case("tiny_v1024_r4_g4")
    g, res = run_and_check(case, T, 21)
    say(f"[verify] tiny T={T} ell={g['ell']} n_acc={g['n_accept']} tau_mean={g['tau_mean']}")
    # every position admitted (exercises the no-bonus case) and nothing admitted
    run_and_check(case, T, 22, ell_override=[4, 4, 4, 4])
    run_and_check(case, T, 23, ell_override=[0, 1, 2, 3])


def test_verify_full_round():
    """The full draft + schedule + verify round at R = 128, gamma = 7."""
    case = Case("round_4b_r128_g7")
    g, res = run_and_check(case, 1.0, 5)
    say(f"[verify] round budget={g['ell'].sum()} tau_mean={g['tau_mean'][0]:.4f} "
        f"c* mean={g['c_star'].mean():.4f}")
    g, res = run_and_check(case, 1.0, 6, ell_override=np.full(128, 7), reqs=np.arange(0, 128, 4))
    say(f"[verify] round ell=7 tau_mean={g['tau_mean'][0]:.4f}")


# rank 256 with ragged sizes: 111 rows (a partial last row tile), 37 requests
# in the sampling pass, a partial last vocabulary tile
synth.custom("edge_round_v9996_r37_g3", V=9996, rank=256, d=64, gamma=3, R=37, dtype="bf16",
             peak="three", target=True)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_verify_ragged_rank256(T):
    case = Case("edge_round_v9996_r37_g3")
    g, res = run_and_check(case, T, 31)
    say(f"[verify] ragged T={T} budget={g['ell'].sum()} tau_mean={g['tau_mean'][0]:.4f}")
    run_and_check(case, T, 32, ell_override=np.full(37, 3))
    run_and_check(case, T, 33, ell_override=np.arange(37) % 4)


# gamma = 16: no 32-row tile meets more than two requests, so the c* pass runs
# the sampling race itself.  A partial last row tile with a vocabulary that is
# not a multiple of 4 (row-by-row loads), and a single request (one half-filled
# row tile) with rank 128 and a partial last vocabulary tile.
synth.custom("fuse_round_v5003_r9_g16", V=5003, rank=256, d=64, gamma=16, R=9, dtype="bf16",
             peak="three", target=True)
synth.custom("fuse_round_v6000_r1_g16", V=6000, rank=128, d=64, gamma=16, R=1, dtype="bf16",
             peak="three", target=True)


@pytest.mark.parametrize("name", ["fuse_round_v5003_r9_g16", "fuse_round_v6000_r1_g16"])
def test_verify_race_in_cstar_pass(name):
    case = Case(name)
    R, g = case.wl.R, case.wl.gamma
    g1, _ = run_and_check(case, 1.0, 41)
    say(f"[verify] {name} budget={g1['ell'].sum()} tau_mean={g1['tau_mean'][0]:.4f}")
    # every position admitted: bonus rows only where ell < gamma
    run_and_check(case, 1.0, 42, ell_override=np.full(R, g))
    # a spread of admitted lengths, including none (a bonus at position 1)
    run_and_check(case, 1.0, 43, ell_override=(np.arange(R) * 5) % (g + 1))
    run_and_check(case, 0.7, 44, ell_override=np.full(R, g - 1))


synth.WORKLOADS["qwen3_8b_r128_g16_target"] = dataclasses.replace(
    synth.WORKLOADS["qwen3_8b_r128_g16"], name="qwen3_8b_r128_g16_target", target=True)


def test_verify_full_size_sampled():
    """Verification at R = 128, gamma = 16, V = 151936 in the benchmark's launch
    configuration, checked against the oracle on every eighth request."""
    case = Case("qwen3_8b_r128_g16_target")
    reqs = np.arange(0, 128, 8)
    g, _ = run_and_check(case, 1.0, 51, reqs=reqs)
    say(f"[verify] full size budget={g['ell'].sum()} tau_mean={g['tau_mean'][0]:.4f}")
    run_and_check(case, 1.0, 52, ell_override=np.arange(128) % 17, reqs=reqs + 3)
    g, _ = run_and_check(case, 0.0, 53, reqs=reqs + 5)
    say(f"[verify] full size greedy budget={g['ell'].sum()} tau_mean={g['tau_mean'][0]:.4f}")


# The largest row count the entry points take: R = 512 requests of gamma = 16
# (8192 rows: the acceptance kernel's and the scheduler's maximum), with a
# vocabulary that is not a multiple of 4.
synth.custom("maxrows_v4099_r512_g16", V=4099, rank=256, d=64, gamma=16, R=512, dtype="bf16",
             peak="three", target=True)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_verify_max_rows(T):
    case = Case("maxrows_v4099_r512_g16")
    reqs = np.arange(0, 512, 16)
    g, _ = run_and_check(case, T, 61, reqs=reqs)
    say(f"[verify] max rows T={T} budget={g['ell'].sum()} tau_mean={g['tau_mean'][0]:.4f}")
    run_and_check(case, T, 62, ell_override=np.arange(512) % 17, reqs=reqs + 5)


def test_max_vocabulary_round():
    """One request, one position at the largest vocabulary the entry points
    take (V = 2^24): draft step (z, token, p, lse, c, a), schedule and
    verification against the oracle.  The weights are a random 4096-row block
    tiled down the vocabulary (drawing 2 x 2^29 fresh values would take minutes
    on the host); U and the target noise are fresh per entry."""
    V = 1 << 24
    small = synth.custom("vmax_block_v4096_r1_g1", V=4096, rank=32, d=16, gamma=1, R=1,
                         dtype="bf16", peak="three", target=True)
    wl = synth.custom("vmax_v16777216_r1_g1", V=V, rank=32, d=16, gamma=1, R=1, dtype="bf16",
                      peak="three", target=True)
    base = synth.generate(small.name, seed=0)
    rng = np.random.default_rng(2024)
    U = (rng.standard_normal((1, 1, V), dtype=np.float32) * np.float32(2.0))
    U[0, 0, rng.choice(V, 3, replace=False)] += np.float32(6.0)
    target = U + rng.standard_normal((1, 1, V), dtype=np.float32)
    inp = dataclasses.replace(base, wl=wl, U=U, target=target,
                              W1_store=np.tile(base.W1_store, (V // 4096, 1)),
                              W2t_store=np.tile(base.W2t_store, (V // 4096, 1)),
                              anchor=np.array([V - 1], dtype=np.int32))
    case = Case.__new__(Case)
    case.inp, case.wl = inp, wl
    case.di = runner.DeviceInputs.upload(inp)
    # the oracle's fp64 weights: the same tiling of the block's exact values
    case.W1 = np.tile(O.as_f64(base.W1_store), (V // 4096, 1))
    case.W2t = np.tile(O.as_f64(base.W2t_store), (V // 4096, 1))
    from tests.gpu_parity import check_draft
    for T in (1.0, 0.0):
        _, host, zs = case.run_draft(T, 71, z_steps=(1,))
        check_draft(case, host, zs, T, 71)
        g, _ = run_and_check(case, T, 72)
        say(f"[verify] V=2^24 T={T} x={host['x'][0]} next={g['next_token']} c*={g['c_star']}")
        # nothing admitted: the bonus token is drawn over the whole vocabulary
        g, _ = run_and_check(case, T, 73, ell_override=[0])
        assert 0 <= g["next_token"][0] < V

"""GPU parity of the prefix schedulers (rank launch + finishing workgroup):
budgets, admitted prefixes and Theta must equal the oracle's bit for bit on
identical a."""
import numpy as np
import pytest
import torch

from oracle import dspark_oracle as O
from semi_autoregressive_drafting_amd import dspark as D
from semi_autoregressive_drafting_amd import synth
from tests.gpu_parity import say

pytestmark = pytest.mark.gpu

COUNTER_BYTES = 17 * 128


def workspace(R, g):
    """The scheduler's workspace: zero-filled before its first use, and left
    with its finishing counters (the first 17 128-byte lines) at zero by
    every call.  The rest is filled with junk, which no call may depend on."""
    n = D.dspark_workspace_bytes(D.DSPARK_OP_SCHEDULE, R, 2, 16, g)
    assert n > COUNTER_BYTES
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    ws[:COUNTER_BYTES].zero_()
    return ws


def gpu_schedule(a, sps, ws=None):
    R, g = a.shape
    ta = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    ts = torch.from_numpy(np.ascontiguousarray(sps, dtype=np.float64)).cuda()
    ell = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    budget = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    theta = torch.zeros(1, dtype=torch.float64, device="cuda")
    D.dspark_schedule(R, g, ta, ts, ts.numel(), ell, budget, theta,
                      workspace(R, g) if ws is None else ws)
    torch.cuda.synchronize()
    return ell.cpu().numpy(), int(budget.item()), float(theta.item())


def assert_same(a, sps, tag="", ws=None):
    ell_g, b_g, th_g = gpu_schedule(a, sps, ws)
    ell_o, b_o, th_o, _, _ = O.schedule(a, sps)
    assert b_g == b_o, (tag, b_g, b_o)
    np.testing.assert_array_equal(ell_g, ell_o)
    assert th_g == th_o, (tag, th_g, th_o)
    return b_g


def _tables(rng, R, g):
    yield "workload", synth.sps_table(R, g)
    knee = rng.uniform(R, R * (1 + g))
    yield "knee", synth.sps_table(R, g, 1e-4 * knee, 1e-4)
    B = np.arange(R * (1 + g) + 1)
    yield "steps", 1.0 / np.maximum(2e-3, 3e-6 * np.ceil(np.maximum(B, 1) / 16) * 16)


@pytest.mark.parametrize("R,g", [(1, 1), (1, 16), (3, 5), (4, 4), (7, 13), (32, 7),
                                 (128, 16), (128, 7), (512, 7), (512, 16), (300, 9)])
def test_schedule_random(R, g):
    rng = np.random.default_rng(R * 100 + g)
    for trial in range(3):
        c = rng.uniform(0.0, 1.0, (R, g)).astype(np.float32)
        c[rng.uniform(size=(R, g)) < 0.1] = 1.0          # ties along a row
        c[rng.uniform(size=(R, g)) < 0.02] = 0.0         # zero survival
        a = O.survival(c)
        for name, sps in _tables(rng, R, g):
            assert_same(a, sps, f"{R}x{g} {name} #{trial}")
    say(f"[schedule] {R}x{g} ok")


def test_schedule_workspace_reused_across_sizes():
    """One workspace sized for the largest call serves smaller calls after it,
    whatever the previous call left in it."""
    ws = workspace(512, 16)
    rng = np.random.default_rng(11)
    for R, g in [(512, 16), (37, 3), (128, 16), (1, 1), (300, 9)]:
        c = rng.uniform(0.0, 1.0, (R, g)).astype(np.float32)
        assert_same(O.survival(c), synth.sps_table(R, g), f"{R}x{g} reused", ws=ws)
        assert int(ws[:COUNTER_BYTES].count_nonzero().item()) == 0  # counters left at zero


def test_schedule_zero_survival():
    """Zero survival (+0 and -0 alike) sorts after every positive value, in
    flat-index order."""
    rng = np.random.default_rng(12)
    a = O.survival(rng.uniform(0.3, 1.0, (24, 6)).astype(np.float32))
    a[3, 2:] = 0.0
    a[7, 4:] = -0.0
    a[9, 5] = 0.0
    for sps in (synth.sps_table(24, 6), np.ones(24 * 7 + 1)):
        assert_same(a, sps, "zero")


def test_schedule_all_equal_keys():
    """Every candidate ties: order falls back to the flat index."""
    a = np.full((16, 8), 0.5, dtype=np.float32)
    assert_same(a, synth.sps_table(16, 8, 1e-3, 1e-5))
    assert_same(np.ones((8, 8), dtype=np.float32), synth.sps_table(8, 8))


def test_schedule_on_the_plan_demo_setting():
    """The handbook's adaptive-verification setting (two request classes, 7
    positions, cost 1/(0.25 ms + forward time)) with confidences drawn here:
    the GPU's budget, prefixes and Theta equal the oracle's, and at batch 16
    every candidate is admitted as the handbook prints (112)."""
    from tests.test_oracle_pins import _forward_time, _golden
    g = _golden("p2_plan_printout.json")
    fwd = _forward_time(_golden("p2_cost_model_printout.json")["model"])
    rng = np.random.default_rng(2024)
    for row in g["rows"]:
        batch, gamma = row["batch"], g["gamma"]
        base = np.where(np.arange(batch) < batch // 2, 0.9, 0.55)[:, None]
        c = np.minimum(base * rng.uniform(0.9, 1.1, (batch, gamma)), 0.99).astype(np.float32)
        a = O.survival(c)
        N = batch * (1 + gamma)
        sps = np.array([1.0 / (0.25e-3 + fwd(B)) for B in range(N + 1)])
        b = assert_same(a, sps)
        if batch == 16:
            assert b == row["admitted"]


# ---------------------------------------------------------------------------
# Asynchronous scheduler: budget from the lagged a, selection from the current a
# ---------------------------------------------------------------------------
def gpu_schedule_async(a_lag, a_cur, sps):
    R, g = a_cur.shape
    ws = workspace(R, g)
    tl = torch.from_numpy(np.ascontiguousarray(a_lag, dtype=np.float32)).cuda()
    tc = torch.from_numpy(np.ascontiguousarray(a_cur, dtype=np.float32)).cuda()
    ts = torch.from_numpy(np.ascontiguousarray(sps, dtype=np.float64)).cuda()
    ell = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    budget = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    theta = torch.zeros(1, dtype=torch.float64, device="cuda")
    D.dspark_schedule_async(R, g, tl, tc, ts, ts.numel(), ell, budget, theta, ws)
    torch.cuda.synchronize()
    return ell.cpu().numpy(), int(budget.item()), float(theta.item())


def assert_same_async(a_lag, a_cur, sps, tag=""):
    ell_g, K_g, th_g = gpu_schedule_async(a_lag, a_cur, sps)
    ell_o, K_o, th_o, _ = O.schedule_async(a_lag, a_cur, sps)
    assert K_g == K_o, (tag, K_g, K_o)
    np.testing.assert_array_equal(ell_g, ell_o, err_msg=tag)
    assert th_g == th_o, (tag, th_g, th_o)
    return K_g


@pytest.mark.parametrize("R,g", [(1, 1), (3, 5), (4, 4), (37, 3), (128, 16), (512, 7),
                                 (512, 16), (300, 9)])
def test_schedule_async_random(R, g):
    rng = np.random.default_rng(R * 1000 + g)
    for trial in range(3):
        cs = []
        for _ in range(2):
            c = rng.uniform(0.0, 1.0, (R, g)).astype(np.float32)
            c[rng.uniform(size=(R, g)) < 0.1] = 1.0
            c[rng.uniform(size=(R, g)) < 0.02] = 0.0
            cs.append(O.survival(c))
        for name, sps in _tables(rng, R, g):
            assert_same_async(cs[0], cs[1], sps, f"{R}x{g} {name} #{trial}")
        # a bumpy table: many local maxima, so the global search matters
        B = np.arange(R * (1 + g) + 1)
        sps = 1.0 / (1e-3 + 1e-5 * B + rng.uniform(0, 3e-4, B.size))
        assert_same_async(cs[0], cs[1], sps, f"{R}x{g} bumpy #{trial}")
    say(f"[schedule_async] {R}x{g} ok")


def test_schedule_async_edges():
    """K = N (flat table), K = 0 (steeply falling table), the hand-built cliff
    (K = 4 where the early stop gives 1), a tie between budgets (smallest wins)
    and all-equal keys (flat-index order)."""
    rng = np.random.default_rng(3)
    a = O.survival(rng.uniform(0.2, 1.0, (16, 8)).astype(np.float32))
    N = 16 * 8
    assert assert_same_async(a, a, np.ones(16 * 9 + 1)) == N
    assert assert_same_async(a, a, 1.0 / (1.0 + np.arange(16 * 9 + 1)) ** 3) == 0
    ones = np.ones((2, 2), dtype=np.float32)
    assert assert_same_async(ones, ones, np.array([0.0, 0.0, 1.0, 0.9, 0.6, 0.55, 0.5])) == 4
    assert assert_same_async(ones, ones, np.array([0.0, 0.0, 1.0, 5.0, 2.0, 3.0, 1.0])) == 1
    half = np.full((16, 8), 0.5, dtype=np.float32)
    assert_same_async(a, half, synth.sps_table(16, 8, 1e-3, 1e-5))

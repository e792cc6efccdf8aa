"""A whole round (draft block, schedule, verify) captured in one HIP graph and
replayed gives the same bits as the same round run eagerly, on every replay,
with other eager work and synchronisations between the replays.  The kernels
clear their accumulators with ordinary stores (no memset nodes)."""
import numpy as np
import pytest
import torch

from semi_autoregressive_drafting_amd import runner, synth
from tests.gpu_parity import say

pytestmark = pytest.mark.gpu

OUTS = ("x", "p", "lse", "c", "a", "ell", "budget", "c_star", "n_accept", "next_token", "tau",
        "tau_mean")


@pytest.mark.parametrize("name,T", [("round_4b_r128_g7", 1.0), ("tiny_v1024_r4_g4", 0.0)])
def test_graph_replay_matches_eager(name, T):
    say(f"[graph] {name} T={T}")
    inp = synth.generate(name, seed=0, target=True)
    di = runner.DeviceInputs.upload(inp)
    ref = runner.RoundBuffers.allocate(di)
    runner.full_round(di, ref, T, 31)
    torch.cuda.synchronize()
    expect = {n: getattr(ref, n).cpu().numpy() for n in OUTS}

    buf = runner.RoundBuffers.allocate(di)
    other = runner.RoundBuffers.allocate(di)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        runner.full_round(di, buf, T, 5)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        runner.full_round(di, buf, T, 31)
    for rep in range(3):
        runner.full_round(di, other, T, 100 + rep)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            np.testing.assert_array_equal(getattr(buf, n).cpu().numpy(), expect[n],
                                          err_msg=f"replay {rep}: {n}")

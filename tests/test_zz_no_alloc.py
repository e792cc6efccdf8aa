"""GPU check of dspark_draft_block_noalloc, the draft block for callers that
cannot allocate: its workspace is the library's static device array instead
of a caller buffer.  Called through the C ABI, it must give the same bits as
dspark_draft_block with a fresh zero-filled workspace, on consecutive calls
whose shapes differ (the second one smaller, so its winner words sit where the
first call left its records: the call must clear them itself)."""
import numpy as np
import pytest
import torch

from semi_autoregressive_drafting_amd import dspark as D, runner, synth
from tests.gpu_parity import Case, say

pytestmark = pytest.mark.gpu

FIELDS = ("x", "p", "lse", "c", "a")
# a ragged shape on the shared launch: partial last request and vocabulary tiles
synth.custom("noalloc_v9996_r130_g3", V=9996, rank=256, d=64, gamma=3, R=130, dtype="bf16",
             peak="three")


def _run(case, T, seed, noalloc):
    di = case.di
    buf = runner.RoundBuffers.allocate(di)
    buf.x[:, 0].copy_(di.anchor)
    args = (di.R, di.V, di.rank, di.d, di.gamma, di.dt, di.W1, di.W2t, di.U, di.h, di.w, T, seed,
            buf.x, buf.p, buf.lse, buf.c, buf.a)
    if noalloc:
        D.dspark_draft_block_noalloc(*args)
    else:
        D.dspark_draft_block(*args, buf.ws)
    torch.cuda.synchronize()
    return {n: getattr(buf, n).cpu().numpy() for n in FIELDS}


@pytest.mark.parametrize("order", [
    (("qwen3_8b_r128_g16", 1.0), ("qwen3_4b_r32_g7", 1.0)),
    (("round_4b_r128_g7", 0.0), ("noalloc_v9996_r130_g3", 1.0)),
])
def test_noalloc_block_matches_block(order):
    for name, T in order:
        say(f"[noalloc] {name} T={T}")
        case = Case(name)
        want = _run(case, T, 77, noalloc=False)
        got = _run(case, T, 77, noalloc=True)
        for n in FIELDS:
            np.testing.assert_array_equal(got[n], want[n], err_msg=f"{name} {n}")
        assert np.all((got["x"] >= 0) & (got["x"] < case.wl.V))
        del case

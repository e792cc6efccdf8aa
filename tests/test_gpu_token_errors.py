"""GPU checks of the token-error word: a token id outside [0, V) read from
device memory by a row gather is clamped into range and recorded; valid data
leaves the word clear; the host query reads and clears it."""
import numpy as np
import pytest
import torch

from semi_autoregressive_drafting_amd import dspark as D, runner, synth
from tests.gpu_parity import say

pytestmark = pytest.mark.gpu

NAME = "tokerr_v1000_r8_g3"
synth.custom(NAME, V=1000, rank=32, d=64, gamma=3, R=8, dtype="bf16", peak="three", target=True)


@pytest.fixture(scope="module")
def setup():
    inp = synth.generate(NAME, seed=0, target=True)
    di = runner.DeviceInputs.upload(inp)
    return inp, di


def _outputs(buf):
    torch.cuda.synchronize()
    return [t.cpu().numpy().copy() for t in (buf.x, buf.p, buf.lse, buf.c, buf.a)]


def test_valid_round_leaves_the_word_clear(setup):
    _, di = setup
    say("[token errors] valid round")
    buf = runner.RoundBuffers.allocate(di)
    D.dspark_token_errors(clear=True)
    runner.full_round(di, buf, 1.0, 5)
    x_star = buf.x.clone()
    runner.train_loss(di, x_star)
    torch.cuda.synchronize()
    assert D.dspark_token_errors() == 0


@pytest.mark.parametrize("bad, clamped", [(1007, 999), (-5, 0), (1000, 999)])
def test_bad_anchor_is_flagged_and_clamped(setup, bad, clamped):
    """The draft block with one anchor outside [0, V) sets the word and drafts
    exactly what the clamped anchor drafts."""
    _, di = setup
    say(f"[token errors] anchor {bad}")
    anchor0 = di.anchor.clone()
    try:
        ref = runner.RoundBuffers.allocate(di)
        di.anchor[3] = clamped
        D.dspark_token_errors(clear=True)
        runner.draft(di, ref, 1.0, 9)
        want = _outputs(ref)
        assert D.dspark_token_errors() == 0
        buf = runner.RoundBuffers.allocate(di)
        di.anchor[3] = bad
        runner.draft(di, buf, 1.0, 9)
        got = _outputs(buf)
        assert D.dspark_token_errors(clear=True) == 1
        assert D.dspark_token_errors() == 0
        got[0][3, 0] = clamped  # the anchor column holds what the caller wrote
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g, w)
    finally:
        di.anchor.copy_(anchor0)


def test_bad_drafted_token_in_verify_is_flagged(setup):
    _, di = setup
    say("[token errors] verify")
    buf = runner.RoundBuffers.allocate(di)
    runner.draft(di, buf, 1.0, 11)
    runner.schedule(di, buf)
    torch.cuda.synchronize()
    D.dspark_token_errors(clear=True)
    buf.x[5, 2] = -3
    runner.verify(di, buf, 1.0, 11)
    torch.cuda.synchronize()
    assert D.dspark_token_errors(clear=True) == 1


def test_bad_target_token_in_training_is_flagged(setup):
    _, di = setup
    say("[token errors] training")
    buf = runner.RoundBuffers.allocate(di)
    runner.draft(di, buf, 1.0, 13)
    x_star = buf.x.clone()
    x_star[0, 1] = di.V + 40
    torch.cuda.synchronize()
    D.dspark_token_errors(clear=True)
    runner.train_loss(di, x_star)
    torch.cuda.synchronize()
    assert D.dspark_token_errors(clear=True) == 1


def test_bad_token_in_batched_confidence_is_flagged(setup):
    _, di = setup
    say("[token errors] confidence")
    R, g = di.R, di.gamma
    x = torch.zeros((R, g + 1), dtype=torch.int32, device="cuda")
    x[:, 0] = di.anchor
    x[6, 1] = 123456
    c = torch.empty((R, g), dtype=torch.float32, device="cuda")
    a = torch.empty_like(c)
    D.dspark_token_errors(clear=True)
    D.dspark_confidence(R, g, di.d, di.rank, di.V, di.dt, di.h, di.W1, x, di.w, c, a)
    torch.cuda.synchronize()
    assert D.dspark_token_errors(clear=True) == 1

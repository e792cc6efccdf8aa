"""A seeded sweep over random ragged shapes: the draft round with verification,
the training gradients and the RNN head, each against the CPU oracle with the
same checks and tolerances as their own test files.  The shapes mix vocabulary
tails (V % 4 and V % 32), partial row tiles, one-request batches and every rank
the gradient and RNN entry points take."""
import numpy as np
import pytest

from semi_autoregressive_drafting_amd import synth
from tests.gpu_parity import Case, check_draft, check_flip_rate, say
from tests import test_gpu_rnn as RNN
from tests import test_gpu_train_grad as GRAD
from tests.test_gpu_verify import run_and_check

pytestmark = pytest.mark.gpu


def _shapes(n=10, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        V = int(rng.integers(50, 6000))
        R = int(rng.choice([1, int(rng.integers(2, 33)), int(rng.integers(33, 141))]))
        gamma = int(rng.integers(1, 7))
        rank = int(rng.choice([32, 64, 128, 256]))
        d = 16 * int(rng.integers(1, 9))
        name = f"sweep{i}_v{V}_r{R}_g{gamma}_k{rank}_d{d}"
        synth.custom(name, V=V, rank=rank, d=d, gamma=gamma, R=R, dtype="bf16", peak="three",
                     target=True)
        out.append(name)
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("name", SHAPES)
def test_sweep_round(name):
    say(f"[sweep] round {name}")
    case = Case(name)
    buf, host, zs = case.run_draft(1.0, 77, z_steps=(1,))
    stats = check_draft(case, host, zs, 1.0, 77)
    check_flip_rate(stats)
    run_and_check(case, 1.0, 78)


@pytest.mark.parametrize("name", SHAPES)
def test_sweep_round_greedy(name):
    say(f"[sweep] greedy round {name}")
    case = Case(name)
    buf, host, zs = case.run_draft(0.0, 80, z_steps=(1,))
    check_flip_rate(check_draft(case, host, zs, 0.0, 80))
    run_and_check(case, 0.0, 81)


@pytest.mark.parametrize("name", SHAPES)
def test_sweep_train_grads(name):
    GRAD._check_all(name, 1.0, None)


@pytest.mark.parametrize("name", SHAPES)
def test_sweep_rnn(name):
    say(f"[sweep] rnn {name}")
    inp, gru, host, _ = RNN._run(name, 0.8, 79)
    RNN._check(inp, gru, host, 0.8, 79)

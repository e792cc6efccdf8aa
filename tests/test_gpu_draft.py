"""GPU parity of the fused Markov draft step (gather, MFMA bias, base-logit add,
online softmax, Gumbel-argmax, confidence, survival) against the CPU oracle,
on every workload and on ragged / edge shapes."""
import numpy as np
import pytest
import torch

from semi_autoregressive_drafting_amd import runner, synth
from tests.gpu_parity import Case, check_draft, check_flip_rate, say

pytestmark = pytest.mark.gpu

SEED = 1234

# ragged and edge shapes: vocabulary tails (V % 32, V % 4), partial request
# tiles on both launch shapes, the smallest and largest ranks, gamma = 1
synth.custom("edge_v997_r37_g3", V=997, rank=16, d=40, gamma=3, R=37, dtype="bf16", peak="three")
synth.custom("edge_v1000_r100_g2", V=1000, rank=48, d=33, gamma=2, R=100, dtype="bf16",
             peak="three")
synth.custom("edge_v2_r1_g1", V=2, rank=4, d=1, gamma=1, R=1, dtype="f32", peak="none",
             weight_std=1.0)
synth.custom("edge_v4096_r129_g2_f32", V=4096, rank=128, d=16, gamma=2, R=129, dtype="f32",
             peak="three")
synth.custom("edge_v40000_r1_g4", V=40000, rank=256, d=128, gamma=4, R=1, dtype="bf16",
             peak="three")


# rank-256 bf16 shapes with 16-byte-aligned rows run the production kernels
# (line-coalesced row and E loads, the skewed MFMA stream) on ragged sizes: a
# partial last vocabulary tile, a partial last request tile (clamped rows) and
# both launch shapes.
synth.custom("edge_v9996_r130_g3", V=9996, rank=256, d=64, gamma=3, R=130, dtype="bf16",
             peak="three")
synth.custom("edge_v8196_r33_g2", V=8196, rank=256, d=40, gamma=2, R=33, dtype="bf16",
             peak="three")
# Vocabularies large enough that every slab of the shared stream runs the
# pipeline through several periods: two request groups with a partial last
# vocabulary tile, and a vocabulary whose rows are not 16-byte aligned
# (per-lane row loads).
synth.custom("edge_v40004_r130_g3", V=40004, rank=256, d=64, gamma=3, R=130, dtype="bf16",
             peak="three")
synth.custom("edge_v40001_r128_g2", V=40001, rank=256, d=48, gamma=2, R=128, dtype="bf16",
             peak="three")
# the largest batch and block: R = 512 (four request groups), gamma = 16
synth.custom("edge_v4099_r512_g16", V=4099, rank=256, d=48, gamma=16, R=512, dtype="bf16",
             peak="three")


@pytest.mark.parametrize("name,T", [
    ("edge_v9996_r130_g3", 1.0), ("edge_v9996_r130_g3", 0.0), ("edge_v8196_r33_g2", 1.0),
    ("edge_v40004_r130_g3", 1.0), ("edge_v40004_r130_g3", 0.0), ("edge_v40001_r128_g2", 1.0),
    ("edge_v4099_r512_g16", 1.0), ("edge_v4099_r512_g16", 0.0),
])
def test_draft_fast_paths_ragged(name, T):
    """z is checked at step 1 only (its debug kernel); the other steps run the
    production kernels and are checked on tokens, p, lse, c and a."""
    say(f"[draft] {name} T={T}")
    case = Case(name)
    _, host, zs = case.run_draft(T, SEED, z_steps=(1,))
    stats = check_draft(case, host, zs, T, SEED)
    check_flip_rate(stats)
    say(f"  {stats}")


@pytest.mark.parametrize("name,T", [
    ("tiny_v1024_r4_g4", 1.0), ("tiny_v1024_r4_g4", 0.0),
    ("bruteforce_v8_g3", 1.0), ("bruteforce_v8_g3", 0.7), ("bruteforce_v8_g3", 0.0),
    ("edge_v997_r37_g3", 1.0), ("edge_v1000_r100_g2", 0.8), ("edge_v1000_r100_g2", 0.0),
    ("edge_v2_r1_g1", 1.0), ("edge_v4096_r129_g2_f32", 1.0), ("edge_v40000_r1_g4", 1.5),
])
def test_draft_small_and_ragged(name, T):
    say(f"[draft] {name} T={T}")
    case = Case(name)
    _, host, zs = case.run_draft(T, SEED, z_steps=range(1, case.wl.gamma + 1))
    stats = check_draft(case, host, zs, T, SEED)
    check_flip_rate(stats)
    say(f"  {stats}")


@pytest.mark.parametrize("name,T,nsample", [
    ("qwen3_4b_r32_g7", 1.0, None),
    ("qwen3_8b_r128_g16", 1.0, 32),
    ("qwen3_14b_r512_g7", 1.0, 48),
    ("qwen3_14b_r512_g7", 0.0, 48),
    ("round_4b_r128_g7", 1.0, 32),
])
def test_draft_full_size(name, T, nsample):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    checks every step on a sample of requests (rows are independent given
    x_{k-1}), z on the first and last step."""
    say(f"[draft] {name} T={T} sample={nsample}")
    case = Case(name)
    g = case.wl.gamma
    _, host, zs = case.run_draft(T, SEED, z_steps=(1, g))
    R = case.wl.R
    if nsample is None:
        reqs = np.arange(R)
    else:  # spread over the batch (both halves of the easy/hard split)
        reqs = np.unique(np.linspace(0, R - 1, nsample).round().astype(int))
    stats = check_draft(case, host, zs, T, SEED, reqs=reqs)
    check_flip_rate(stats)
    say(f"  {stats}")


@pytest.mark.parametrize("name", ["qwen3_4b_r32_g7", "qwen3_8b_r128_g16", "edge_v40004_r130_g3"])
def test_draft_is_deterministic(name):
    """Two runs give bit-identical outputs: records are merged in a fixed
    order, and the winner words' atomic maximum does not depend on the order
    in which workgroups arrive."""
    case = Case(name)
    _, h1, _ = case.run_draft(1.0, 7)
    _, h2, _ = case.run_draft(1.0, 7)
    for n in h1:
        np.testing.assert_array_equal(h1[n], h2[n], err_msg=n)


def test_draft_block_matches_single_steps():
    """dspark_draft_block, and its two phases called in turn, give the same bits
    as gamma dspark_draft_step calls."""
    from semi_autoregressive_drafting_amd import dspark as D
    for name in ("qwen3_4b_r32_g7", "edge_v1000_r100_g2", "tiny_v1024_r4_g4",
                 "edge_v40004_r130_g3", "qwen3_8b_r128_g16", "edge_v9996_r130_g3",
                 "edge_v40001_r128_g2"):
        case = Case(name)
        _, h1, _ = case.run_draft(1.0, 11)
        di = case.di
        buf = runner.RoundBuffers.allocate(di)
        runner.draft(di, buf, 1.0, 11)
        torch.cuda.synchronize()
        for n in ("x", "p", "lse", "c", "a"):
            np.testing.assert_array_equal(getattr(buf, n).cpu().numpy(), h1[n], err_msg=name + n)
        # the same block as its two phases (steps, then the merge)
        buf2 = runner.RoundBuffers.allocate(di)
        runner.draft_phases(di, buf2, 1.0, 11, D.DSPARK_PHASE_STEPS)
        runner.draft_phases(di, buf2, 1.0, 11, D.DSPARK_PHASE_MERGE)
        torch.cuda.synchronize()
        for n in ("x", "p", "lse", "c", "a"):
            np.testing.assert_array_equal(getattr(buf2, n).cpu().numpy(), h1[n],
                                          err_msg=name + n + " (phases)")


def test_draft_block_greedy_matches_single_steps():
    """The same at T = 0 on shared rank-256 shapes."""
    for name in ("qwen3_8b_r128_g16", "edge_v40004_r130_g3"):
        case = Case(name)
        _, h1, _ = case.run_draft(0.0, 5)
        buf = runner.RoundBuffers.allocate(case.di)
        runner.draft(case.di, buf, 0.0, 5)
        torch.cuda.synchronize()
        for n in ("x", "p", "lse", "c", "a"):
            np.testing.assert_array_equal(getattr(buf, n).cpu().numpy(), h1[n], err_msg=name + n)


def test_batched_confidence_matches_fused():
    """dspark_confidence over a drafted block reproduces the c and a that the
    draft steps computed, bit for bit."""
    from semi_autoregressive_drafting_amd import dspark as D
    case = Case("tiny_v1024_r4_g4")
    buf, host, _ = case.run_draft(1.0, 3)
    di = case.di
    c = torch.zeros_like(buf.c)
    a = torch.zeros_like(buf.a)
    D.dspark_confidence(di.R, di.gamma, di.d, di.rank, di.V, di.dt, di.h, di.W1, buf.x, di.w, c, a)
    np.testing.assert_array_equal(c.cpu().numpy(), host["c"])
    np.testing.assert_array_equal(a.cpu().numpy(), host["a"])
    case = Case("qwen3_4b_r32_g7")
    buf, host, _ = case.run_draft(1.0, 3)
    di = case.di
    c = torch.zeros_like(buf.c)
    a = torch.zeros_like(buf.a)
    D.dspark_confidence(di.R, di.gamma, di.d, di.rank, di.V, di.dt, di.h, di.W1, buf.x, di.w, c, a)
    np.testing.assert_array_equal(c.cpu().numpy(), host["c"])
    np.testing.assert_array_equal(a.cpu().numpy(), host["a"])


def test_counter_uniforms_bit_exact():
    """With U = 0, W = 0 and T = 1 every id has the same logit, so every block
    has the same mass and the draft token is decided by the noise alone: the
    block is the argmax of the block uniforms (DRAFT stream, counter = block),
    the id the argmax of the id uniforms inside it (DRAFT_ENTRY stream,
    counter = id).  The GPU's token must equal the one the oracle's own
    uniforms give (independent implementations of the same counter
    generator)."""
    from oracle import dspark_oracle as O
    synth.custom("flat_v4096_r64_g2", V=4096, rank=16, d=8, gamma=2, R=64, dtype="bf16",
                 peak="none", weight_std=0.0)
    case = Case("flat_v4096_r64_g2")
    case.di.U.zero_()
    _, host, _ = case.run_draft(1.0, 99)
    nb = 4096 // O.DRAFT_BLOCK
    for k in (1, 2):
        for r in range(64):
            ub = O.uniforms(99, O.STREAM_DRAFT, r, k, np.arange(nb, dtype=np.uint32))
            b = int(np.argmax(ub))
            ids = np.arange(b * O.DRAFT_BLOCK, (b + 1) * O.DRAFT_BLOCK, dtype=np.uint32)
            ue = O.uniforms(99, O.STREAM_DRAFT_ENTRY, r, k, ids)
            assert host["x"][r, k] == int(ids[np.argmax(ue)]), (r, k)

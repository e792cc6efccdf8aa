"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its workspaces, and rejects bad arguments on the host
before any HIP call (fake non-NULL addresses are never dereferenced)."""
import os
import re

import pytest

from semi_autoregressive_drafting_amd import dspark as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

pytestmark = pytest.mark.skipif(not os.path.exists(D.LIB_PATH),
                                reason="libdspark.so not built (run __graft_entry__.build())")

FAKE = 0x10000  # 16-byte aligned, non-NULL, never dereferenced by a failing call


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dspark_status|size_t|const char\*)\s+(dspark_\w+)\(",
                                 text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = D.load()
    names = declared_functions()
    assert set(names) == set(D.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_nm_lists_the_c_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", D.LIB_PATH], capture_output=True,
                         text=True).stdout
    for n in declared_functions():
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_status_strings():
    assert D.status_string(0) == "ok"
    assert "NULL" in D.status_string(D.DSPARK_ERR_NULL)
    assert D.status_string(99) == "unknown status"


def test_workspace_sizes():
    f = D.dspark_workspace_bytes
    assert f(D.DSPARK_OP_DRAFT_STEP, 0, 1024, 32, 4) == 0
    assert f(D.DSPARK_OP_DRAFT_STEP, 513, 1024, 32, 4) == 0
    assert f(D.DSPARK_OP_DRAFT_STEP, 4, 1, 32, 4) == 0
    assert f(D.DSPARK_OP_DRAFT_STEP, 4, 1024, 32, 17) == 0
    assert f(D.DSPARK_OP_SCHEDULE, 128, 151936, 256, 16) > 0
    assert f(99, 4, 1024, 32, 4) == 0
    # at least one 5-field record per request and slab; 256-byte aligned regions
    w128 = f(D.DSPARK_OP_DRAFT_STEP, 128, 151936, 256, 16)
    assert w128 >= 5 * 128 * 4 * 32 and w128 % 256 == 0
    assert f(D.DSPARK_OP_DRAFT_STEP, 512, 151936, 256, 7) > 0
    assert f(D.DSPARK_OP_VERIFY, 128, 151936, 256, 7) > 128 * 7 * 8


def _step(**kw):
    a = dict(R=4, V=1024, rank=32, d=64, gamma=4, k=1, dt=D.DSPARK_F32, W1=FAKE, W2t=FAKE,
             U=FAKE, h=FAKE, w=FAKE, temperature=1.0, seed=0, x=FAKE, p=FAKE, lse=FAKE, c=FAKE,
             a=FAKE, z_debug=None, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    lib = D.load()
    return lib.dspark_draft_step(a["R"], a["V"], a["rank"], a["d"], a["gamma"], a["k"], a["dt"],
                                 a["W1"], a["W2t"], a["U"], a["h"], a["w"], a["temperature"],
                                 a["seed"], a["x"], a["p"], a["lse"], a["c"], a["a"],
                                 a["z_debug"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(W1=None), D.DSPARK_ERR_NULL),
    (dict(U=None), D.DSPARK_ERR_NULL),
    (dict(x=None), D.DSPARK_ERR_NULL),
    (dict(h=None), D.DSPARK_ERR_NULL),              # h without w
    (dict(c=None), D.DSPARK_ERR_NULL),              # confidence needs c and a
    (dict(dt=7), D.DSPARK_ERR_DTYPE),
    (dict(R=0), D.DSPARK_ERR_SHAPE),
    (dict(R=513), D.DSPARK_ERR_SHAPE),
    (dict(V=1), D.DSPARK_ERR_SHAPE),
    (dict(gamma=17, k=1), D.DSPARK_ERR_SHAPE),
    (dict(rank=30), D.DSPARK_ERR_SHAPE),            # fp32 rank multiple of 4
    (dict(rank=132), D.DSPARK_ERR_SHAPE),
    (dict(rank=24, dt=D.DSPARK_BF16), D.DSPARK_ERR_SHAPE),   # bf16 rank multiple of 16
    (dict(rank=272, dt=D.DSPARK_BF16), D.DSPARK_ERR_SHAPE),
    (dict(d=0), D.DSPARK_ERR_SHAPE),
    (dict(W2t=FAKE + 4), D.DSPARK_ERR_SHAPE),       # misaligned weights
    (dict(U=FAKE + 4), D.DSPARK_ERR_SHAPE),         # misaligned logits with V % 4 == 0
    (dict(k=0), D.DSPARK_ERR_VALUE),
    (dict(k=5), D.DSPARK_ERR_VALUE),
    (dict(temperature=-1.0), D.DSPARK_ERR_VALUE),
    (dict(temperature=float("nan")), D.DSPARK_ERR_VALUE),
    (dict(temperature=float("inf")), D.DSPARK_ERR_VALUE),
    (dict(ws=None), D.DSPARK_ERR_WORKSPACE),
    (dict(ws_bytes=16), D.DSPARK_ERR_WORKSPACE),
])
def test_draft_step_validation(kw, status):
    assert _step(**kw) == status


def test_draft_block_validation():
    f = D.load().dspark_draft_block
    args = [4, 1024, 32, 64, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 0, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE, 1 << 30, None]
    bad = list(args); bad[6] = None
    assert f(*bad) == D.DSPARK_ERR_NULL
    bad = list(args); bad[4] = 0
    assert f(*bad) == D.DSPARK_ERR_SHAPE
    bad = list(args); bad[11] = -2.0
    assert f(*bad) == D.DSPARK_ERR_VALUE
    bad = list(args); bad[19] = 8
    assert f(*bad) == D.DSPARK_ERR_WORKSPACE


def test_draft_block_noalloc_validation():
    """The no-allocation block validates like dspark_draft_block before any HIP
    call (there is no workspace argument to get wrong)."""
    f = D.load().dspark_draft_block_noalloc
    args = [4, 1024, 32, 64, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 0, FAKE, FAKE, FAKE,
            FAKE, FAKE, None]
    bad = list(args); bad[6] = None
    assert f(*bad) == D.DSPARK_ERR_NULL
    bad = list(args); bad[13] = None
    assert f(*bad) == D.DSPARK_ERR_NULL
    bad = list(args); bad[4] = 0
    assert f(*bad) == D.DSPARK_ERR_SHAPE
    bad = list(args); bad[0] = 513
    assert f(*bad) == D.DSPARK_ERR_SHAPE
    bad = list(args); bad[5] = 7
    assert f(*bad) == D.DSPARK_ERR_DTYPE
    bad = list(args); bad[11] = float("nan")
    assert f(*bad) == D.DSPARK_ERR_VALUE
    bad = list(args); bad[9] = None   # h without w
    assert f(*bad) == D.DSPARK_ERR_NULL


def test_noalloc_scratch_fits_every_accepted_shape():
    """The static workspace of dspark_draft_block_noalloc (22 MiB) holds the
    draft workspace of the largest shape the ABI accepts (R = 512, gamma = 16),
    at any vocabulary size."""
    f = D.dspark_workspace_bytes
    biggest = max(f(D.DSPARK_OP_DRAFT_STEP, R, V, 256, g)
                  for R in (1, 96, 97, 128, 129, 384, 511, 512) for g in (1, 7, 16)
                  for V in (2, 1024, 151936, 1 << 24))
    assert biggest == f(D.DSPARK_OP_DRAFT_STEP, 512, 151936, 256, 16)
    assert biggest <= 22 << 20


def test_schedule_validation():
    lib = D.load()
    f = lib.dspark_schedule
    assert f(4, 4, None, FAKE, 21, FAKE, FAKE, FAKE, None, 0, None) == D.DSPARK_ERR_NULL
    assert f(4, 4, FAKE, FAKE, 21, None, FAKE, FAKE, None, 0, None) == D.DSPARK_ERR_NULL
    assert f(4, 4, FAKE, FAKE, 20, FAKE, FAKE, FAKE, None, 0, None) == D.DSPARK_ERR_SHAPE
    assert f(512, 17, FAKE, FAKE, 10 ** 6, FAKE, FAKE, FAKE, None, 0, None) == D.DSPARK_ERR_SHAPE
    assert f(600, 4, FAKE, FAKE, 10 ** 6, FAKE, FAKE, FAKE, None, 0, None) == D.DSPARK_ERR_SHAPE
    need = D.dspark_workspace_bytes(D.DSPARK_OP_SCHEDULE, 4, 2, 16, 4)
    assert f(4, 4, FAKE, FAKE, 21, FAKE, FAKE, FAKE, None, need, None) == D.DSPARK_ERR_WORKSPACE
    assert f(4, 4, FAKE, FAKE, 21, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        D.DSPARK_ERR_WORKSPACE
    assert f(4, 4, FAKE, FAKE, 21, FAKE, FAKE, FAKE, FAKE + 8, need, None) == \
        D.DSPARK_ERR_WORKSPACE


def test_schedule_workspace_size():
    """The scheduler's workspace grows with R*gamma and covers the sorted
    positions (int32) and the prefix sums G at every position 0..N (fp64);
    beyond 8192 candidates there is no size."""
    ws = lambda R, g: D.dspark_workspace_bytes(D.DSPARK_OP_SCHEDULE, R, 2, 16, g)
    assert ws(1, 1) > 0
    assert ws(128, 16) >= 128 * 16 * 4 + (128 * 16 + 1) * 8
    assert ws(512, 16) > ws(128, 16) > ws(4, 4)
    assert ws(512, 16) <= 160 << 10
    assert ws(600, 16) == 0 and ws(512, 17) == 0


def test_draft_block_phases_validation():
    f = D.load().dspark_draft_block_phases
    args = [128, 151936, 256, 4096, 16, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 0,
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30]
    assert f(*args, 0, None) == D.DSPARK_ERR_VALUE
    assert f(*args, 4, None) == D.DSPARK_ERR_VALUE
    bad = list(args)
    bad[6] = None
    assert f(*bad, 3, None) == D.DSPARK_ERR_NULL


def test_train_loss_validation():
    f = D.load().dspark_train_loss
    base = [4, 1024, 32, 64, 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 4.0, 0.1, 0.9,
            1.0, FAKE, FAKE, FAKE, 1 << 30, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a5=7) == D.DSPARK_ERR_DTYPE
    assert call(a12=None) == D.DSPARK_ERR_NULL          # x_star
    assert call(a19=None) == D.DSPARK_ERR_NULL          # sums
    assert call(a0=0) == D.DSPARK_ERR_SHAPE
    assert call(a3=0) == D.DSPARK_ERR_SHAPE             # d
    assert call(a2=30) == D.DSPARK_ERR_SHAPE            # fp32 rank not a multiple of 4
    assert call(a13=0.0) == D.DSPARK_ERR_VALUE          # T = 0 has no softmax
    assert call(a14=0.0) == D.DSPARK_ERR_VALUE          # lambda
    assert call(a15=float("nan")) == D.DSPARK_ERR_VALUE
    assert call(a21=16) == D.DSPARK_ERR_WORKSPACE
    assert D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_LOSS, 4, 1024, 32, 4) > \
        D.dspark_workspace_bytes(D.DSPARK_OP_VERIFY, 4, 1024, 32, 4)


def test_train_loss_grad_validation():
    f = D.load().dspark_train_loss_grad
    # bf16, rank 64; outputs terms, sums, dU, dW1, dW2t, dh, dw at 18 .. 24
    base = [4, 1024, 64, 64, 4, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 4.0, 0.1, 0.9,
            1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 34, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a5=0) == D.DSPARK_ERR_DTYPE             # gradients need bf16 weights
    assert call(a5=7) == D.DSPARK_ERR_DTYPE
    for i in range(20, 25):                             # every gradient output is required
        assert call(**{f"a{i}": None}) == D.DSPARK_ERR_NULL
    assert call(a2=48) == D.DSPARK_ERR_SHAPE            # rank not a multiple of 32
    assert call(a2=288) == D.DSPARK_ERR_SHAPE           # rank above 256
    assert call(a13=0.0) == D.DSPARK_ERR_VALUE
    need = D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_GRAD, 4, 1024, 64, 4)
    assert need > D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_LOSS, 4, 1024, 64, 4)
    # the query is sized for the largest d; the forward's workspace is too small
    assert call(a26=D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_LOSS, 4, 1024, 64, 4)) == \
        D.DSPARK_ERR_WORKSPACE
    assert D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_GRAD, 4, 1024, 48, 4) == 0
    # the transposed W2t copy dominates at full size: rank x V bf16
    big = D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_GRAD, 128, 151936, 256, 16)
    assert 256 * 151936 * 2 < big < 1 << 30


def test_draft_block_rnn_validation():
    f = D.load().dspark_draft_block_rnn
    # bf16, rank 64, d 64; W_ih, W_hh, b_ih, b_hh at 11 .. 14; state 22; rows 23
    # (optional); ws_bytes 25
    base = [4, 1024, 64, 64, 4, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 7,
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a5=0) == D.DSPARK_ERR_DTYPE             # the state rows are bf16
    for i in (9, 10, 11, 12, 13, 14, 22):               # h, w, GRU weights and state
        assert call(**{f"a{i}": None}) == D.DSPARK_ERR_NULL
    assert call(a2=48) == D.DSPARK_ERR_SHAPE            # rank not a multiple of 32
    assert call(a3=40) == D.DSPARK_ERR_SHAPE            # d not a multiple of 16
    assert call(a15=-1.0) == D.DSPARK_ERR_VALUE
    need = D.dspark_workspace_bytes(D.DSPARK_OP_DRAFT_RNN, 4, 1024, 64, 4)
    assert need > D.dspark_workspace_bytes(D.DSPARK_OP_DRAFT_STEP, 4, 1024, 64, 4)
    assert call(a25=need - 1) == D.DSPARK_ERR_WORKSPACE
    assert D.dspark_workspace_bytes(D.DSPARK_OP_DRAFT_RNN, 4, 1024, 48, 4) == 0


def test_verify_rnn_validation():
    f = D.load().dspark_verify_rnn
    # rows at 10; ws_bytes at 22
    base = [4, 1024, 32, 4, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 7,
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a10=None) == D.DSPARK_ERR_NULL          # the bias rows are required
    assert call(a10=FAKE + 8) == D.DSPARK_ERR_SHAPE     # and 16-byte aligned
    assert call(a9=None) == D.DSPARK_ERR_NULL
    assert call(a14=-1.0) == D.DSPARK_ERR_VALUE
    assert call(a22=16) == D.DSPARK_ERR_WORKSPACE


def test_schedule_async_validation():
    f = D.load().dspark_schedule_async
    need = D.dspark_workspace_bytes(D.DSPARK_OP_SCHEDULE, 4, 2, 16, 4)
    assert f(4, 4, None, FAKE, FAKE, 21, FAKE, FAKE, FAKE, FAKE, need, None) == D.DSPARK_ERR_NULL
    assert f(4, 4, FAKE, None, FAKE, 21, FAKE, FAKE, FAKE, FAKE, need, None) == D.DSPARK_ERR_NULL
    assert f(4, 4, FAKE, FAKE, FAKE, 21, FAKE, None, FAKE, FAKE, need, None) == D.DSPARK_ERR_NULL
    assert f(4, 4, FAKE, FAKE, FAKE, 20, FAKE, FAKE, FAKE, FAKE, need, None) == D.DSPARK_ERR_SHAPE
    assert f(0, 4, FAKE, FAKE, FAKE, 10 ** 6, FAKE, FAKE, FAKE, FAKE, need, None) == \
        D.DSPARK_ERR_SHAPE
    assert f(512, 17, FAKE, FAKE, FAKE, 10 ** 6, FAKE, FAKE, FAKE, FAKE, need, None) == \
        D.DSPARK_ERR_SHAPE
    assert f(4, 4, FAKE, FAKE, FAKE, 21, FAKE, FAKE, FAKE, None, need, None) == \
        D.DSPARK_ERR_WORKSPACE
    assert f(4, 4, FAKE, FAKE, FAKE, 21, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        D.DSPARK_ERR_WORKSPACE


def test_confidence_validation():
    f = D.load().dspark_confidence
    assert f(4, 4, 64, 32, 1024, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == D.DSPARK_ERR_NULL
    assert f(4, 4, 64, 32, 1024, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == D.DSPARK_ERR_DTYPE
    assert f(4, 4, 0, 32, 1024, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == D.DSPARK_ERR_SHAPE
    assert f(4, 4, 64, 31, 1024, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == D.DSPARK_ERR_SHAPE


def _verify(**kw):
    a = dict(R=4, V=1024, rank=32, gamma=4, dt=0, W1=FAKE, W2t=FAKE, U=FAKE, target=FAKE,
             x=FAKE, lse_d=FAKE, p_d_x=FAKE, ell=FAKE, temperature=1.0, seed=0, c_star=FAKE,
             n_accept=FAKE, next_token=FAKE, tau=FAKE, tau_mean=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return D.load().dspark_verify(*[a[k] for k in (
        "R", "V", "rank", "gamma", "dt", "W1", "W2t", "U", "target", "x", "lse_d", "p_d_x",
        "ell", "temperature", "seed", "c_star", "n_accept", "next_token", "tau", "tau_mean",
        "ws", "ws_bytes")], None)


@pytest.mark.parametrize("kw,status", [
    (dict(target=None), D.DSPARK_ERR_NULL),
    (dict(tau_mean=None), D.DSPARK_ERR_NULL),
    (dict(dt=3), D.DSPARK_ERR_DTYPE),
    (dict(gamma=0), D.DSPARK_ERR_SHAPE),
    (dict(target=FAKE + 8), D.DSPARK_ERR_SHAPE),
    (dict(temperature=-0.5), D.DSPARK_ERR_VALUE),
    (dict(ws_bytes=0), D.DSPARK_ERR_WORKSPACE),
])
def test_verify_validation(kw, status):
    assert _verify(**kw) == status


def test_python_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        D._ptr(torch.zeros(4))


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus 2 exits at once with a message."""
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_token_errors_query_plumbing():
    """The token-error query checks its arguments before any HIP call, and
    without a usable GPU reports a launch error (leaving *flag alone) instead
    of crashing; the Python wrapper raises on that status."""
    import ctypes
    f = D.load().dspark_token_errors
    flag = ctypes.c_uint32(12345)
    assert f(None, 0) == D.DSPARK_ERR_NULL
    assert f(ctypes.byref(flag), 2) == D.DSPARK_ERR_VALUE
    assert f(ctypes.byref(flag), -1) == D.DSPARK_ERR_VALUE
    assert flag.value == 12345
    import torch
    if not torch.cuda.is_available():
        assert f(ctypes.byref(flag), 0) == D.DSPARK_ERR_LAUNCH
        assert f(ctypes.byref(flag), 1) == D.DSPARK_ERR_LAUNCH
        assert flag.value == 12345
        with pytest.raises(D.DsparkError):
            D.dspark_token_errors()

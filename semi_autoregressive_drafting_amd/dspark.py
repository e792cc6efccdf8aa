"""Python binding of libdspark.so (the C ABI in include/dspark.h).

Argument marshalling only: every function forwards to the C entry point of the
same name with device pointers taken from torch tensors and the current torch
stream.  Nothing here computes; there is no fallback when the library is
missing -- importing the functions works anywhere, calling them requires the
built library (and, for compute calls, a GPU).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSPARK_LIB selects another build of the same library (e.g. the one whose
# host layer is built with sanitizers, build.build_host_sanitized()).
LIB_PATH = os.environ.get("DSPARK_LIB") or os.path.join(_HERE, "libdspark.so")

DSPARK_OK, DSPARK_ERR_NULL, DSPARK_ERR_SHAPE, DSPARK_ERR_DTYPE, DSPARK_ERR_VALUE, \
    DSPARK_ERR_WORKSPACE, DSPARK_ERR_LAUNCH = range(7)
DSPARK_F32, DSPARK_BF16 = 0, 1
DSPARK_OP_DRAFT_STEP, DSPARK_OP_SCHEDULE, DSPARK_OP_VERIFY, DSPARK_OP_TRAIN_LOSS, \
    DSPARK_OP_TRAIN_GRAD, DSPARK_OP_DRAFT_RNN = 0, 1, 2, 3, 4, 5
DSPARK_PHASE_STEPS, DSPARK_PHASE_MERGE = 1, 2

EXPORTS = ("dspark_workspace_bytes", "dspark_status_string", "dspark_draft_step",
           "dspark_draft_block", "dspark_draft_block_phases", "dspark_confidence", "dspark_schedule", "dspark_schedule_async",
           "dspark_verify", "dspark_train_loss", "dspark_train_loss_grad",
           "dspark_draft_block_rnn", "dspark_verify_rnn", "dspark_draft_block_noalloc",
           "dspark_token_errors")

_lib = None


class DsparkError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def load():
    """Load libdspark.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m semi_autoregressive_drafting_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, U64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, ctypes.c_size_t
    L.dspark_workspace_bytes.argtypes = [I, I, I, I, I]
    L.dspark_workspace_bytes.restype = SZ
    L.dspark_status_string.argtypes = [I]
    L.dspark_status_string.restype = ctypes.c_char_p
    L.dspark_token_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32), I]
    L.dspark_token_errors.restype = I
    L.dspark_draft_step.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, F, U64,
                                    P, P, P, P, P, P, P, SZ, P]
    L.dspark_draft_step.restype = I
    L.dspark_draft_block.argtypes = [I, I, I, I, I, I, P, P, P, P, P, F, U64,
                                     P, P, P, P, P, P, SZ, P]
    L.dspark_draft_block.restype = I
    L.dspark_draft_block_phases.argtypes = [I, I, I, I, I, I, P, P, P, P, P, F, U64,
                                            P, P, P, P, P, P, SZ, I, P]
    L.dspark_draft_block_phases.restype = I
    L.dspark_draft_block_noalloc.argtypes = [I, I, I, I, I, I, P, P, P, P, P, F, U64,
                                             P, P, P, P, P, P]
    L.dspark_draft_block_noalloc.restype = I
    L.dspark_confidence.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P]
    L.dspark_confidence.restype = I
    L.dspark_schedule.argtypes = [I, I, P, P, I, P, P, P, P, SZ, P]
    L.dspark_schedule.restype = I
    L.dspark_schedule_async.argtypes = [I, I, P, P, P, I, P, P, P, P, SZ, P]
    L.dspark_schedule_async.restype = I
    L.dspark_verify.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, F, U64,
                                P, P, P, P, P, P, SZ, P]
    L.dspark_verify.restype = I
    L.dspark_train_loss.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, F, F, F, F, F,
                                    P, P, P, SZ, P]
    L.dspark_train_loss.restype = I
    L.dspark_train_loss_grad.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, F, F, F, F, F,
                                         P, P, P, P, P, P, P, P, SZ, P]
    L.dspark_train_loss_grad.restype = I
    L.dspark_draft_block_rnn.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, F, U64,
                                         P, P, P, P, P, P, P, P, SZ, P]
    L.dspark_verify_rnn.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, F, U64,
                                    P, P, P, P, P, P, SZ, P]
    L.dspark_verify_rnn.restype = I
    L.dspark_draft_block_rnn.restype = I
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().dspark_status_string(int(status)).decode()


def _ptr(t):
    """Device pointer of a torch tensor (or an int address / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("dspark: tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("dspark: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if not torch.cuda.is_available():
        return None
    return torch.cuda.current_stream().cuda_stream


def _call(fn, *args):
    status = getattr(load(), fn)(*args)
    if status != DSPARK_OK:
        raise DsparkError(fn, status)


def dspark_workspace_bytes(op, R, V, rank, gamma) -> int:
    return int(load().dspark_workspace_bytes(op, R, V, rank, gamma))


def dspark_token_errors(clear=False) -> int:
    """The current device's token-error word (1 if some kernel met a token id
    outside [0, V) since the last clear); clear=True resets it.  Synchronise
    the streams that ran the kernels first."""
    flag = ctypes.c_uint32(0)
    _call("dspark_token_errors", ctypes.byref(flag), 1 if clear else 0)
    return int(flag.value)


def dspark_draft_step(R, V, rank, d, gamma, k, dt, W1, W2t, U, h, w, temperature, seed,
                      x, p, lse, c, a, z_debug, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_draft_step", R, V, rank, d, gamma, k, dt, _ptr(W1), _ptr(W2t), _ptr(U),
          _ptr(h), _ptr(w), float(temperature), int(seed), _ptr(x), _ptr(p), _ptr(lse),
          _ptr(c), _ptr(a), _ptr(z_debug), _ptr(ws), int(ws_bytes), _stream(stream))


def dspark_draft_block(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, temperature, seed,
                       x, p, lse, c, a, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_draft_block", R, V, rank, d, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U),
          _ptr(h), _ptr(w), float(temperature), int(seed), _ptr(x), _ptr(p), _ptr(lse),
          _ptr(c), _ptr(a), _ptr(ws), int(ws_bytes), _stream(stream))


def dspark_draft_block_noalloc(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, temperature, seed,
                               x, p, lse, c, a, stream=None):
    _call("dspark_draft_block_noalloc", R, V, rank, d, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U),
          _ptr(h), _ptr(w), float(temperature), int(seed), _ptr(x), _ptr(p), _ptr(lse),
          _ptr(c), _ptr(a), _stream(stream))


def dspark_draft_block_phases(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, temperature, seed,
                              x, p, lse, c, a, ws, phases, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_draft_block_phases", R, V, rank, d, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U),
          _ptr(h), _ptr(w), float(temperature), int(seed), _ptr(x), _ptr(p), _ptr(lse),
          _ptr(c), _ptr(a), _ptr(ws), int(ws_bytes), int(phases), _stream(stream))


def dspark_confidence(R, gamma, d, rank, V, dt, h, W1, x, w, c, a, stream=None):
    _call("dspark_confidence", R, gamma, d, rank, V, dt, _ptr(h), _ptr(W1), _ptr(x), _ptr(w),
          _ptr(c), _ptr(a), _stream(stream))


def dspark_schedule(R, gamma, a, sps, sps_len, ell, budget, theta, ws, ws_bytes=None,
                    stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_schedule", R, gamma, _ptr(a), _ptr(sps), int(sps_len), _ptr(ell),
          _ptr(budget), _ptr(theta), _ptr(ws), int(ws_bytes), _stream(stream))


def dspark_schedule_async(R, gamma, a_lag, a_cur, sps, sps_len, ell, budget, theta, ws,
                          ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_schedule_async", R, gamma, _ptr(a_lag), _ptr(a_cur), _ptr(sps), int(sps_len),
          _ptr(ell), _ptr(budget), _ptr(theta), _ptr(ws), int(ws_bytes), _stream(stream))


def dspark_verify(R, V, rank, gamma, dt, W1, W2t, U, target, x, lse_d, p_d_x, ell,
                  temperature, seed, c_star, n_accept, next_token, tau, tau_mean, ws,
                  ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_verify", R, V, rank, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U), _ptr(target),
          _ptr(x), _ptr(lse_d), _ptr(p_d_x), _ptr(ell), float(temperature), int(seed),
          _ptr(c_star), _ptr(n_accept), _ptr(next_token), _ptr(tau), _ptr(tau_mean), _ptr(ws),
          int(ws_bytes), _stream(stream))


def dspark_train_loss(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, target, x_star, temperature,
                      lam, alpha_ce, alpha_tv, alpha_conf, terms, sums, ws, ws_bytes=None,
                      stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_train_loss", R, V, rank, d, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U), _ptr(h),
          _ptr(w), _ptr(target), _ptr(x_star), float(temperature), float(lam), float(alpha_ce),
          float(alpha_tv), float(alpha_conf), _ptr(terms), _ptr(sums), _ptr(ws), int(ws_bytes),
          _stream(stream))


def dspark_train_loss_grad(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, target, x_star,
                           temperature, lam, alpha_ce, alpha_tv, alpha_conf, terms, sums, dU, dW1,
                           dW2t, dh, dw, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_train_loss_grad", R, V, rank, d, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U),
          _ptr(h), _ptr(w), _ptr(target), _ptr(x_star), float(temperature), float(lam),
          float(alpha_ce), float(alpha_tv), float(alpha_conf), _ptr(terms), _ptr(sums), _ptr(dU),
          _ptr(dW1), _ptr(dW2t), _ptr(dh), _ptr(dw), _ptr(ws), int(ws_bytes), _stream(stream))


def dspark_draft_block_rnn(R, V, rank, d, gamma, dt, W1, W2t, U, h, w, W_ih, W_hh, b_ih, b_hh,
                           temperature, seed, x, p, lse, c, a, state, rows, ws, ws_bytes=None,
                           stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_draft_block_rnn", R, V, rank, d, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U),
          _ptr(h), _ptr(w), _ptr(W_ih), _ptr(W_hh), _ptr(b_ih), _ptr(b_hh), float(temperature),
          int(seed), _ptr(x), _ptr(p), _ptr(lse), _ptr(c), _ptr(a), _ptr(state), _ptr(rows),
          _ptr(ws), int(ws_bytes), _stream(stream))


def dspark_verify_rnn(R, V, rank, gamma, dt, W1, W2t, U, target, x, rows, lse_d, p_d_x, ell,
                      temperature, seed, c_star, n_accept, next_token, tau, tau_mean, ws,
                      ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _call("dspark_verify_rnn", R, V, rank, gamma, dt, _ptr(W1), _ptr(W2t), _ptr(U), _ptr(target),
          _ptr(x), _ptr(rows), _ptr(lse_d), _ptr(p_d_x), _ptr(ell), float(temperature), int(seed),
          _ptr(c_star), _ptr(n_accept), _ptr(next_token), _ptr(tau), _ptr(tau_mean), _ptr(ws),
          int(ws_bytes), _stream(stream))

"""Device-side orchestration of one DSpark round through the C ABI.

Uploads a workload's inputs to GPU memory and enqueues the entry points of
libdspark.so in order (gamma draft steps, schedule, verify).  It only moves
buffers and calls the library; every step of the method runs in its kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import dspark as D
from .synth import Inputs


@dataclass
class DeviceInputs:
    R: int
    V: int
    rank: int
    d: int
    gamma: int
    dt: int
    W1: torch.Tensor
    W2t: torch.Tensor
    U: torch.Tensor
    h: torch.Tensor
    w: torch.Tensor
    anchor: torch.Tensor
    sps: torch.Tensor
    target: torch.Tensor | None

    @staticmethod
    def upload(inp: Inputs, device="cuda") -> "DeviceInputs":
        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)
        wl = inp.wl
        return DeviceInputs(
            R=len(inp.req_ids), V=wl.V, rank=wl.rank, d=wl.d, gamma=wl.gamma,
            dt=D.DSPARK_BF16 if wl.dtype == "bf16" else D.DSPARK_F32,
            W1=dev(inp.W1_store), W2t=dev(inp.W2t_store), U=dev(inp.U), h=dev(inp.h_store),
            w=dev(inp.w), anchor=dev(inp.anchor.astype(np.int32)), sps=dev(inp.sps),
            target=dev(inp.target) if inp.target is not None else None)


@dataclass
class RoundBuffers:
    x: torch.Tensor        # [R, gamma+1] int32
    p: torch.Tensor        # [R, gamma] f32
    lse: torch.Tensor
    c: torch.Tensor
    a: torch.Tensor
    ws: torch.Tensor       # draft-step workspace
    ell: torch.Tensor      # [R] int32
    budget: torch.Tensor   # [1] int32
    theta: torch.Tensor    # [1] f64
    c_star: torch.Tensor   # [R, gamma] f32
    n_accept: torch.Tensor
    next_token: torch.Tensor
    tau: torch.Tensor
    tau_mean: torch.Tensor
    vws: torch.Tensor      # verify workspace
    sws: torch.Tensor      # scheduler workspace

    @staticmethod
    def allocate(di: DeviceInputs, device="cuda") -> "RoundBuffers":
        R, g = di.R, di.gamma
        f32 = dict(dtype=torch.float32, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        ws = D.dspark_workspace_bytes(D.DSPARK_OP_DRAFT_STEP, R, di.V, di.rank, g)
        vws = D.dspark_workspace_bytes(D.DSPARK_OP_VERIFY, R, di.V, di.rank, g)
        sws = D.dspark_workspace_bytes(D.DSPARK_OP_SCHEDULE, R, di.V, di.rank, g)
        return RoundBuffers(
            x=torch.zeros((R, g + 1), **i32), p=torch.zeros((R, g), **f32),
            lse=torch.zeros((R, g), **f32), c=torch.zeros((R, g), **f32),
            a=torch.zeros((R, g), **f32),
            ws=torch.zeros(max(ws, 16), dtype=torch.uint8, device=device),  # zero-filled once
            ell=torch.zeros(R, **i32), budget=torch.zeros(1, **i32),
            theta=torch.zeros(1, dtype=torch.float64, device=device),
            c_star=torch.zeros((R, g), **f32), n_accept=torch.zeros(R, **i32),
            next_token=torch.zeros(R, **i32), tau=torch.zeros(R, **i32),
            tau_mean=torch.zeros(1, **f32),
            vws=torch.empty(max(vws, 16), dtype=torch.uint8, device=device),
            sws=torch.zeros(max(sws, 16), dtype=torch.uint8, device=device))  # zero-filled once


def draft_step(di: DeviceInputs, buf: RoundBuffers, k: int, temperature: float, seed: int,
               z_debug: torch.Tensor | None = None, confidence: bool = True):
    D.dspark_draft_step(di.R, di.V, di.rank, di.d, di.gamma, k, di.dt, di.W1, di.W2t, di.U,
                        di.h if confidence else None, di.w if confidence else None,
                        temperature, seed, buf.x, buf.p, buf.lse,
                        buf.c if confidence else None, buf.a if confidence else None,
                        z_debug, buf.ws)


def draft(di: DeviceInputs, buf: RoundBuffers, temperature: float, seed: int):
    """gamma sequential draft steps (with confidence and survival) in one call."""
    buf.x[:, 0].copy_(di.anchor)
    D.dspark_draft_block(di.R, di.V, di.rank, di.d, di.gamma, di.dt, di.W1, di.W2t, di.U, di.h,
                         di.w, temperature, seed, buf.x, buf.p, buf.lse, buf.c, buf.a, buf.ws)


def draft_phases(di: DeviceInputs, buf: RoundBuffers, temperature: float, seed: int,
                 phases: int, copy_anchor: bool = True):
    """One phase (or both) of draft(): D.DSPARK_PHASE_STEPS runs the anchor
    copy (unless the caller has placed the anchor itself) and the gamma
    streaming steps, D.DSPARK_PHASE_MERGE the record merge."""
    if phases & D.DSPARK_PHASE_STEPS and copy_anchor:
        buf.x[:, 0].copy_(di.anchor)
    D.dspark_draft_block_phases(di.R, di.V, di.rank, di.d, di.gamma, di.dt, di.W1, di.W2t, di.U,
                                di.h, di.w, temperature, seed, buf.x, buf.p, buf.lse, buf.c,
                                buf.a, buf.ws, phases)


def schedule(di: DeviceInputs, buf: RoundBuffers):
    D.dspark_schedule(di.R, di.gamma, buf.a, di.sps, di.sps.numel(), buf.ell, buf.budget,
                      buf.theta, buf.sws)


def schedule_async(di: DeviceInputs, buf: RoundBuffers, a_lag: torch.Tensor):
    """Asynchronous scheduling: budget from a_lag (survival two steps old),
    selection from buf.a."""
    D.dspark_schedule_async(di.R, di.gamma, a_lag, buf.a, di.sps, di.sps.numel(), buf.ell,
                            buf.budget, buf.theta, buf.sws)


def verify(di: DeviceInputs, buf: RoundBuffers, temperature: float, seed: int):
    D.dspark_verify(di.R, di.V, di.rank, di.gamma, di.dt, di.W1, di.W2t, di.U, di.target,
                    buf.x, buf.lse, buf.p, buf.ell, temperature, seed, buf.c_star,
                    buf.n_accept, buf.next_token, buf.tau, buf.tau_mean, buf.vws)


def full_round(di: DeviceInputs, buf: RoundBuffers, temperature: float, seed: int):
    """One pass of the whole hot path: draft (gamma steps, confidence, survival),
    schedule, verify."""
    draft(di, buf, temperature, seed)
    schedule(di, buf)
    if di.target is not None:
        verify(di, buf, temperature, seed)


def train_loss(di: DeviceInputs, x_star: torch.Tensor, temperature: float = 1.0,
               lam: float | None = None, alphas=(0.1, 0.9, 1.0), ws: torch.Tensor | None = None):
    """The training losses of the workload's blocks with x_star [R][gamma+1] as
    the target block; returns (terms [R][gamma][4], sums [4]) on the device."""
    R, g = di.R, di.gamma
    lam = float(g) if lam is None else lam
    if ws is None:
        nb = D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_LOSS, R, di.V, di.rank, g)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=di.U.device)
    terms = torch.empty((R, g, 4), dtype=torch.float32, device=di.U.device)
    sums = torch.empty(4, dtype=torch.float64, device=di.U.device)
    D.dspark_train_loss(R, di.V, di.rank, di.d, g, di.dt, di.W1, di.W2t, di.U, di.h, di.w,
                        di.target, x_star, temperature, lam, alphas[0], alphas[1], alphas[2],
                        terms, sums, ws)
    return terms, sums


def train_loss_grad(di: DeviceInputs, x_star: torch.Tensor, temperature: float = 1.0,
                    lam: float | None = None, alphas=(0.1, 0.9, 1.0), ws: torch.Tensor | None = None):
    """The training losses and their gradients; returns a dict of device tensors
    terms [R][gamma][4], sums [4], dU [R][gamma][V], dW1 [V][rank],
    dW2t [V][rank], dh [R][gamma][d], dw [d + rank]."""
    R, g, V, rank, d = di.R, di.gamma, di.V, di.rank, di.d
    lam = float(g) if lam is None else lam
    dev = di.U.device
    if ws is None:
        nb = D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_GRAD, R, V, rank, g)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    out = {"terms": torch.empty((R, g, 4), dtype=torch.float32, device=dev),
           "sums": torch.empty(4, dtype=torch.float64, device=dev),
           "dU": torch.empty((R, g, V), dtype=torch.float32, device=dev),
           "dW1": torch.empty((V, rank), dtype=torch.float32, device=dev),
           "dW2t": torch.empty((V, rank), dtype=torch.float32, device=dev),
           "dh": torch.empty((R, g, d), dtype=torch.float32, device=dev),
           "dw": torch.empty(d + rank, dtype=torch.float32, device=dev)}
    D.dspark_train_loss_grad(R, V, rank, d, g, di.dt, di.W1, di.W2t, di.U, di.h, di.w, di.target,
                             x_star, temperature, lam, alphas[0], alphas[1], alphas[2],
                             out["terms"], out["sums"], out["dU"], out["dW1"], out["dW2t"],
                             out["dh"], out["dw"], ws)
    return out


@dataclass
class RnnWeights:
    W_ih: torch.Tensor
    W_hh: torch.Tensor
    b_ih: torch.Tensor
    b_hh: torch.Tensor

    @staticmethod
    def upload(gru, device="cuda") -> "RnnWeights":
        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)
        return RnnWeights(*(dev(a) for a in gru))


def draft_rnn(di: DeviceInputs, buf: RoundBuffers, rw: RnnWeights, temperature: float, seed: int,
              state: torch.Tensor, ws: torch.Tensor, rows: torch.Tensor | None = None):
    """gamma steps of the RNN head (state update, then the draft step) and the
    record merge; s_gamma lands in `state` [R][rank] fp32 and, if given, the
    bias rows bf16(s_k) of every position in `rows` [R][gamma][rank] (int16
    storage).  `ws` holds dspark_workspace_bytes(DSPARK_OP_DRAFT_RNN, ...)
    bytes, zero-filled once."""
    buf.x[:, 0].copy_(di.anchor)
    D.dspark_draft_block_rnn(di.R, di.V, di.rank, di.d, di.gamma, di.dt, di.W1, di.W2t, di.U, di.h,
                             di.w, rw.W_ih, rw.W_hh, rw.b_ih, rw.b_hh, temperature, seed, buf.x,
                             buf.p, buf.lse, buf.c, buf.a, state, rows, ws)


def verify_rnn(di: DeviceInputs, buf: RoundBuffers, rows: torch.Tensor, temperature: float,
               seed: int):
    """Verification of an RNN-head block, its bias rows from draft_rnn."""
    D.dspark_verify_rnn(di.R, di.V, di.rank, di.gamma, di.dt, di.W1, di.W2t, di.U, di.target,
                        buf.x, rows, buf.lse, buf.p, buf.ell, temperature, seed, buf.c_star,
                        buf.n_accept, buf.next_token, buf.tau, buf.tau_mean, buf.vws)

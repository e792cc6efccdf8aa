"""Seeded synthetic inputs for the DSpark drafting hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no bias, softmax, sampling, confidence, schedule or
verification).  Both the HIP path and the CPU oracle read the arrays it returns,
so the two sides always see the same bytes.

Workloads (shapes follow the Qwen3 family the pages evaluate on: vocabulary
151936, Markov rank 256, block lengths 7 and 16, batches up to 512):

  tiny_v1024_r4_g4         V=1024, rank 32, d 64, gamma 4, R 4, all fp32,
                           plus target logits = U + N(0, 1)
  qwen3_4b_r32_g7          V=151936, rank 256, d 2560, gamma 7,  R 32,  bf16
  qwen3_8b_r128_g16        V=151936, rank 256, d 4096, gamma 16, R 128, bf16,
                           requests 0..R/2-1 "easy", R/2..R-1 "hard"
  qwen3_14b_r512_g7        V=151936, rank 256, d 5120, gamma 7,  R 512, bf16
  round_4b_r128_g7         V=151936, rank 256, d 2560, gamma 7,  R 128, bf16,
                           plus target logits = U + N(0, 1)
  bruteforce_v8_g3         V=8, rank 4, d 4, gamma 3, R 1, fp32 (enumeration)

Distributions (one PCG64 stream per array, and per request for the per-request
arrays, so any subset of requests can be regenerated on its own):
  U       N(0, 2^2) fp32.  tiny: 3 distinct random tokens per row get +6.
          Others: a Zipf(1.1)-ranked peak per row: 64 distinct uniform token
          ids, the i-th (i = 1..64) gets + P * i^-1.1, with P ~ U[4, 10]
          (easy requests: P = 10, hard: P = 3).
  W1, W2  N(0, 0.05^2), rounded to bf16 (round-to-nearest-even) for bf16
          workloads.  W2 (rank x V in the pages' notation) is stored
          vocabulary-major as W2t[V, rank] (the layout of a rank->vocab linear
          layer's weight).
  h       N(0, 1).  Easy/hard split: h = z + mu * w_h / |w_h|^2 with mu = +3
          (easy) or -1 (hard), so that w_h . h = w_h . z + mu.
  w       N(0, 1/(d + rank)) fp32, ordered [w_h (d); w_e (rank)].
  anchor  uniform token ids (int32).
  target  U + N(0, 1) fp32 (full-round and tiny workloads).
  sps     SPS(B) = 1 / max(5.97e-3, 3.24e-5 * B) steps/s for B = 0..R(1+gamma).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

# Array tags for the per-array seed sequences.
_TAG_U, _TAG_PEAK, _TAG_W1, _TAG_W2, _TAG_H, _TAG_W, _TAG_ANCHOR, _TAG_TARGET = range(1, 9)
_TAG_GRU = 9


@dataclass(frozen=True)
class Workload:
    name: str
    V: int
    rank: int
    d: int
    gamma: int
    R: int
    dtype: str                    # "f32" or "bf16": W1, W2t and h
    temperatures: tuple = (1.0,)
    weight_std: float = 0.05
    peak: str = "zipf"            # "zipf", "three", "none"
    easy_hard: bool = False
    target: bool = False
    sps_c0: float = 5.97e-3       # flat part of the step-time model (s)
    sps_kappa: float = 3.24e-5    # per-token slope of the step-time model (s)
    description: str = ""


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_v1024_r4_g4", V=1024, rank=32, d=64, gamma=4, R=4, dtype="f32",
                 peak="three", temperatures=(1.0, 0.0), target=True,
                 description="tiny CPU-checkable instance, all fp32"),
        Workload("qwen3_4b_r32_g7", V=151936, rank=256, d=2560, gamma=7, R=32, dtype="bf16",
                 description="Qwen3-4B-shaped draft round"),
        Workload("qwen3_8b_r128_g16", V=151936, rank=256, d=4096, gamma=16, R=128,
                 dtype="bf16", easy_hard=True,
                 description="Qwen3-8B-shaped long block, half easy / half hard requests"),
        Workload("qwen3_14b_r512_g7", V=151936, rank=256, d=5120, gamma=7, R=512,
                 dtype="bf16", temperatures=(1.0, 0.0),
                 description="Qwen3-14B-shaped saturated batch, greedy and T=1"),
        Workload("round_4b_r128_g7", V=151936, rank=256, d=2560, gamma=7, R=128,
                 dtype="bf16", target=True,
                 description="full draft + verify round with synthetic target logits"),
        Workload("bruteforce_v8_g3", V=8, rank=4, d=4, gamma=3, R=1, dtype="f32",
                 weight_std=1.0, peak="none", temperatures=(1.0, 0.7),
                 description="brute-force enumeration instance"),
    ]
}


def custom(name: str, **kw) -> Workload:
    """Register an ad-hoc workload (edge and ragged shapes for tests)."""
    wl = Workload(name=name, **kw)
    WORKLOADS[name] = wl
    return wl


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, tags)])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """All arrays of one workload instance.  Weights and h are given both as the
    storage the GPU reads (`*_store`: uint16 bf16 bits or float32) and as exact
    float32 values (`*_f32`)."""
    wl: Workload
    seed: int
    req_ids: np.ndarray           # which requests these rows are (subset support)
    U: np.ndarray                 # [n, gamma, V] f32
    W1_store: np.ndarray          # [V, rank] uint16 bits or f32
    W2t_store: np.ndarray         # [V, rank] uint16 bits or f32
    h_store: np.ndarray           # [n, gamma, d] uint16 bits or f32
    w: np.ndarray                 # [d + rank] f32
    anchor: np.ndarray            # [n] int32
    sps: np.ndarray               # [R(1+gamma)+1] f64
    target: np.ndarray | None = None   # [n, gamma, V] f32
    extra: dict = field(default_factory=dict)

    @property
    def W1_f32(self):
        return bf16_bits_to_f32(self.W1_store) if self.W1_store.dtype == np.uint16 else self.W1_store

    @property
    def W2t_f32(self):
        return bf16_bits_to_f32(self.W2t_store) if self.W2t_store.dtype == np.uint16 else self.W2t_store

    @property
    def h_f32(self):
        return bf16_bits_to_f32(self.h_store) if self.h_store.dtype == np.uint16 else self.h_store


def sps_table(R: int, gamma: int, c0: float = 5.97e-3, kappa: float = 3.24e-5) -> np.ndarray:
    B = np.arange(R * (1 + gamma) + 1, dtype=np.float64)
    return 1.0 / np.maximum(c0, kappa * B)


def _weights(wl: Workload, seed: int, tag: int) -> np.ndarray:
    x = _rng(seed, tag).standard_normal((wl.V, wl.rank), dtype=np.float32) * np.float32(wl.weight_std)
    return f32_to_bf16_bits(x) if wl.dtype == "bf16" else x


def _request_rows(wl: Workload, seed: int, req: int, w_h: np.ndarray):
    """U row block, h row block and (optionally) target block of one request."""
    g = wl.gamma
    U = _rng(seed, _TAG_U, req).standard_normal((g, wl.V), dtype=np.float32) * np.float32(2.0)
    prng = _rng(seed, _TAG_PEAK, req)
    if wl.peak == "three":
        for k in range(g):
            ids = prng.choice(wl.V, size=3, replace=False)
            U[k, ids] += np.float32(6.0)
    elif wl.peak == "zipf":
        ranks = np.arange(1, 65, dtype=np.float64) ** -1.1
        for k in range(g):
            if wl.easy_hard:
                P = 10.0 if req < wl.R // 2 else 3.0
            else:
                P = prng.uniform(4.0, 10.0)
            ids = prng.choice(wl.V, size=64, replace=False)
            U[k, ids] += (P * ranks).astype(np.float32)
    hz = _rng(seed, _TAG_H, req).standard_normal((g, wl.d), dtype=np.float32)
    if wl.easy_hard:
        mu = 3.0 if req < wl.R // 2 else -1.0
        shift = (mu * w_h.astype(np.float64) / float(np.dot(w_h.astype(np.float64), w_h))).astype(np.float32)
        hz = hz + shift[None, :]
    T = None
    if wl.target:
        T = U + _rng(seed, _TAG_TARGET, req).standard_normal((g, wl.V), dtype=np.float32)
    return U, hz, T


def generate(name: str, seed: int = 0, requests=None, threads: int | None = None,
             target: bool | None = None) -> Inputs:
    """Build the inputs of workload `name`.  `requests` (optional) selects a subset
    of request indices; each request's rows do not depend on which others are made.
    `target` overrides whether target logits (U + N(0, 1)) are drawn."""
    wl = WORKLOADS[name]
    if target is not None and target != wl.target:
        wl = Workload(**{**wl.__dict__, "target": target})
    req_ids = np.arange(wl.R) if requests is None else np.asarray(requests, dtype=np.int64)
    n = len(req_ids)
    w = (_rng(seed, _TAG_W).standard_normal(wl.d + wl.rank, dtype=np.float32)
         * np.float32(1.0 / np.sqrt(wl.d + wl.rank)))
    W1 = _weights(wl, seed, _TAG_W1)
    W2t = _weights(wl, seed, _TAG_W2)
    anchor_all = _rng(seed, _TAG_ANCHOR).integers(0, wl.V, size=wl.R, dtype=np.int64).astype(np.int32)

    U = np.empty((n, wl.gamma, wl.V), dtype=np.float32)
    h = np.empty((n, wl.gamma, wl.d), dtype=np.float32)
    T = np.empty((n, wl.gamma, wl.V), dtype=np.float32) if wl.target else None
    w_h = w[: wl.d]

    def work(i):
        u, hh, t = _request_rows(wl, seed, int(req_ids[i]), w_h)
        U[i] = u
        h[i] = hh
        if T is not None:
            T[i] = t

    nthreads = threads or min(16, os.cpu_count() or 1)
    if n * wl.gamma * wl.V > 4_000_000 and nthreads > 1:
        with _cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(n)))
    else:
        for i in range(n):
            work(i)
    h_store = f32_to_bf16_bits(h) if wl.dtype == "bf16" else h
    return Inputs(wl=wl, seed=seed, req_ids=req_ids, U=U, W1_store=W1, W2t_store=W2t,
                  h_store=h_store, w=w, anchor=anchor_all[req_ids],
                  sps=sps_table(wl.R, wl.gamma, wl.sps_c0, wl.sps_kappa), target=T)


def gru_weights(wl: Workload, seed: int = 0):
    """Weights of the RNN head's gated state update, gate blocks in the order
    (reset, update, new): W_ih [3 rank][rank + d] and W_hh [3 rank][rank] in the
    workload's storage (bf16 bits or fp32), N(0, 1/(rank + d)) and
    N(0, 1/rank) so that gate pre-activations are O(1); b_ih, b_hh [3 rank]
    fp32 ~ N(0, 0.1^2)."""
    g = _rng(seed, _TAG_GRU)
    H, D = wl.rank, wl.rank + wl.d
    W_ih = g.standard_normal((3 * H, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    W_hh = g.standard_normal((3 * H, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    b_ih = g.standard_normal(3 * H, dtype=np.float32) * np.float32(0.1)
    b_hh = g.standard_normal(3 * H, dtype=np.float32) * np.float32(0.1)
    if wl.dtype == "bf16":
        W_ih, W_hh = f32_to_bf16_bits(W_ih), f32_to_bf16_bits(W_hh)
    return W_ih, W_hh, b_ih, b_hh

#!/usr/bin/env python3
"""Benchmark of the DSpark drafting hot path on one MI355X.

One step = one pass of the whole hot path over one batch: gamma sequential
Markov draft steps (gather, MFMA bias, base-logit add, online softmax,
Gumbel-argmax, confidence head, survival product), the prefix scheduler and
verification (c*, rejection sampling).  Workload: R = 128 requests, gamma = 16,
V = 151936, rank 256, d = 4096, bf16 weights, fp32 logits (the Qwen3-8B-shaped
long-block workload), plus synthetic target logits U + N(0, 1) for the
verification pass.  All inputs are resident in GPU memory before timing starts.

Prints one JSON line.  `value` = draft tokens per second of the whole round
(R * gamma / wall-clock time per round).  `roofline` covers the draft step
kernel (markov_step_shared), timed with events on the stream it runs on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

WORKLOAD = "qwen3_8b_r128_g16"
HBM_PEAK_GBS = 8000.0
TEMPERATURE = 1.0


def draft_step_bytes(R, V, rank, d):
    """Algorithmic HBM bytes of one draft step: W2 once (rank*V bf16), U_k
    (R*V fp32), the gathered W1 rows (R*rank bf16), h_k (R*d bf16) and the
    per-request outputs (token, p, lse, c, a: 20 bytes)."""
    return rank * V * 2 + R * V * 4 + R * rank * 2 + R * d * 2 + R * 20


def verify_bytes(R, V, rank, gamma):
    """Algorithmic bytes of verification: the target logits twice (normaliser
    pass, then the fused pass), U and W2 once."""
    return 2 * R * gamma * V * 4 + R * gamma * V * 4 + rank * V * 2


def train_loss_bytes(R, V, rank, d, gamma):
    """Algorithmic bytes of the forward training losses: the target logits
    twice (normaliser pass, then the TV pass), U and W2 twice (draft
    normaliser pass, then the TV pass) and h once."""
    n = R * gamma
    return 2 * n * V * 4 + 2 * n * V * 4 + 2 * rank * V * 2 + n * d * 2


def train_grad_bytes(R, V, rank, d, gamma):
    """Algorithmic bytes of the losses with every gradient: the forward
    passes; the logit-gradient pass (target, U and W2 read, dU written); the
    two contractions (dU read by each, W2 transposed once, dW2t written);
    dW1 cleared and the confidence-head inputs read once more."""
    n = R * gamma
    fwd = train_loss_bytes(R, V, rank, d, gamma)
    return (fwd + (2 * n * V * 4 + rank * V * 2 + n * V * 4) + 2 * n * V * 4
            + 2 * rank * V * 2 + V * rank * 4 + V * rank * 4 + n * d * 2)


PROFILE_COUNTERS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                "dspark_round_qwen3_8b_r128_g16_hbm_counters.txt")


# Sources the draft step kernel is compiled from (the counters go stale when
# any of them changes).
DRAFT_KERNEL_SOURCES = ("markov_step.hip", "mfma_stream.h", "dspark_device.h", "draft_step.h")


def sources_sha256():
    """Hash of the draft kernel's sources (by name and bytes, in that order)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "semi_autoregressive_drafting_amd", "csrc")
    for name in DRAFT_KERNEL_SOURCES:
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the draft kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (both scaled by a plain-copy calibration),
    or None when the kernel sources have changed since it was taken."""
    try:
        with open(PROFILE_COUNTERS) as fh:
            lines = [l for l in fh if l.startswith("traffic markov_step_shared ")]
    except OSError:
        return None
    if not lines:
        return None
    kv = dict(t.split("=", 1) for t in lines[-1].split()[2:])
    if kv.get("source_sha256") != sources_sha256():
        return None
    return int(kv["read_bytes"]) + int(kv["write_bytes"])


COLD_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "dspark_markov_step_qwen3_8b_r128_g16_cold_kernel_stats.txt")


def profiled_cold_us():
    """Average kernel duration of the cold single draft steps from the
    committed rocprofv3 kernel-trace summary of `bench.py --cold-only`, or
    None when the kernel sources have changed since it was taken."""
    try:
        with open(COLD_PROFILE) as fh:
            lines = [l for l in fh if l.startswith("cold markov_step_shared ")]
    except OSError:
        return None
    if not lines:
        return None
    kv = dict(t.split("=", 1) for t in lines[-1].split()[2:])
    if kv.get("source_sha256") != sources_sha256():
        return None
    return float(kv["avg_us"])


def read_ceiling(nbytes, launches=20):
    """Pure-read streams over nbytes with the probe kernels (libdspark_probe.so).

    'rotating' reads a different nbytes window of a pool several times larger
    than the MALL at each launch (so every byte comes from HBM), 'resident'
    re-reads one window (as the draft step re-reads W2 every step).  The
    probe's variants are swept (16-byte loads in flight per lane, nontemporal
    or cached loads, interleaved or one slice per workgroup, grid size); the
    fastest rotating variant is the read ceiling.  GB/s per launch, timed with
    HIP events on the stream the probe runs on."""
    import torch
    lib = _probe_lib()
    nbytes = (nbytes + 255) // 256 * 256
    slots = 12
    pool = torch.empty(nbytes * slots, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    grids = (256, 512, 1024, 2048, 4096)
    sink = torch.zeros(max(grids), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(mode, unroll, nt, blocked, grid):
        def launch(i):
            off = (i % slots) * nbytes if mode == "rotating" else 0
            rc = lib.dspark_probe_read_ex(pool.data_ptr() + off, nbytes, sink.data_ptr(), grid,
                                          unroll, nt, blocked, stream)
            if rc != 0:
                raise RuntimeError(f"dspark_probe_read_ex failed: {rc}")
        for i in range(slots):
            launch(i)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(launches):
            launch(i)
        ev1.record()
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / launches
        return {"us_per_launch": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
                "loads_in_flight": unroll, "nontemporal": bool(nt), "blocked": bool(blocked),
                "grid": grid}

    sweep = [timed("rotating", u, nt, bl, g) for u in (4, 8, 16) for nt in (0, 1)
             for bl in (0, 1) for g in grids]
    best = max(sweep, key=lambda e: e["GBps"])
    plain = next(e for e in sweep if (e["loads_in_flight"], e["nontemporal"], e["blocked"],
                                      e["grid"]) == (4, False, False, 2048))
    resident = timed("resident", best["loads_in_flight"], int(best["nontemporal"]),
                     int(best["blocked"]), best["grid"])
    del pool
    return {"bytes": nbytes, "rotating": best, "plain_4_in_flight": plain, "resident": resident,
            "variants_swept": len(sweep),
            "top5": [[e["loads_in_flight"], int(e["nontemporal"]), int(e["blocked"]), e["grid"],
                      e["GBps"]] for e in sorted(sweep, key=lambda e: -e["GBps"])[:5]]}


def one_step_block(di, k):
    """Inputs and buffers of a one-step draft block on position k's U and h
    rows: its STEPS phase is exactly one launch of the draft-step kernel."""
    import dataclasses
    from semi_autoregressive_drafting_amd import runner
    di1 = dataclasses.replace(di, gamma=1, U=di.U[:, k - 1:k].contiguous(),
                              h=di.h[:, k - 1:k].contiguous(), target=None)
    return di1, runner.RoundBuffers.allocate(di1)


def _probe_lib():
    import ctypes
    from semi_autoregressive_drafting_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.dspark_probe_read_ex.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    lib.dspark_probe_read_ex.restype = ctypes.c_int
    return lib


def cold_single_steps(di, n, flush_bytes=1 << 30, modes=("cold", "hot")):
    """One draft-step launch at a time (a one-step block, events around its
    STEPS phase only).  'cold': right after a cached read over flush_bytes
    (four times the MALL), which leaves neither W2, U nor W1 in L2 or the
    MALL (a read leaves no dirty lines behind to be written back during the
    step).  'hot': the same launch right after an identical untimed one, so
    that everything it reads is cached.  Nothing synchronises the host between
    the flush (or the untimed launch) and the timed launch, so the GPU is busy
    up to it.  Microseconds per launch."""
    import torch
    from semi_autoregressive_drafting_amd import dspark as D
    from semi_autoregressive_drafting_amd import runner
    di1, b1 = one_step_block(di, 1)
    lib = _probe_lib()
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    scratch.fill_(3)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def launch(seed):
        b1.x[:, 0].copy_(di1.anchor)
        runner.draft_phases(di1, b1, TEMPERATURE, seed, D.DSPARK_PHASE_STEPS, copy_anchor=False)

    out = {m: [] for m in modes}
    for s in range(n + 2):
        for mode in modes:
            if mode == "cold":
                if lib.dspark_probe_read_ex(scratch.data_ptr(), flush_bytes, sink.data_ptr(),
                                            4096, 16, 0, 0, stream) != 0:
                    raise RuntimeError("flush read failed")
            else:
                launch(800 + s)
                runner.draft_phases(di1, b1, TEMPERATURE, 800 + s, D.DSPARK_PHASE_MERGE)
            b1.x[:, 0].copy_(di1.anchor)
            e0.record()
            runner.draft_phases(di1, b1, TEMPERATURE, 800 + s, D.DSPARK_PHASE_STEPS,
                                copy_anchor=False)
            e1.record()
            runner.draft_phases(di1, b1, TEMPERATURE, 800 + s, D.DSPARK_PHASE_MERGE)
            torch.cuda.synchronize()
            if s >= 2:
                out[mode].append(e0.elapsed_time(e1) * 1e3)
    del scratch, b1, di1
    return out


def other_workloads(nb=10):
    """The draft block at the other workload shapes (tokens/s, microseconds
    per step, HBM fraction of the step), and the whole round with
    verification at the 4B-shaped round workload (realised tau)."""
    import torch
    from semi_autoregressive_drafting_amd import dspark as D
    from semi_autoregressive_drafting_amd import runner, synth
    res = {}
    for name, temps in (("qwen3_4b_r32_g7", (1.0,)), ("qwen3_14b_r512_g7", (0.0, 1.0)),
                        ("round_4b_r128_g7", (1.0,))):
        wl = synth.WORKLOADS[name]
        inp = synth.generate(name, seed=0, target=wl.target)
        di = runner.DeviceInputs.upload(inp)
        buf = runner.RoundBuffers.allocate(di)
        del inp
        R, g, V, rank, d = di.R, di.gamma, di.V, di.rank, di.d
        sb = draft_step_bytes(R, V, rank, d)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for T in temps:
            for s in range(3):
                runner.draft(di, buf, T, 1000 + s)
            steps_us, block_us = [], []
            for s in range(nb):
                buf.x[:, 0].copy_(di.anchor)
                ev[0].record()
                runner.draft_phases(di, buf, T, 1100 + s, D.DSPARK_PHASE_STEPS, copy_anchor=False)
                ev[1].record()
                runner.draft_phases(di, buf, T, 1100 + s, D.DSPARK_PHASE_MERGE)
                ev[2].record()
                torch.cuda.synchronize()
                steps_us.append(ev[0].elapsed_time(ev[1]) * 1e3)
                block_us.append(ev[0].elapsed_time(ev[2]) * 1e3)
            st = float(np.median(steps_us)) / g
            bl = float(np.median(block_us))
            e = {"R": R, "gamma": g, "d": d, "temperature": T,
                 "draft_tokens_per_s": round(R * g / (bl * 1e-6), 1),
                 "block_us": round(bl, 2), "us_per_step": round(st, 2),
                 "step_bytes": sb, "step_GBps": round(sb / st / 1e3, 1),
                 "frac": round(sb / st / 1e3 / HBM_PEAK_GBS, 4)}
            if wl.target:
                r_us, taus = [], []
                for s in range(nb + 2):
                    ev[0].record()
                    runner.draft(di, buf, T, 1200 + s)
                    runner.schedule(di, buf)
                    ev[1].record()
                    runner.verify(di, buf, T, 1200 + s)
                    ev[2].record()
                    torch.cuda.synchronize()
                    if s >= 2:
                        r_us.append((ev[0].elapsed_time(ev[2]) * 1e3, ev[1].elapsed_time(ev[2]) * 1e3))
                        taus.append(float(buf.tau_mean.item()))
                rr = float(np.median([u[0] for u in r_us]))
                vv = float(np.median([u[1] for u in r_us]))
                vb = verify_bytes(R, V, rank, g)
                e.update({"round_us": round(rr, 2),
                          "round_draft_tokens_per_s": round(R * g / (rr * 1e-6), 1),
                          "verify_us": round(vv, 2),
                          "verify_frac": round(vb / vv / 1e3 / HBM_PEAK_GBS, 4),
                          "tau_mean": round(float(np.mean(taus)), 4),
                          "budget_last_round": int(buf.budget.item())})
            res[f"{name}_T{T:g}"] = e
        del di, buf
        torch.cuda.empty_cache()
    return res


def cpu_baseline(inp, seed):
    """The CPU oracle, as it stands, on the same workload: all R requests
    (half easy, half hard) through the whole round (gamma draft steps with
    confidence and survival, schedule, verify), on one BLAS thread and on all
    host cores."""
    from threadpoolctl import threadpool_limits
    from oracle import dspark_oracle as O

    wl = inp.wl
    reqs = np.arange(wl.R)
    W1, W2t = O.as_f64(inp.W1_store), O.as_f64(inp.W2t_store)
    h = O.as_f64(inp.h_store[reqs])
    U = inp.U[reqs].astype(np.float64)
    def run(threads):
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            rnd = O.draft_round(U, h, inp.w, W1, W2t, inp.anchor[reqs], TEMPERATURE, seed, reqs)
            ell, b, th, _, _ = O.schedule(rnd["a"], inp.sps[: len(reqs) * (1 + wl.gamma) + 1])
            O.verify(inp.U[reqs], inp.target[reqs], W1, W2t, rnd["x"], ell, TEMPERATURE, seed,
                     reqs)
            return time.perf_counter() - t0

    host_cores = len(os.sched_getaffinity(0))
    dt1 = run(1)
    dtn = run(host_cores)
    tokens = len(reqs) * wl.gamma
    return {"value": tokens / dt1, "unit": "draft tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"all {wl.R} requests ({wl.R // 2} easy, {wl.R // 2} hard), one full "
                      f"round (gamma={wl.gamma} draft steps + schedule + verify), fp64 NumPy, "
                      f"1 BLAS thread, {dt1:.1f} s",
            "host_cores": host_cores,
            "all_cores": {"value": tokens / dtn, "blas_threads": host_cores,
                          "seconds": round(dtn, 2)}}


def cpu_oracle_next_rows(inp, x_star_row, seed):
    """The oracle, as it stands, on small samples of the rows beyond the round
    (one BLAS thread): the RNN head's block, the training losses and their
    gradients.  Rates are per request-position of the sample."""
    from threadpoolctl import threadpool_limits
    from oracle import dspark_oracle as O
    from semi_autoregressive_drafting_amd import synth

    wl = inp.wl
    W1, W2t = O.as_f64(inp.W1_store), O.as_f64(inp.W2t_store)
    gru = synth.gru_weights(wl, 0)
    g64 = (O.as_f64(gru[0]), O.as_f64(gru[1]), gru[2].astype(np.float64), gru[3].astype(np.float64))
    out = {}
    with threadpool_limits(limits=1):
        reqs = np.arange(16)
        t0 = time.perf_counter()
        O.rnn_draft_round(inp.U[reqs], O.as_f64(inp.h_store[reqs]), inp.w, W1, W2t, g64,
                          inp.anchor[reqs], TEMPERATURE, seed, reqs)
        dt = time.perf_counter() - t0
        out["rnn_head_block"] = {"value": len(reqs) * wl.gamma / dt, "unit": "draft tokens/s",
                                 "sample": f"{len(reqs)} requests, gamma={wl.gamma}", "seconds": round(dt, 2)}
        reqs = np.arange(8)
        xs = np.repeat(x_star_row[None], len(reqs), axis=0)
        t0 = time.perf_counter()
        O.train_losses(inp.U[reqs], inp.target[reqs], W1, W2t, inp.h_store[reqs], inp.w, xs)
        dt = time.perf_counter() - t0
        out["train_loss_forward"] = {"value": len(reqs) * wl.gamma / dt, "unit": "positions/s",
                                     "sample": f"{len(reqs)} requests", "seconds": round(dt, 2)}
        reqs = np.arange(4)
        t0 = time.perf_counter()
        O.train_loss_grads(inp.U[reqs], inp.target[reqs], W1, W2t, inp.h_store[reqs], inp.w, xs[:4])
        dt = time.perf_counter() - t0
        out["train_loss_with_gradients"] = {"value": len(reqs) * wl.gamma / dt, "unit": "positions/s",
                                            "sample": f"{len(reqs)} requests", "seconds": round(dt, 2)}
    out["cores"] = 1
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the read ceiling, cold steps, asynchronous scheduler and graph "
                         "replay (for counter-collection runs)")
    ap.add_argument("--train-only", action="store_true",
                    help="only run the training losses with every gradient (K times, the "
                         "drafted block standing in for x*), for counter collection")
    ap.add_argument("--cold-only", action="store_true",
                    help="only run single draft-step launches, each after a cache flush (so "
                         "that a kernel trace shows the cold kernel alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (x4), so that "
                         "FETCH_SIZE / WRITE_SIZE counters can be scaled to bytes")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel() * 4, "launches": 4}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from semi_autoregressive_drafting_amd import dspark as D
    from semi_autoregressive_drafting_amd import runner, synth

    t_gen = time.perf_counter()
    inp = synth.generate(WORKLOAD, seed=0, target=True)
    di = runner.DeviceInputs.upload(inp)
    buf = runner.RoundBuffers.allocate(di)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    R, g, V, rank, d = di.R, di.gamma, di.V, di.rank, di.d
    di_wl = inp.wl
    if args.train_only:
        runner.draft(di, buf, TEMPERATURE, 1)
        x_star = buf.x.clone()
        gws = torch.empty(D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_GRAD, R, V, rank, g),
                          dtype=torch.uint8, device="cuda")
        for _ in range(args.steps):
            gout = runner.train_loss_grad(di, x_star, ws=gws)
            del gout
        torch.cuda.synchronize()
        print(json.dumps({"workload": WORKLOAD, "train_loss_grad_calls": args.steps}), flush=True)
        return
    if args.cold_only:
        single = cold_single_steps(di, args.steps, modes=("cold",))
        sb = draft_step_bytes(R, V, rank, d)
        cm = float(np.median(single["cold"]))
        print(json.dumps({"workload": WORKLOAD, "launches": args.steps + 2, "bytes_per_launch": sb,
                          "cold_us_median_events": round(cm, 2)}), flush=True)
        return

    def one_round(seed, ev=None):
        # the anchor copy and the gamma streaming steps, then the record merge;
        # the events bracket the gamma step launches only
        buf.x[:, 0].copy_(di.anchor)
        if ev is not None:
            ev[0].record()
        runner.draft_phases(di, buf, TEMPERATURE, seed, D.DSPARK_PHASE_STEPS, copy_anchor=False)
        if ev is not None:
            ev[1].record()
        runner.draft_phases(di, buf, TEMPERATURE, seed, D.DSPARK_PHASE_MERGE)
        runner.schedule(di, buf)
        runner.verify(di, buf, TEMPERATURE, seed)

    # warm-up rounds (the first rounds after start-up run at lower clocks)
    for w in range(args.warmup):
        one_round(10_000 + w)
    torch.cuda.synchronize()

    # Timed region: K whole rounds; the two events per round bracket the gamma
    # back-to-back draft-step launches.
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        one_round(s, evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    draft_ms = np.array([evs[s][0].elapsed_time(evs[s][1]) for s in range(K)])
    step_ms = draft_ms / g   # per draft-step launch, gaps between the launches included
    ms_round = wall / K * 1e3
    value = R * g / (wall / K)

    # Phase breakdown from separate rounds (events between the phases).
    nb = 5
    ph = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nb)]
    for s in range(nb):
        ph[s][0].record()
        runner.draft(di, buf, TEMPERATURE, 500 + s)
        ph[s][1].record()
        runner.schedule(di, buf)
        ph[s][2].record()
        runner.verify(di, buf, TEMPERATURE, 500 + s)
        ph[s][3].record()
    torch.cuda.synchronize()
    block_ms = np.array([ph[s][0].elapsed_time(ph[s][1]) for s in range(nb)])
    sched_ms = np.array([ph[s][1].elapsed_time(ph[s][2]) for s in range(nb)])
    ver_ms = np.array([ph[s][2].elapsed_time(ph[s][3]) for s in range(nb)])
    extras = not args.no_extras
    # the asynchronous scheduler on the same candidates (budget from a copy
    # standing in for the survival of two steps earlier)
    async_us = [float("nan")]
    if extras:
        a_lag = buf.a.clone()
        ea = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        async_us = []
        for s in range(nb):
            ea[0].record()
            runner.schedule_async(di, buf, a_lag)
            ea[1].record()
            torch.cuda.synchronize()
            async_us.append(ea[0].elapsed_time(ea[1]) * 1e3)

    # The forward training losses on the same block, the drafted tokens
    # standing in for the target block x* (anchor in column 0).
    train, train_grad = None, None
    x_star_host = None
    if extras:
        x_star = buf.x.clone()
        x_star_host = x_star[0].cpu().numpy().astype(np.int64)
        tws = torch.empty(D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_LOSS, R, V, rank, g),
                          dtype=torch.uint8, device="cuda")
        for _ in range(2):
            runner.train_loss(di, x_star, ws=tws)
        et = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t_us = []
        for s in range(nb):
            et[0].record()
            _, tsums = runner.train_loss(di, x_star, ws=tws)
            et[1].record()
            torch.cuda.synchronize()
            t_us.append(et[0].elapsed_time(et[1]) * 1e3)
        tb = train_loss_bytes(R, V, rank, d, g)
        t_med = float(np.median(t_us))
        train = {"us": round(t_med, 2), "bytes": tb, "achieved_GBps": round(tb / (t_med * 1e-6) / 1e9, 1),
                 "frac_of_hbm_peak": round(tb / (t_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 "positions_per_s": round(R * g / (t_med * 1e-6), 1),
                 "weighted_sums": [round(float(v), 6) for v in tsums.cpu().tolist()]}
        del tws
        # losses and every gradient
        gws = torch.empty(D.dspark_workspace_bytes(D.DSPARK_OP_TRAIN_GRAD, R, V, rank, g),
                          dtype=torch.uint8, device="cuda")
        for _ in range(2):
            gout = runner.train_loss_grad(di, x_star, ws=gws)
        del gout
        g_us = []
        for s in range(nb):
            et[0].record()
            gout = runner.train_loss_grad(di, x_star, ws=gws)
            et[1].record()
            torch.cuda.synchronize()
            g_us.append(et[0].elapsed_time(et[1]) * 1e3)
            del gout
        gb = train_grad_bytes(R, V, rank, d, g)
        g_med = float(np.median(g_us))
        train_grad = {"us": round(g_med, 2), "bytes": gb,
                      "achieved_GBps": round(gb / (g_med * 1e-6) / 1e9, 1),
                      "frac_of_hbm_peak": round(gb / (g_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "positions_per_s": round(R * g / (g_med * 1e-6), 1)}
        del gws

    # The RNN head's draft block on the same inputs (GRU weights from the
    # generator's RNN stream): input projection, then per step the state
    # update and the draft step, then the merge.
    rnn = None
    if extras:
        gru = synth.gru_weights(di_wl, 0)
        rw = runner.RnnWeights.upload(gru)
        rstate = torch.empty((R, rank), dtype=torch.float32, device="cuda")
        rws = torch.zeros(D.dspark_workspace_bytes(D.DSPARK_OP_DRAFT_RNN, R, V, rank, g),
                          dtype=torch.uint8, device="cuda")
        for s in range(3):
            runner.draft_rnn(di, buf, rw, TEMPERATURE, 600 + s, rstate, rws)
        # back-to-back blocks with an event between each, as for the Markov
        # block (draft_block_with_copy_and_merge), so that neither figure
        # carries the launch latency of an idle queue
        erb = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
        erb[0].record()
        for s in range(nb):
            runner.draft_rnn(di, buf, rw, TEMPERATURE, 610 + s, rstate, rws)
            erb[s + 1].record()
        torch.cuda.synchronize()
        r_us = [erb[s].elapsed_time(erb[s + 1]) * 1e3 for s in range(nb)]
        r_med = float(np.median(r_us))
        er = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        # the RNN head's whole round: its block (bias rows written out),
        # schedule, and verification with those rows
        rrows = torch.empty((R, g, rank), dtype=torch.int16, device="cuda")
        rr_us = []
        for s in range(nb + 2):
            er[0].record()
            runner.draft_rnn(di, buf, rw, TEMPERATURE, 620 + s, rstate, rws, rrows)
            runner.schedule(di, buf)
            runner.verify_rnn(di, buf, rrows, TEMPERATURE, 620 + s)
            er[1].record()
            torch.cuda.synchronize()
            if s >= 2:
                rr_us.append(er[0].elapsed_time(er[1]) * 1e3)
        rr_med = float(np.median(rr_us))
        rnn = {"block_us": round(r_med, 2), "us_per_step": round(r_med / g, 2),
               "vs_markov_block": round(r_med / float(block_ms.mean() * 1e3), 3),
               "draft_tokens_per_s": round(R * g / (r_med * 1e-6), 1),
               "round_us": round(rr_med, 2),
               "round_draft_tokens_per_s": round(R * g / (rr_med * 1e-6), 1)}
        del rws, rstate, rrows

    # One draft-step launch alone, after a flush of L2 and the MALL (cold)
    # and with its inputs cached (hot).
    single = cold_single_steps(di, 8) if extras else None

    sb = draft_step_bytes(R, V, rank, d)
    ceiling = read_ceiling(sb) if extras else None
    others = other_workloads() if extras else None

    # The same round replayed from one captured HIP graph (no host launches).
    graph = None
    try:
        if not extras:
            raise RuntimeError("skipped (--no-extras)")
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_round(900)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            one_round(901)
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(K):
            gr.replay()
        torch.cuda.synchronize()
        g_round = (time.perf_counter() - tg) / K
        del gr
        # the gamma-step loop alone, captured once and replayed back to back
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            runner.draft_phases(di, buf, TEMPERATURE, 902, D.DSPARK_PHASE_STEPS)
        for _ in range(3):
            gs.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            gs.replay()
        e1.record()
        torch.cuda.synchronize()
        g_steps_us = e0.elapsed_time(e1) * 1e3 / K
        runner.draft_phases(di, buf, TEMPERATURE, 902, D.DSPARK_PHASE_MERGE)  # leave ws clean
        torch.cuda.synchronize()
        del gs
        graph = {"round_us": round(g_round * 1e6, 2),
                 "draft_tokens_per_s": round(R * g / g_round, 1),
                 "step_loop_us_per_step": round(g_steps_us / g, 2)}
    except Exception as exc:  # graph capture unavailable: report it, keep the eager numbers
        graph = {"error": str(exc)[:200]}

    step_s = float(step_ms.mean()) * 1e-3
    achieved = sb / step_s / 1e9
    cold_kernel_us = profiled_cold_us()
    vb = verify_bytes(R, V, rank, g)
    out = {
        "metric": "Markov-head draft tokens/s at R=128,γ=16,V=152k; % of HBM roofline",
        "value": round(value, 1),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_round, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: R={R}, gamma={g}, V={V}, rank={rank}, d={d}, "
                               "bf16 W1/W2/h, fp32 logits, T=1, verify target U+N(0,1)",
                   "R": R, "gamma": g, "V": V, "rank": rank, "d": d,
                   "temperature": TEMPERATURE},
        "roofline": {"kernel": "markov_step_shared (one draft step; HIP events around the gamma "
                               "back-to-back launches of a draft block, divided by gamma)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "bytes_per_launch": sb,
                     "avg_launch_us": round(step_s * 1e6, 2),
                     "frac_of_read_ceiling": (round(achieved / ceiling["rotating"]["GBps"], 4)
                                              if ceiling else None),
                     # cold: every byte from HBM (L2 and MALL flushed before the launch);
                     # kernel-only from the committed kernel trace, and from HIP events
                     # around one launch (launch latency included) measured here
                     "frac_cold": (round(sb / cold_kernel_us / 1e3 / HBM_PEAK_GBS, 4)
                                   if cold_kernel_us else None),
                     "cold_kernel_us": cold_kernel_us,
                     "frac_cold_events": (round(sb / float(np.median(single["cold"])) / 1e3
                                                / HBM_PEAK_GBS, 4) if single else None),
                     "cold_launch_us_events": (round(float(np.median(single["cold"])), 2)
                                               if single else None)},
        "read_ceiling": ceiling,
        "single_step": ({"cold_us_median": round(float(np.median(single["cold"])), 2),
                         "hot_us_median": round(float(np.median(single["hot"])), 2),
                         "cold_us": [round(v, 2) for v in single["cold"]],
                         "note": "one launch per event pair (launch latency included); a "
                                 "cached 1 GiB read before each cold launch flushes L2 and "
                                 "the MALL"}
                        if single else None),
        "other_workloads": others,
        "graph": graph,
        "breakdown_us": {"draft_step_mean": round(float(step_ms.mean()) * 1e3, 2),
                         "draft_step_median": round(float(np.median(step_ms)) * 1e3, 2),
                         "draft_step_min": round(float(step_ms.min()) * 1e3, 2),
                         "draft_steps_total": round(float(draft_ms.mean()) * 1e3, 2),
                         "draft_block_with_copy_and_merge": round(float(block_ms.mean()) * 1e3, 2),
                         "schedule": round(float(sched_ms.mean()) * 1e3, 2),
                         "schedule_async": round(float(np.median(async_us)), 2),
                         "verify": round(float(ver_ms.mean()) * 1e3, 2),
                         "round_wall": round(ms_round * 1e3, 2)},
        "rnn_head_block": rnn,
        "train_loss_forward": train,
        "train_loss_with_gradients": train_grad,
        "verify_roofline": {"bytes": vb, "achieved_GBps": round(vb / (ver_ms.mean() * 1e-3) / 1e9, 1)},
        "draft_only_tokens_per_s": round(R * g / (block_ms.mean() * 1e-3), 1),
        "budget_last_round": int(buf.budget.item()),
        "tau_mean_last_round": round(float(buf.tau_mean.item()), 4),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and os.environ.get("RANK", "0") == "0":
        print("# timing the CPU oracle on a bounded sample ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, 0)
        if extras:
            out["cpu_oracle_next_rows"] = cpu_oracle_next_rows(inp, x_star_host, 0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

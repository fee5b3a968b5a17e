"""Throughput of the LaCT layer (ShortConv2D + update + apply) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c5a]

One step is one pass of the whole layer over the workload's synthetic tokens,
already resident in HBM: V' = ShortConv2D(V) (if the workload has it), the
update with the workload's inner steps, and apply over every query row.
Prints one JSON line.  ``value`` is update tokens per second.  The ``roofline``
entry covers the gradient kernel, timed with HIP events on its own stream
inside the timed region.  ``cpu_baseline`` times the CPU oracle (fp32 NumPy)
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c5a")
    ap.add_argument("--frames", type=int, default=0, help="override the workload's frame count")
    ap.add_argument("--cpu-sample-frames", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-only", action="store_true",
                    help="only time the CPU oracle on the workload (no GPU use); prints one JSON line")
    ap.add_argument("--oracle-threads", type=int, default=0,
                    help="limit the oracle's BLAS threads (0 = the library default, all cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter scaling)")
    ap.add_argument("--no-profile-events", action="store_true")
    ap.add_argument("--host-stream", type=int, default=0, metavar="BATCH",
                    help="time the out-of-core update instead: K, V, eta in pinned host memory, streamed "
                         "in batches of BATCH tokens (PCIe-inclusive; not the headline)")
    ap.add_argument("--sweep", action="store_true",
                    help="time ZipMap-shaped layers at 125..2000 frames and fit t = t0 + beta*N")
    return ap.parse_args()


def _code_only(text):
    """C++ source with comments removed and whitespace collapsed (string literals in
    these files hold no comment markers), so that editing a comment keeps the digest."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def grad_source_digest():
    """sha256 over the code the gradient kernel is compiled from: grad.hip, common.h and
    the part of kernels.h up to the end of GradParams (tile constants and the
    parameter block); declarations after it belong to other kernels."""
    import hashlib
    csrc = os.path.join(ROOT, "test_weight_layers_amd", "csrc")
    h = hashlib.sha256()
    for f in ("grad.hip", "common.h"):
        with open(os.path.join(csrc, f)) as fh:
            h.update(_code_only(fh.read()).encode())
    with open(os.path.join(csrc, "kernels.h")) as fh:
        text = fh.read()
    start = text.index("struct GradParams")
    h.update(_code_only(text[:text.index("};", start) + 2]).encode())
    return h.hexdigest()


def measured_mfma_peak(iters: int = 65536, reps: int = 5) -> float:
    """Dense bf16 MFMA rate (TFLOP/s) of the library's register-only probe kernel, timed
    with events on the current stream after two warm-up launches (median of `reps`).
    65,536 rounds make a launch of about 7 ms: shorter launches read low while the clock
    ramps up (about 2.07 PFLOP/s at 0.5 ms, 2.29 at 2 ms, 2.41 from 7 ms on, the same
    over a second of back-to-back launches)."""
    import numpy as np
    import torch
    from test_weight_layers_amd import ttt
    for _ in range(2):
        ttt.mfma_rate_probe(iters)
    torch.cuda.synchronize()
    rates = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        f = ttt.mfma_rate_probe(iters)
        e1.record()
        e1.synchronize()
        rates.append(f / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return float(np.median(rates))


def measured_traffic(d):
    """HBM bytes per launch of the gradient kernel from the committed rocprofv3 counter summary,
    or None when the kernel's source changed since the counters were taken (or d differs)."""
    path = os.path.join(ROOT, "profiles", "lact_c5a_hbm_traffic.md")
    if d != 256 or not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("traffic_bytes_per_launch grad_fast_kernel<256"):
            rec["bytes"] = float(line.split(":")[1])
        elif line.startswith("gradient_kernel_source_sha256:"):
            rec["sha"] = line.split(":")[1].strip()
    if rec.get("sha") != grad_source_digest():
        return None
    return rec.get("bytes")


def flops(cfg, n, nq):
    """Algorithmic FLOPs: update 12*N*d*m*H per inner step, apply 6*Nq*d*m*H."""
    H, d, m = cfg.heads, cfg.d, cfg.m
    grad = 12.0 * n * d * m * H
    apply = 6.0 * nq * d * m * H
    r, c = min(d, m), max(d, m)
    ns = 5 * (4.0 * r * r * c + 2.0 * r ** 3) * 3 * H
    conv = 18.0 * n * H * d if cfg.conv else 0.0
    return grad, apply, ns, conv


def gate_flops(cfg, nq):
    """Gated output: the C x C gate product per apply row (RMSNorm/SiLU not counted)."""
    return 2.0 * nq * (cfg.heads * cfg.d) ** 2 if cfg.gate else 0.0


def per_call_stats(marks):
    """Median and p90 over the timed steps of each API call's HIP-event time (and of
    the whole step, from its first to its last mark)."""
    import numpy as np
    calls, steps = {}, []
    first = None
    for (tag, e), nxt in zip(marks, marks[1:] + [None]):
        if tag == "start":
            first = e
        if nxt is not None and nxt[0] != "start":
            calls.setdefault(nxt[0], []).append(e.elapsed_time(nxt[1]))
        if nxt is None or nxt[0] == "start":
            steps.append(first.elapsed_time(e))
    calls["step"] = steps
    return {k: {"median": float(np.median(v)), "p90": float(np.percentile(v, 90)), "n": len(v)}
            for k, v in calls.items()}


def copy_calibration():
    import torch
    n = 1 << 30   # 1 GiB
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def cpu_baseline(cfg, frames, threads=0):
    """Time the fp32 NumPy oracle on `frames` frames of the same workload (BLAS limited
    to `threads` threads when > 0)."""
    import contextlib
    from threadpoolctl import threadpool_limits

    import oracle
    from test_weight_layers_amd import synth
    n = frames * cfg.tokens_per_frame
    inp = synth.make_inputs(cfg, n=n, nq_extra=0)
    f32 = lambda t: t.detach().float().numpy()
    args = [f32(inp.w1), f32(inp.w3), f32(inp.w2), f32(inp.k), f32(inp.v), f32(inp.eta), f32(inp.q)]
    conv = None
    if cfg.conv:
        conv = dict(wconv=f32(inp.wconv), frames=frames, tokens_per_frame=cfg.tokens_per_frame,
                    n_special=cfg.n_special, grid_h=cfg.grid_h, grid_w=cfg.grid_w)
    limit = threadpool_limits(limits=threads) if threads > 0 else contextlib.nullcontext()
    with limit:
        dt, threads_used = _time_oracle(oracle, synth, cfg, args, conv, f32, inp)
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads_used), "kind": "oracle",
            "sample": f"{frames} frames x {cfg.tokens_per_frame} tokens = {n} tokens of {cfg.name}, "
                      f"fp32 NumPy oracle, full layer (conv={cfg.conv}, steps={cfg.steps}, apply"
                      f"{', streamed in chunks' if cfg.chunk_frames else ''}"
                      f"{', norm-preserving step' if cfg.norm_preserve else ''}"
                      f"{', gated output' if cfg.gate else ''}), "
                      f"{dt:.2f} s wall"}


def _time_oracle(oracle, synth, cfg, args, conv, f32, inp):
    from threadpoolctl import threadpool_info
    t0 = time.perf_counter()
    if cfg.chunk_frames:
        oracle.stream(*args, cfg.lr, cfg.steps, chunk=cfg.chunk_frames * cfg.tokens_per_frame,
                      norm_preserve=cfg.norm_preserve)
    else:
        if conv is not None:
            args[4] = oracle.shortconv2d(args[4], **conv)
        w_hat, _, _ = oracle.update(*args[:6], cfg.lr, cfg.steps, norm_preserve=cfg.norm_preserve)
        o = oracle.apply(*w_hat, args[6])
        if cfg.gate:
            wg, gamma = synth.gate_weights(cfg.seed, cfg.heads * cfg.d, inp.k.dtype)
            oracle.output_gate(o, f32(wg), f32(gamma), cfg.gate_eps)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return dt, threads


def timed_median(fn, reps, warmup, min_warm_s=0.2):
    """Median seconds of `reps` calls of fn, each bracketed by HIP events on the current
    stream, after at least `warmup` calls and `min_warm_s` seconds of warm-up."""
    import numpy as np
    import torch
    t_end = time.perf_counter() + min_warm_s
    i = 0
    while i < warmup or time.perf_counter() < t_end:
        fn()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3


def linear_sweep(steps, warmup):
    """Update (1 step) + apply on the same N tokens of the ZipMap 4x256/512 shape at
    125..2000 frames (prefixes of one draw); least-squares fit of time against N.
    Beside it, the apply of one fixed batch of queries (32 frames) with the weights
    each N produced: a query's cost does not depend on how many tokens were absorbed
    (ZipMap 关键设计 4, querying the fast weights as a scene state)."""
    import numpy as np
    import torch
    from dataclasses import replace
    from test_weight_layers_amd import synth, ttt
    from test_weight_layers_amd.configs import CONFIGS
    frames = [125, 250, 500, 750, 1000, 2000]
    cfg = replace(CONFIGS["c4"], frames=max(frames), extra_query=0, steps=1)
    torch.cuda.set_device(0)
    ttt.load()
    full = synth.to_device(synth.make_inputs(cfg), "cuda")
    H, d, m = cfg.heads, cfg.d, cfg.m
    w0 = (full.w1, full.w3, full.w2)
    nfix = 32 * cfg.tokens_per_frame
    q_fix = full.q[:nfix]
    o_fix = torch.empty((nfix, H * d), dtype=q_fix.dtype, device="cuda")
    ws_f = torch.empty(ttt.apply_workspace_bytes(H, d, m, nfix, q_fix.dtype), dtype=torch.uint8, device="cuda")
    # Every size gets its own buffers; the sizes are then timed round-robin for several
    # passes, so that the GPU's clock (which falls under long sustained load) is the same
    # on average for every size, and each size keeps the median over its passes.
    setups = []
    for f in frames:
        n = f * cfg.tokens_per_frame
        k, v, q, eta = full.k[:n], full.v[:n], full.q[:n], full.eta[:, :n]
        w_out = tuple(torch.empty_like(x) for x in w0)
        o = torch.empty((n, H * d), dtype=k.dtype, device="cuda")
        ws_u = torch.empty(ttt.update_workspace_bytes(H, d, m, n, k.dtype), dtype=torch.uint8, device="cuda")
        ws_a = torch.empty(ttt.apply_workspace_bytes(H, d, m, n, k.dtype), dtype=torch.uint8, device="cuda")

        def step(k=k, v=v, q=q, eta=eta, w_out=w_out, o=o, ws_u=ws_u, ws_a=ws_a):
            ttt.update(w0, k, v, eta, cfg.lr, 1, out=w_out, workspace=ws_u)
            ttt.apply(w_out, q, out=o, workspace=ws_a)

        def fixed_q(w_out=w_out):
            ttt.apply(w_out, q_fix, out=o_fix, workspace=ws_f)

        setups.append((f, n, step, fixed_q))
    passes = 5
    times = {f: [] for f in frames}
    fixed_times = {f: [] for f in frames}
    for _ in range(passes):
        for f, n, step, fixed_q in setups:
            # each timing: median of `steps` event-timed calls after >= 200 ms of warm-up
            times[f].append(timed_median(step, steps, warmup))
            fixed_times[f].append(timed_median(fixed_q, steps, warmup))
    rows = [(n, float(np.median(times[f]))) for f, n, _, _ in setups]
    fixed = [float(np.median(fixed_times[f])) for f in frames]
    for (f, n, _, _), (_, t), fx in zip(setups, rows, fixed):
        print(json.dumps({"sweep_frames": f, "tokens": n, "ms": t * 1e3, "apply_fixed_ms": fx * 1e3,
                          "ms_per_pass": [x * 1e3 for x in times[f]]}), flush=True)
    ns = np.array([r[0] for r in rows], float)
    ts = np.array([r[1] for r in rows], float)
    A = np.stack([np.ones_like(ns), ns], 1)
    # The acceptance test is on relative residuals, so the fit minimises them: least
    # squares on the rows scaled by 1 / t.  The unweighted fit, which lets the largest
    # sizes dominate, is reported beside it.
    (t0, beta), *_ = np.linalg.lstsq(A / ts[:, None], np.ones_like(ts), rcond=None)
    fit = t0 + beta * ns
    r2 = 1.0 - np.sum((ts - fit) ** 2) / np.sum((ts - ts.mean()) ** 2)
    (t0_u, beta_u), *_ = np.linalg.lstsq(A, ts, rcond=None)
    fit_u = t0_u + beta_u * ns
    i1000 = frames.index(1000)
    out = {"sweep": "zipmap-shape 4x256/512, update (1 step) + apply on the same N tokens; per size the "
                    f"median over {passes} round-robin passes of the median of {steps} event-timed calls "
                    "after >= 200 ms of warm-up",
           "frames": frames, "tokens": ns.tolist(), "seconds": ts.tolist(), "t0_s": t0,
           "fit": "least squares on relative residuals (rows scaled by 1/t)",
           "beta_s_per_token": beta, "r2": r2, "max_rel_residual": float(np.max(np.abs(ts - fit) / ts)),
           "rel_residuals": ((ts - fit) / ts).tolist(),
           "unweighted_fit": {"t0_s": t0_u, "beta_s_per_token": beta_u,
                              "max_rel_residual": float(np.max(np.abs(ts - fit_u) / ts))},
           "t0_over_t_at_1000_frames": float(t0 / ts[i1000]),
           "tokens_per_s_asymptotic": 1.0 / beta,
           "apply_fixed_queries": nfix, "apply_fixed_seconds": fixed,
           "apply_fixed_spread": float(max(fixed) / min(fixed) - 1.0)}
    print(json.dumps(out), flush=True)


def host_stream(cfg, batch, steps, warmup):
    """Out-of-core update of the workload's tokens from pinned host memory (VGG-T3 关键发现 2)."""
    import torch
    from test_weight_layers_amd import synth, ttt
    torch.cuda.set_device(0)
    ttt.load()
    inp = synth.make_inputs(cfg, nq_extra=0)
    H, d, m = cfg.heads, cfg.d, cfg.m
    n = inp.k.shape[0]
    kh, vh, eh = inp.k.pin_memory(), inp.v.pin_memory(), inp.eta.contiguous().pin_memory()
    w0 = tuple(t.cuda() for t in (inp.w1, inp.w3, inp.w2))
    w_out = tuple(torch.empty_like(x) for x in w0)
    ws = torch.empty(ttt.update_host_workspace_bytes(H, d, m, batch, kh.stride(0), kh.dtype), dtype=torch.uint8,
                     device="cuda")

    def step():
        ttt.update_host(w0, kh, vh, eh, cfg.lr, cfg.steps, batch=batch, out=w_out, workspace=ws,
                        norm_preserve=cfg.norm_preserve)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ttt.profile_reset()
    ttt.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ttt.profile_enable(False)
    kt = ttt.profile_read()
    bytes_h2d = 2.0 * n * kh.stride(0) * kh.element_size() * cfg.steps + 4.0 * H * n * cfg.steps
    print(json.dumps({"mode": "out-of-core update (host-streamed K, V, eta)", "workload": cfg.name,
                      "update_tokens": n, "inner_steps": cfg.steps, "batch_tokens": batch,
                      "tokens_per_s": n * steps / el, "ms_per_update": el * 1e3 / steps,
                      "h2d_gb_per_update": bytes_h2d / 1e9, "h2d_gbs": bytes_h2d * steps / el / 1e9,
                      "gradient_kernel_ms_per_update": kt["grad"][0] / steps}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer's multi-GPU sharding "
              "is a design note, not built.", file=sys.stderr)
        sys.exit(2)
    if args.oracle_only:
        from test_weight_layers_amd.configs import CONFIGS
        cfg = CONFIGS[args.config]
        frames = min(args.cpu_sample_frames, args.frames or cfg.frames)
        print(json.dumps({"workload": cfg.name, "cpu_baseline": cpu_baseline(cfg, frames, args.oracle_threads)}),
              flush=True)
        return
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    if args.sweep:
        linear_sweep(args.steps, args.warmup)
        return
    from test_weight_layers_amd import synth, ttt
    from test_weight_layers_amd.configs import CONFIGS

    cfg = CONFIGS[args.config]
    if args.frames:
        cfg = cfg.with_frames(args.frames)
    if args.host_stream:
        host_stream(cfg, args.host_stream, args.steps, args.warmup)
        return
    torch.cuda.set_device(0)
    ttt.load()
    t_gen = time.perf_counter()
    inp = synth.to_device(synth.make_inputs(cfg), "cuda")
    gen_s = time.perf_counter() - t_gen
    H, d, m = cfg.heads, cfg.d, cfg.m
    n, nq = inp.k.shape[0], inp.q.shape[0]
    dt = inp.k.dtype
    geo = dict(frames=cfg.frames, tokens_per_frame=cfg.tokens_per_frame, n_special=cfg.n_special,
               grid_h=cfg.grid_h, grid_w=cfg.grid_w)
    w0 = (inp.w1, inp.w3, inp.w2)
    w_out = tuple(torch.empty_like(x) for x in w0)
    o = torch.empty((nq, H * d), dtype=dt, device="cuda")
    chunk = cfg.chunk_frames * cfg.tokens_per_frame
    # per-call HIP events on the launch stream (torch's current stream, which the
    # library launches on), recorded between the API calls of each timed step
    marks, recording = [], [False]

    def mark(tag):
        if recording[0]:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append((tag, e))

    if chunk:
        # causal stream: per chunk apply with the current W, then update W from the chunk
        ws = torch.empty(ttt.stream_workspace_bytes(H, d, m, chunk, dt), dtype=torch.uint8, device="cuda")

        def step():
            for a, b in zip(w_out, w0):
                a.copy_(b)
            mark("start")
            ttt.stream(w_out, inp.k, inp.v, inp.eta, inp.q, cfg.lr, cfg.steps, chunk, out=o, workspace=ws,
                       norm_preserve=cfg.norm_preserve)
            mark("stream")
    else:
        v2 = torch.empty_like(inp.v)
        ws_u = torch.empty(ttt.update_workspace_bytes(H, d, m, n, dt), dtype=torch.uint8, device="cuda")
        nws = ttt.apply_workspace_bytes(H, d, m, nq, dt)
        ws_a = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        if cfg.gate:
            wg, gamma = (t.cuda() for t in synth.gate_weights(cfg.seed, H * d, dt))
            o_gated = torch.empty_like(o)

        def step():
            v = inp.v
            mark("start")
            if cfg.conv:
                ttt.shortconv2d(inp.v, inp.wconv, **geo, out=v2)
                v = v2
                mark("conv")
            ttt.update(w0, inp.k, v, inp.eta, cfg.lr, cfg.steps, out=w_out, workspace=ws_u,
                       norm_preserve=cfg.norm_preserve)
            mark("update")
            ttt.apply(w_out, inp.q, out=o, workspace=ws_a)
            mark("apply")
            if cfg.gate:
                ttt.output_gate(o, wg, gamma, cfg.gate_eps, out=o_gated)
                mark("gate")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    marks.clear()
    recording[0] = True
    prof = not args.no_profile_events
    ttt.profile_reset()
    ttt.profile_enable(prof)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    recording[0] = False
    ttt.profile_enable(False)
    kt = ttt.profile_read() if prof else {}
    ms_step = elapsed * 1e3 / args.steps

    grad_f, apply_f, ns_f, conv_f = flops(cfg, n, nq)
    updates_per_step = 1
    grad_launch_f = grad_f
    if chunk:   # one update (and one Newton-Schulz) per chunk
        updates_per_step = (n + chunk - 1) // chunk
        grad_launch_f = flops(cfg, chunk, 0)[0]
    value = n * args.steps / elapsed
    out = {
        "metric": "TTT layer tokens/sec (update+apply) on 1 MI355X; % dense-bf16 MFMA peak",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32", "data": "synthetic (seeded N(0,1)/U(0,0.1) tokens, "
        "random-init fast weights)",
        "config": {"workload": cfg.name, "frames": cfg.frames, "tokens_per_frame": cfg.tokens_per_frame,
                   "update_tokens": n, "apply_tokens": nq, "heads": H, "d": d, "hidden": m,
                   "inner_steps": cfg.steps, "shortconv2d": cfg.conv, "lr": cfg.lr,
                   "stream_chunk_tokens": chunk or None, "norm_preserving_step": cfg.norm_preserve,
                   "gated_output": cfg.gate},
        "input_gen_s": round(gen_s, 2),
    }
    peak = PEAK_BF16_TFLOPS if dt == torch.bfloat16 else PEAK_F32_TFLOPS
    if kt:
        g_ms, g_n = kt["grad"]
        a_ms, a_n = kt["apply"]
        per_kernel = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps}
                      for k, v in kt.items()}
        out["kernels"] = per_kernel
        gemm_flops = (grad_f * cfg.steps + apply_f + gate_flops(cfg, nq)) * args.steps
        gemm_ms = g_ms + a_ms + (kt["gate"][0] if cfg.gate else 0.0)
        out["mfma_pct_gemm_phases"] = 100.0 * gemm_flops / (gemm_ms * 1e-3) / (peak * 1e12)
        out["mfma_pct_whole_layer"] = (100.0 * (gemm_flops + ns_f * cfg.steps * updates_per_step * args.steps)
                                       / elapsed / (peak * 1e12))
        grad_avg_s = g_ms * 1e-3 / g_n
        achieved = grad_launch_f / grad_avg_s / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": "grad (fused forward + SwiGLU backward + weight-gradient "
                           "contractions)", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                           "frac": achieved / peak,
                           "traffic": measured_traffic(d) if cfg.name.startswith("c5a") else None,
                           "avg_launch_ms": grad_avg_s * 1e3, "flop_per_launch": grad_launch_f}
        if a_n:
            a_avg = a_ms * 1e-3 / a_n
            apply_launch_f = apply_f * args.steps / a_n
            out["apply_kernel"] = {"achieved_tflops": apply_launch_f / a_avg / 1e12,
                                   "frac": apply_launch_f / a_avg / 1e12 / peak,
                                   "avg_launch_ms": a_avg * 1e3}
        if cfg.gate and kt["gate"][1]:
            q_ms, q_n = kt["gate"]
            q_avg = q_ms * 1e-3 / q_n
            q_f = gate_flops(cfg, nq)
            out["gate_kernel"] = {"achieved_tflops": q_f / q_avg / 1e12, "peak": peak,
                                  "frac": q_f / q_avg / 1e12 / peak, "avg_launch_ms": q_avg * 1e3,
                                  "flop_per_launch": q_f}
        if cfg.conv and kt["conv"][1]:
            c_avg = kt["conv"][0] * 1e-3 / kt["conv"][1]
            conv_bytes = 2.0 * n * H * d * inp.v.element_size()
            out["conv_kernel"] = {"achieved_gbs": conv_bytes / c_avg / 1e9, "peak_gbs": PEAK_HBM_GBS,
                                  "frac": conv_bytes / c_avg / 1e9 / PEAK_HBM_GBS, "avg_launch_ms": c_avg * 1e3}
        if dt == torch.bfloat16:
            # the matrix cores' sustained dense bf16 rate on this machine (register-only MFMA
            # chains on every SIMD), next to the published peak the fractions above use
            p_meas = measured_mfma_peak()
            out["mfma_peak_measured"] = {"tflops": p_meas, "published_tflops": peak,
                                         "probe": "ttt_mfma_rate_probe, 65536 rounds x 8 chains per wave, "
                                                  "2 waves per SIMD, median of 5 launches"}
            out["mfma_pct_gemm_phases_of_measured_peak"] = 100.0 * gemm_flops / (gemm_ms * 1e-3) / (p_meas * 1e12)
    if marks:
        out["per_call_ms"] = per_call_stats(marks)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_sample_frames, cfg.frames), args.oracle_threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

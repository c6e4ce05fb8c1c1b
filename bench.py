"""Benchmark of the GPTQ layer path on one MI355X.

One step is the whole layer path on device-resident inputs:
  H = 2 X^T X (gptq_hessian_accumulate), U = chol((H + lambda I)^-1)
  (gptq_prepare_hinv), and the column sweep with packing and loss
  (gptq_quantize_layer).
Default workload: the 175B-class layer W 49152 x 12288 fp16, 3-bit, group
128, with 128 x 2048 = 262144 fp16 calibration tokens of width 12288, damp
0.01, B = 128 (seeded synthetic inputs standing in for C4 activations and
real weights). This is the largest layer one GPU quantizes on its own.

Prints one JSON line. `value` is weight columns quantized per second for
the whole layer path (d_col / step time); per-stage times, the Hessian
TFLOP/s, each stage against its roofline (the dominant stage's as
`roofline`), the same path on the 4096 x 4096 attention-projection layer,
and the float64 oracle's rate on this machine's CPU cores are reported
beside it.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GPTQ layer quantize time (ms) + weight-cols/s; Hessian SYRK TFLOP/s, % peak"
PEAK_FP16_MFMA = 2.5e15  # dense fp16 MFMA, MI355X
PEAK_FP32_MFMA = 157.3e12
PEAK_FP64_MFMA = 78.6e12
PEAK_HBM = 8.0e12


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def upload_activations(cfg, torch, dev):
    from workload import activation_chunks

    X = torch.empty((cfg.n_tokens, cfg.d_col), dtype=getattr(torch, cfg.x_dtype), device=dev)
    t, t0, shown = 0, time.perf_counter(), time.perf_counter()
    for ch in activation_chunks(cfg, threads=min(16, os.cpu_count() or 8)):
        X[t : t + ch.shape[0]].copy_(torch.from_numpy(ch))
        t += ch.shape[0]
        if time.perf_counter() - shown > 20:
            shown = time.perf_counter()
            log(f"bench: {t} of {cfg.n_tokens} tokens generated and uploaded ({shown - t0:.0f} s)")
    return X


def counter_traffic_bytes(profile: str, source: str, tag: str):
    """HBM bytes per call of one stage from a committed counter summary.

    The summary under profiles/ holds a line
    `bench-traffic[<tag>]: source_sha256=... fetch_kib=... write_kib=...
    fetch_scale=... write_scale=...` with FETCH_SIZE and WRITE_SIZE (KiB
    per call, summed over the stage's kernels), the copy-calibration
    scales and the SHA-256 of the kernel source they were taken with.
    Returns None when that source has changed since (the counters no
    longer describe the kernel) or the line is missing.
    """
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", profile)
    src = os.path.join(ROOT, "post_weight_quantization_17_amd", "csrc", source)
    try:
        text = open(path).read()
        m = re.search(rf"bench-traffic\[{re.escape(tag)}\]: source_sha256=(\w+) fetch_kib=(\S+) write_kib=(\S+) "
                      rf"fetch_scale=(\S+) write_scale=(\S+)", text)
        if not m or hashlib.sha256(open(src, "rb").read()).hexdigest() != m.group(1):
            return None
        fk, wk, fs, ws = (float(m.group(i)) for i in range(2, 6))
        return (fk * fs + wk * ws) * 1024.0
    except OSError:
        return None


def cpu_baseline(cfg, budget_rows=256, budget_tokens=8192, budget_width=6144):
    """The float64 oracle timed on a bounded sample of the same layer, on
    this machine's host cores (BLAS threads set to the cores this process
    may run on).

    Sample (rows are independent given U, and the Hessian's cost is linear
    in tokens): the Hessian of the first `budget_tokens` tokens, its time
    scaled by n_tokens / budget_tokens; the damped factor (route A as the
    oracle states it) at full width up to `budget_width`, else of the
    leading budget_width x budget_width block of that Hessian with its time
    scaled by (d / budget_width)^3 (dense Cholesky and inversion cost d^3);
    the plain column sweep of a fixed seeded subset of `budget_rows` rows
    with the full-width factor's shape, its time scaled by d_row /
    budget_rows. The whole oracle runs when the layer is that small.
    """
    import oracle.gptq_oracle as O
    from workload import activation_chunks, weights

    cores = len(os.sched_getaffinity(0))
    blas_threads = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        limiter = threadpool_limits(cores)
        blas_threads = max([p.get("num_threads", 0) for p in threadpool_info()] or [0]) or None
    except Exception:  # pragma: no cover - threadpoolctl is part of the image
        limiter = None
    chunks, got = [], 0
    for ch in activation_chunks(cfg, threads=4):
        chunks.append(ch)
        got += ch.shape[0]
        if got >= budget_tokens:
            break
    Xs = np.concatenate(chunks)[:budget_tokens]
    n_rows = min(budget_rows, cfg.d_row)
    rows = np.sort(np.random.default_rng(0).choice(cfg.d_row, n_rows, replace=False))
    Ws = weights(cfg, rows=rows)
    fw = min(cfg.d_col, budget_width)
    t0 = time.perf_counter()
    H = O.hessian([Xs[i : i + 4096] for i in range(0, len(Xs), 4096)])
    t1 = time.perf_counter()
    O.prepare_hinv(H[:fw, :fw], cfg.damp)
    t2 = time.perf_counter()
    # the sweep needs a factor of full width: the Hessian's diagonal part
    # gives one at O(d) cost (the sweep's own cost does not depend on U's values)
    U = np.diag(1.0 / np.sqrt(np.diag(H) * (1 + cfg.damp)))
    t2b = time.perf_counter()
    O.quantize_layer(Ws, U, cfg.bits, cfg.group_size, cfg.block)
    t3 = time.perf_counter()
    if limiter is not None:
        limiter.restore_original_limits()
    t_h = (t1 - t0) * cfg.n_tokens / len(Xs)
    t_u = (t2 - t1) * (cfg.d_col / fw) ** 3
    t_q = (t3 - t2b) * cfg.d_row / n_rows
    total = t_h + t_u + t_q
    full = len(Xs) == cfg.n_tokens and n_rows == cfg.d_row and fw == cfg.d_col
    return {
        "value": cfg.d_col / total,
        "unit": "weight-cols/s",
        "cores": int(cores),
        "blas_threads": blas_threads,
        "kind": "oracle",
        "sample": (
            "float64 numpy oracle, whole layer" if full else
            f"float64 numpy oracle: Hessian of {len(Xs)} of {cfg.n_tokens} tokens (time x{cfg.n_tokens / len(Xs):.0f}), "
            f"damped factor at width {fw} of {cfg.d_col} (time x{(cfg.d_col / fw) ** 3:.1f}), plain sweep of "
            f"{n_rows} seeded rows of {cfg.d_row} (time x{cfg.d_row / n_rows:.0f}); measured {t3 - t0:.1f} s on "
            f"{cores} cores, extrapolated layer time {total:.1f} s"
        ),
        "stage_s": {"hessian": t_h, "prepare_hinv": t_u, "quantize_layer": t_q},
        "measured_s": t3 - t0,
    }


def matvec_measure(g, torch, q, W, cfg, reps=50, replays=10):
    """Quantized-matrix x fp16-vector product on the layer's packed output
    (batch 1), timed by replaying a HIP graph of `reps` calls (host launch
    overhead would otherwise dominate a kernel of a few microseconds). The
    replayed result is checked against an eager call. The dense fp16 product
    on the same layer is timed the same way for comparison."""
    dev = W.device
    d_row, d_col = W.shape
    gen = torch.Generator(device="cpu").manual_seed(1)
    x = torch.randn((1, d_col), generator=gen).to(torch.float16).to(dev)
    y = torch.empty((1, d_row), dtype=torch.float32, device=dev)
    call = lambda: g.gptq_dequant_matvec(q.packed, q.scales, q.zeros, d_col, cfg.bits, cfg.group_size, x, y=y)
    call()
    torch.cuda.synchronize()
    ref = y.clone()

    def time_graph(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * replays)

    us = time_graph(call)
    if not torch.equal(y, ref):
        raise RuntimeError("graph replay of the packed matrix-vector product differs from the eager call")
    Wh = W.to(torch.float16)
    yd = torch.empty((1, d_row), dtype=torch.float16, device=dev)
    dense_us = time_graph(lambda: torch.matmul(x, Wh.t(), out=yd))
    nbytes = (q.packed.numel() + q.scales.numel() + q.zeros.numel()) * 4 + x.numel() * 2 + y.numel() * 4
    return {
        "batch": 1,
        "us": us,
        "bytes": nbytes,
        "gbps": nbytes / (us * 1e-6) / 1e9,
        "frac_hbm": nbytes / (us * 1e-6) / PEAK_HBM,
        "fp16_dense_us": dense_us,
        "fp16_dense_bytes": Wh.numel() * 2,
        "kernel": (
            "dequant_matvec_pairs" if cfg.group_size == -1 or cfg.group_size % 32 == 0 else "dequant_matvec_kernel"
        ) + " (gptq_dequant_matvec), timed by HIP graph replay",
    }


def act_order_measure(g, torch, H, W, q_nat, cfg, ws_u, ws_q, steps=3):
    """The layer in act-order from the same Hessian: permutation, gathers of
    H and W, factor, sweep, and the codes gathered back to the original
    column order, each timed with HIP events on the current stream. Reports
    the per-step time of these stages, the W gather's HBM rate, and the
    layer loss beside the natural order's."""
    dev = W.device
    d = H.shape[0]
    perm = torch.empty(d, dtype=torch.int32, device=dev)
    inv = torch.empty(d, dtype=torch.int32, device=dev)
    Hp = torch.empty_like(H)
    Wp = torch.empty_like(W)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    hv = g.Hinv(torch.empty_like(H), torch.empty((), dtype=torch.float32, device=dev),
                torch.empty((), dtype=torch.int32, device=dev))
    q = g.gptq_quantize_layer(W, H, cfg.bits, cfg.group_size, cfg.block, ws=ws_q)  # allocates the outputs once
    codes_orig = torch.empty_like(q.codes)
    names = ["perm", "gather_H", "prepare_hinv", "gather_W", "quantize_layer", "gather_codes"]

    def run(ev=None):
        calls = [
            lambda: g.gptq_act_order_perm(H, perm, inv),
            lambda: g.gptq_gather(H, perm, perm, out=Hp, info=info),
            lambda: g.gptq_prepare_hinv(Hp, cfg.damp, ws=ws_u, out=hv),
            lambda: g.gptq_gather(W, None, perm, out=Wp, info=info),
            lambda: g.gptq_quantize_layer(Wp, hv.U, cfg.bits, cfg.group_size, cfg.block, ws=ws_q, out=q),
            lambda: g.gptq_gather(q.codes, None, inv, out=codes_orig, info=info),
        ]
        for k, c in enumerate(calls):
            if ev:
                ev[k].record()
            c()
        if ev:
            ev[len(calls)].record()

    run()
    torch.cuda.synchronize()
    if int(hv.info.item()) != 0 or int(info.item()) != 0:
        raise RuntimeError("act-order path failed")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for k in range(steps):
        run(evs[k])
    torch.cuda.synchronize()
    t = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    w_bytes = 2.0 * W.numel() * W.element_size()
    return {
        "stages_ms": t,
        "ms_after_hessian": float(sum(t.values())),
        "gather_W_gbps": w_bytes / (t["gather_W"] * 1e-3) / 1e9,
        "loss_act_order": float(q.loss.item()),
        "loss_natural_order": float(q_nat.loss.item()),
        "steps": steps,
    }


def pipeline_measure(g, torch, X, W, cfg, steps=2):
    """The calibration pipeline on the layer's activations X [N, d] (fp16):
    (a) q/k/v sharing one Hessian and factor, each layer swept with it; (b)
    an MLP block d -> 11008 -> d quantized layer by layer, the down layer
    calibrated on the quantized up layer's output, each quantized layer run
    on the tokens by gptq_dequant_gemm (ReLU fused for the up layer). Weights
    beyond the layer's own are seeded synthetic N(0, sigma^2) fp16. Every
    stage is timed with HIP events on the current stream (1 untimed, `steps`
    timed runs). For comparison only, the same two products through the
    library GEMM (dequantize to fp16, then torch.matmul) are timed apart."""
    dev = X.device
    d = X.shape[1]
    gen = torch.Generator(device=dev).manual_seed(7)
    sig = cfg.w_sigma
    Wk = (sig * torch.randn(W.shape, generator=gen, device=dev)).to(W.dtype)
    Wv = (sig * torch.randn(W.shape, generator=gen, device=dev)).to(W.dtype)
    d_ff = 11008
    W_up = (sig * torch.randn((d_ff, d), generator=gen, device=dev)).to(torch.float16)
    W_down = (sig * torch.randn((d, d_ff), generator=gen, device=dev)).to(torch.float16)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def qkv(e=None):
        if e:
            e[0].record()
        H = g.gptq_hessian_accumulate(X)
        if e:
            e[1].record()
        hv = g.gptq_prepare_hinv(H, cfg.damp)
        if e:
            e[2].record()
        for Wl in (W, Wk, Wv):
            g.gptq_quantize_layer(Wl, hv.U, cfg.bits, cfg.group_size, cfg.block)
        if e:
            e[3].record()

    qkv()
    es = [[ev() for _ in range(4)] for _ in range(steps)]
    for k in range(steps):
        qkv(es[k])
    torch.cuda.synchronize()
    m = lambda e, i, j: float(np.mean([x[i].elapsed_time(x[j]) for x in e]))
    qkv_ms = {"hessian": m(es, 0, 1), "prepare_hinv": m(es, 1, 2), "quantize_3_layers": m(es, 2, 3),
              "total": m(es, 0, 3)}

    def block(e=None):
        marks = []

        def mark():
            if e is not None:
                t = ev()
                t.record()
                marks.append(t)

        mark()
        H_up = g.gptq_hessian_accumulate(X)
        mark()
        hv_up = g.gptq_prepare_hinv(H_up, cfg.damp)
        mark()
        q_up = g.gptq_quantize_layer(W_up, hv_up.U, cfg.bits, cfg.group_size, cfg.block)
        mark()
        X1 = g.gptq_dequant_gemm(q_up.packed, q_up.scales, q_up.zeros, d, cfg.bits, cfg.group_size, X, relu=True)
        mark()
        H_dn = g.gptq_hessian_accumulate(X1)
        mark()
        hv_dn = g.gptq_prepare_hinv(H_dn, cfg.damp)
        mark()
        q_dn = g.gptq_quantize_layer(W_down, hv_dn.U, cfg.bits, cfg.group_size, cfg.block)
        mark()
        X2 = g.gptq_dequant_gemm(q_dn.packed, q_dn.scales, q_dn.zeros, d_ff, cfg.bits, cfg.group_size, X1)
        mark()
        if e is not None:
            e.append(marks)
        return hv_up, hv_dn, q_up, q_dn, X1, X2

    hv_up, hv_dn, q_up, q_dn, X1, X2 = block()
    torch.cuda.synchronize()
    if int(hv_up.info.item()) != 0 or int(hv_dn.info.item()) != 0:
        raise RuntimeError("factorization failed in the MLP block")
    runs = []
    for _ in range(steps):
        block(runs)
    torch.cuda.synchronize()
    names = ["hessian_up", "prepare_hinv_up", "quantize_up", "dequant_gemm_relu_up", "hessian_down",
             "prepare_hinv_down", "quantize_down", "dequant_gemm_down"]
    blk = {n: float(np.mean([r[i].elapsed_time(r[i + 1]) for r in runs])) for i, n in enumerate(names)}
    blk["total"] = float(np.mean([r[0].elapsed_time(r[-1]) for r in runs]))
    n = X.shape[0]
    gemm_flops = 2.0 * n * d * d_ff
    blk["dequant_gemm_tflops"] = {
        "up": gemm_flops / (blk["dequant_gemm_relu_up"] * 1e-3) / 1e12,
        "down": gemm_flops / (blk["dequant_gemm_down"] * 1e-3) / 1e12,
    }

    # comparison only: the library GEMM on the dequantized fp16 weights
    Wh_up = g.gptq_dequantize(q_up.packed, q_up.scales, q_up.zeros, d, cfg.bits, cfg.group_size, torch.float16)
    Wh_dn = g.gptq_dequantize(q_dn.packed, q_dn.scales, q_dn.zeros, d_ff, cfg.bits, cfg.group_size, torch.float16)
    lib_ms = {}
    for name, (A, Bt) in {"up": (X, Wh_up), "down": (X1, Wh_dn)}.items():
        torch.matmul(A, Bt.t())
        a0, a1 = ev(), ev()
        a0.record()
        for _ in range(steps):
            torch.matmul(A, Bt.t())
        a1.record()
        torch.cuda.synchronize()
        lib_ms[name] = a0.elapsed_time(a1) / steps
    del Wh_up, Wh_dn
    return {
        "qkv_shared_input_ms": qkv_ms,
        "mlp_block": {"d_model": d, "d_ff": d_ff, "tokens": n, "stages_ms": blk},
        "library_gemm_ms_for_comparison": lib_ms,
        "steps": steps,
    }


def layer_leg(g, torch, cfg, X, W, steps, warmup):
    """The layer path (Hessian, factor, sweep) on device-resident X and W:
    `warmup` untimed steps (the first event-timed per stage and reported as
    the cold step), then `steps` steps, each stage bracketed by HIP events
    on torch's current stream, which is the stream every call enqueues on.
    Returns the times and the last step's outputs."""
    dev = X.device
    d, n = cfg.d_col, cfg.n_tokens
    ws_h = torch.empty(g.gptq_hessian_workspace_size(n, d, X.dtype), dtype=torch.uint8, device=dev)
    ws_u = torch.empty(g.gptq_prepare_hinv_workspace_size(d), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(
        g.gptq_quantize_layer_workspace_size(cfg.d_row, d, cfg.bits, cfg.group_size, cfg.block), dtype=torch.uint8,
        device=dev)
    H = torch.empty((d, d), dtype=torch.float32, device=dev)
    hv = g.Hinv(
        torch.empty((d, d), dtype=torch.float32, device=dev),
        torch.empty((), dtype=torch.float32, device=dev),
        torch.empty((), dtype=torch.int32, device=dev),
    )
    eye = torch.eye(d, dtype=torch.float32, device=dev)
    q = g.gptq_quantize_layer(W, eye, cfg.bits, cfg.group_size, cfg.block, ws=ws_q)  # allocates the outputs once
    del eye

    def step(ev=None):
        if ev:
            ev[0].record()
        g.gptq_hessian_accumulate(X, H=H, ws=ws_h)
        if ev:
            ev[1].record()
        g.gptq_prepare_hinv(H, cfg.damp, ws=ws_u, out=hv)
        if ev:
            ev[2].record()
        g.gptq_quantize_layer(W, hv.U, cfg.bits, cfg.group_size, cfg.block, ws=ws_q, out=q)
        if ev:
            ev[3].record()

    # The first warm-up step is the cold call (code objects load, the factor's
    # auxiliary stream is created); it is event-timed and reported apart.
    cold = None
    for w in range(warmup):
        if w == 0:
            cev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            step(cev)
            torch.cuda.synchronize()
            cold = {
                "total": cev[0].elapsed_time(cev[3]),
                "hessian": cev[0].elapsed_time(cev[1]),
                "prepare_hinv": cev[1].elapsed_time(cev[2]),
                "quantize_layer": cev[2].elapsed_time(cev[3]),
            }
        else:
            step()
    torch.cuda.synchronize()
    if int(hv.info.item()) != 0:
        raise RuntimeError(f"factorization failed: info={int(hv.info.item())}")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for k in range(steps):
        step(evs[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end) / steps
    stages = {
        "hessian": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
        "prepare_hinv": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
        "quantize_layer": float(np.mean([e[2].elapsed_time(e[3]) for e in evs])),
    }
    median_ms = float(np.median([e[0].elapsed_time(e[3]) for e in evs]))
    log(f"bench: {cfg.name}: {steps} steps in {wall:.3f} s wall; per step {ms:.3f} ms "
        f"(H {stages['hessian']:.3f}, U {stages['prepare_hinv']:.3f}, Q {stages['quantize_layer']:.3f})")
    return dict(ms=ms, median_ms=median_ms, stages=stages, cold=cold, wall_s=wall, H=H, hv=hv, q=q, ws_u=ws_u,
                ws_q=ws_q)


def stage_rooflines(cfg, stages):
    """Each stage against the roofline that bounds it, on algorithmic work:
    the Hessian's triangle N d (d + 1) flops on the fp16 MFMA peak, the
    factor's 2 d^3 / 3 flops (route B) on the fp64 peak, the sweep's
    deferred-update flops sum over blocks of 2 d_row B (d_col - i2) on the
    fp32 peak. `traffic` is HBM bytes per call from the committed counter
    summary of that workload, or null when none matches the current source."""
    d, n = cfg.d_col, cfg.n_tokens
    prof = f"{cfg.name}_counters.md"
    syrk_flops = float(n) * d * (d + 1)
    chol_flops = 2.0 * d**3 / 3.0
    trail_flops = float(sum(2.0 * cfg.d_row * cfg.block * (d - i2) for i2 in range(cfg.block, d, cfg.block)))

    def rl(kernel, flops, ms, peak, dtype, source, tag):
        achieved = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "dtype": dtype, "kernel": kernel, "achieved": achieved, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved * 1e12 / peak,
                "traffic": counter_traffic_bytes(prof, source, tag), "traffic_unit": "bytes",
                "per_launch_flops": flops, "launch_ms": ms}

    return {
        "hessian": rl("syrk_f16_lds + syrk_reduce (one gptq_hessian_accumulate call)", syrk_flops,
                      stages["hessian"], PEAK_FP16_MFMA, "f16 in, f32 accumulate", "hessian.hip", "hessian"),
        "prepare_hinv": rl("hinv_* chain (one gptq_prepare_hinv call; route B, fp64)", chol_flops,
                           stages["prepare_hinv"], PEAK_FP64_MFMA, "f64", "hinv.hip", "prepare_hinv"),
        "quantize_layer": rl("gptq_sweep + loss_final (one gptq_quantize_layer call); flops of the deferred update "
                             "only", trail_flops, stages["quantize_layer"], PEAK_FP32_MFMA, "f32", "quantize.hip",
                             "quantize_layer"),
    }


SECOND_LAYER = "attn_proj_4096x4096_4bit_g128"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="opt175b_49152x12288_3bit_g128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only the layer path of --config (no act-order, packed-product, second-layer or "
                         "pipeline legs)")
    ap.add_argument(
        "--copy-calibration",
        action="store_true",
        help="only run a plain 1 GiB device-to-device copy (3 times), the reference for HBM byte counters",
    )
    args = ap.parse_args()
    if args.gpus != 1:
        print(
            f"bench.py measures one GPU: the GPTQ layer path here runs on a single MI355X "
            f"(--gpus {args.gpus} is not supported; multi-GPU sharding is described in DESIGN.md)",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_copy": 1 << 30, "bytes_written_per_copy": 1 << 30}))
        return

    import post_weight_quantization_17_amd as g
    from workload import CONFIGS, weights

    g.load()
    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    log(f"bench: {cfg.name}: W {cfg.d_row}x{cfg.d_col} {cfg.w_dtype}, X {cfg.n_tokens}x{cfg.d_col} {cfg.x_dtype}")
    t0 = time.perf_counter()
    X = upload_activations(cfg, torch, dev)
    W = torch.from_numpy(weights(cfg)).to(dev)
    torch.cuda.synchronize()
    log(f"bench: inputs resident in HBM after {time.perf_counter() - t0:.1f} s")

    leg = layer_leg(g, torch, cfg, X, W, args.steps, args.warmup)
    ms, stages = leg["ms"], leg["stages"]
    d, n = cfg.d_col, cfg.n_tokens
    rls = stage_rooflines(cfg, stages)
    dominant = max(stages, key=stages.get)
    syrk_tflops = rls["hessian"]["achieved"]
    out = {
        "metric": METRIC,
        "value": d / (ms * 1e-3),
        "unit": "weight-cols/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in / f32 accumulate (H); f64 (factor); f32 (sweep)",
        "data": "synthetic (seeded; stands in for C4 activations and real weights)",
        "config": {
            "workload": cfg.name,
            "d_row": cfg.d_row,
            "d_col": d,
            "n_tokens": n,
            "bits": cfg.bits,
            "group_size": cfg.group_size,
            "block": cfg.block,
            "damp": cfg.damp,
        },
        "stages_ms": stages,
        "layer_ms": ms,
        "quantize_layer_ms": stages["quantize_layer"],
        "median_step_ms": leg["median_ms"],
        "cold_step_ms": leg["cold"],
        "quantize_weight_cols_per_s": d / (stages["quantize_layer"] * 1e-3),
        "weights_per_s": cfg.d_row * d / (ms * 1e-3),
        "hessian_tflops": syrk_tflops,
        "hessian_pct_fp16_peak": 100.0 * rls["hessian"]["frac"],
        "prepare_hinv_tflops_fp64": rls["prepare_hinv"]["achieved"],
        "quantize_trailing_tflops_lower_bound": rls["quantize_layer"]["achieved"],
        "roofline": dict(rls[dominant], stage=dominant),
        "stage_rooflines": rls,
        "roofline_floor_ms": float(sum(r["per_launch_flops"] / (r["peak"] * 1e12) * 1e3 for r in rls.values())),
        "cpu_baseline": None,
    }
    log(f"bench: dominant stage {dominant}: {rls[dominant]['achieved']:.1f} TFLOP/s = "
        f"{100 * rls[dominant]['frac']:.1f}% of {rls[dominant]['peak']:.1f}")
    if not args.layer_only:
        out["act_order"] = act_order_measure(g, torch, leg["H"], W, leg["q"], cfg, leg["ws_u"], leg["ws_q"])
        ao = out["act_order"]
        log(f"bench: act-order path after H {ao['ms_after_hessian']:.3f} ms {ao['stages_ms']}; "
            f"loss {ao['loss_act_order']:.6g} (natural order {ao['loss_natural_order']:.6g})")
        out["dequant_matvec"] = matvec_measure(g, torch, leg["q"], W, cfg)
        log(f"bench: packed matrix-vector product {out['dequant_matvec']['us']:.2f} us "
            f"({out['dequant_matvec']['gbps']:.0f} GB/s); dense fp16 {out['dequant_matvec']['fp16_dense_us']:.2f} us")
        cfg2 = CONFIGS[SECOND_LAYER] if cfg.name != SECOND_LAYER else None
        if cfg2 is not None:
            del leg, X, W
            torch.cuda.empty_cache()
            X2 = upload_activations(cfg2, torch, dev)
            W2 = torch.from_numpy(weights(cfg2)).to(dev)
            leg2 = layer_leg(g, torch, cfg2, X2, W2, 10, 3)
            rl2 = stage_rooflines(cfg2, leg2["stages"])
            out["second_layer"] = {
                "workload": cfg2.name, "ms_per_step": leg2["ms"], "median_step_ms": leg2["median_ms"],
                "stages_ms": leg2["stages"], "cold_step_ms": leg2["cold"],
                "weight_cols_per_s": cfg2.d_col / (leg2["ms"] * 1e-3), "stage_rooflines": rl2, "steps": 10,
            }
            del leg2
        else:  # the headline layer is the 4096-wide layer: the pipeline runs on its activations
            X2, W2, cfg2 = X, W, cfg
        if X2.dtype == torch.float16:
            out["pipeline"] = pipeline_measure(g, torch, X2, W2, cfg2)
            pl = out["pipeline"]
            log(f"bench: q/k/v sharing one Hessian {pl['qkv_shared_input_ms']['total']:.2f} ms "
                f"{pl['qkv_shared_input_ms']}")
            log(f"bench: MLP block layer by layer {pl['mlp_block']['stages_ms']['total']:.2f} ms "
                f"{pl['mlp_block']['stages_ms']}")
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(cfg)
        log(f"bench: oracle {out['cpu_baseline']['sample']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of GPTQ's per-layer quantization path on one MI355X.

Workload: one Llama-7B-shaped attention projection, W 4096 x 4096 bf16, from
262144 bf16 calibration tokens (128 sequences x 2048), 4-bit asymmetric,
group size 128, block 128, damping 0.01 -- synthetic seeded inputs that stand
in for a real model's weights and activations.

One step = the whole path on resident inputs: zero H, H += 2 X^T X over all
tokens, damping + factorization -> U, the greedy column loop with lazy
trailing updates, and packing.  Each stage is bracketed by HIP events on the
stream the library launches on.  Prints one JSON line on stdout; progress
goes to stderr.  Besides the throughput the line holds: `roofline` (the
Hessian accumulation, the dominant kernel, against the bf16 matrix peak),
`e2e_roofline_frac` (the sum of every stage's time at its roofline divided
by the measured step time, stage floors in `roofline_bound_ms`),
`trailing_gemm` (the far trailing updates' kernels, timed by the profiler
over one more quantize call, against the bf16 matrix peak; the near updates
inside a group of blocks run in the column loop's launch) and `cpu_baseline`
(the float64 oracle on a bounded sample of the same problem).  --layer small
runs the 256 x 256 fp32 layer, whose oracle baseline is the whole problem.

--workload gptq2d instead times two-sided rounding (gptq2d_round) of an n x n
float64 matrix under seeded upper-triangular bases triu(I + 0.1 N(0,1)),
n = 1024 by default; one step is one whole rounding.  --workload w4a16 times
the dequantized 4-bit product (gptq_w4a16_matmul) of an m x 4096 bf16 X with
the packed 4096 x 4096 g128 weights (m = 4096 by default).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix (and packed vector) peak
PEAK_HBM_GBS = 8000.0


FAR_GROUP = 4  # blocks per group of the quantizer's far trailing update


def far_update_flops(d_out: int, d_in: int, block: int) -> float:
    """Algorithmic flops of the far trailing updates: after each group of
    FAR_GROUP blocks, W[:, after the group] -= Err U[group, after the group]."""
    nb = -(-d_in // block)
    f = 0.0
    for g0 in range(0, nb, FAR_GROUP):
        gcol = min(d_in, min(nb, g0 + FAR_GROUP) * block)
        if gcol < d_in:
            f += 2.0 * d_out * (gcol - g0 * block) * (d_in - gcol)
    return f


def roofline_bound_ms(wl) -> dict:
    """Time of each stage at its roofline (MI355X published peaks) and the sum
    T_rl: SYRK n d(d+1) flop and trailing update d_out d_in (d_in - B) flop at
    the bf16 matrix peak (the SYRK of fp32 X at the fp32 peak), factorization and triangular inverse 2 d^3 / 3 flop
    and the column loop d_out d_in (B - 1) flop at the fp32 peak, packing (W
    read, codes, fp16 scales and zeros written) at HBM bandwidth."""
    d, n, do, b = wl.d_in, wl.n_tokens, wl.d_out, wl.block
    ng = 1 if wl.group_size == -1 else d // wl.group_size
    wbytes = 2 if wl.w_dtype == "bf16" else 4
    t = {
        "syrk": n * d * (d + 1) / ((PEAK_BF16_TFLOPS if wl.x_dtype == "bf16" else
                                    PEAK_FP32_TFLOPS) * 1e9),
        "factorization": (2.0 * d ** 3 / 3.0) / (PEAK_FP32_TFLOPS * 1e9),
        "column_loop": do * d * (b - 1) / (PEAK_FP32_TFLOPS * 1e9),
        "trailing": do * d * max(d - b, 0) / (PEAK_BF16_TFLOPS * 1e9),
        "pack": (do * d * (wbytes + wl.bits / 8.0) + do * ng * 4) / (PEAK_HBM_GBS * 1e6),
    }
    t["total"] = sum(t.values())
    return t


def device_kernel_ms(fn, names):
    """Device time (ms) of the kernels whose names contain any of `names`,
    over one call of fn, from torch's profiler (which records every kernel the
    process launches, the library's included); None if it records none."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    tot, seen = 0.0, 0
    for e in prof.events():
        if str(getattr(e, "device_type", "")).endswith("CUDA") and any(k in e.name for k in names):
            dt = getattr(e, "device_time", None)
            if dt is None:
                dt = getattr(e, "cuda_time", 0.0)
            tot += float(dt)
            seen += 1
    return tot / 1e3 if seen else None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "post_weight_quantization_syrk_amd", "csrc", "syrk.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profile():
    """HBM-side bytes of one Hessian accumulation (SYRK + split-K reduction)
    from the committed counter summary, if it was taken on the current kernel
    source (else None): FETCH_SIZE x 2 + WRITE_SIZE x 1, the factors that a
    1 GiB device copy gives for the same counters."""
    p = os.path.join(ROOT, "profiles", "syrk_bf16_attn4096_262144tok_traffic.json")
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("syrk_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, synth, max_seconds=30.0, act_order=False, static_groups=False, n_mats=1):
    """The float64 oracle, as it stands, on a bounded sample of the workload,
    scaled to whole-layer weights/s (with act_order: the ordered path)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    n_tok, n_rows = min(4096, wl.n_tokens), min(256, wl.d_out)
    sub = synth.scaled(wl, n_tokens=n_tok, chunk_tokens=n_tok)
    x = synth.as_f64(synth.x_chunk(sub, 0), wl.x_dtype)
    t0 = time.perf_counter()
    H0 = oracle.hessian([x])
    t_h = (time.perf_counter() - t0) * (wl.n_tokens / n_tok)
    W = synth.as_f64(synth.w_matrix(wl), wl.w_dtype)[:n_rows]
    t_a = 0.0
    if act_order:
        t0 = time.perf_counter()
        perm, _ = oracle.activation_order([x])
        t_a = (time.perf_counter() - t0) * (wl.n_tokens / n_tok)
        Hs = np.tril(H0) + np.tril(H0, -1).T
        t0 = time.perf_counter()
        oracle.prepare(Hs[np.ix_(perm, perm)], wl.damp)
        t_p = time.perf_counter() - t0
        t0 = time.perf_counter()
        r = oracle.gptq_ordered(W, H0, perm, damp=wl.damp, bits=wl.bits, group_size=wl.group_size,
                                sym=wl.sym, block=wl.block, static_groups=static_groups)
        # gptq_ordered factorizes again: that part is not per row
        t_q = max(0.0, time.perf_counter() - t0 - t_p) * (wl.d_out / n_rows)
    else:
        t0 = time.perf_counter()
        p = oracle.prepare(H0, wl.damp)
        t_p = time.perf_counter() - t0
        t0 = time.perf_counter()
        r = oracle.gptq(W, p["U"], p["dead"], bits=wl.bits, group_size=wl.group_size, sym=wl.sym,
                        block=wl.block)
        t_q = (time.perf_counter() - t0) * (wl.d_out / n_rows)
    t0 = time.perf_counter()
    oracle.pack_rows(r["codes"], wl.bits)
    oracle.fp16_bits(r["scales"])
    oracle.fp16_bits(r["zeros"])
    t_k = (time.perf_counter() - t0) * (wl.d_out / n_rows)
    # n_mats matrices share the Hessian and the factorization
    total = t_h + t_a + t_p + n_mats * (t_q + t_k)
    return {
        "value": n_mats * wl.d_out * wl.d_in / total,
        "unit": "weights/s",
        "cores": cores,
        "blas_threads": blas_threads,
        "kind": "oracle",
        "sample": (f"Hessian over {n_tok} of {wl.n_tokens} tokens (x{wl.n_tokens // n_tok}); "
                   f"full {wl.d_in}x{wl.d_in} factorization; column loop and packing on {n_rows} "
                   f"of {wl.d_out} rows (x{wl.d_out // n_rows}); float64 numpy/LAPACK, "
                   f"elementwise numpy single-threaded"),
        "seconds": total,
        "stage_seconds_extrapolated": {"hessian": t_h, "act_order": t_a, "prepare": t_p,
                                       "quantize": t_q, "pack": t_k},
    }


def gptq2d_bytes(n: int) -> float:
    """Algorithmic bytes of one two-sided rounding: entry (i, j) reads R_L[i][i:]
    and column j of the running array from row i on (16 (n - i) bytes), reads
    and rewrites its row up to column j and reads column j of R_R (24 (j + 1)),
    and reads Y[i][j] and writes Z[i][j] (16)."""
    return 16.0 * n * (n * (n + 1) / 2) + 24.0 * n * (n * (n + 1) / 2) + 16.0 * n * n


def bench_gptq2d(args):
    import numpy as np
    import torch
    import oracle
    from post_weight_quantization_syrk_amd import gptq, synth

    n = args.n
    dev = "cuda:0"
    torch.cuda.set_device(0)
    gptq.lib()
    y, rl, rr = synth.two_sided_inputs(n)
    Y, RL, RR = (torch.from_numpy(a).to(dev) for a in (y, rl, rr))
    Z = torch.empty((n, n), dtype=torch.float64, device=dev)
    ws = torch.empty(gptq.gptq2d_workspace(n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    log(f"two-sided rounding n={n}: warmup {args.warmup}")
    for _ in range(args.warmup):
        gptq.gptq2d_round(Y, RL, RR, Z=Z, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        gptq.gptq2d_round(Y, RL, RR, Z=Z, ws=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_ev = e0.elapsed_time(e1) / args.steps
    persistent = n <= 1024  # rows held in one wave's registers
    launches = 1 if persistent else 2 * n - 1
    hops = 2 * n - 1  # anti-diagonals: the dependent chain in either schedule
    gbs = gptq2d_bytes(n) / (ms_ev / 1e3) / 1e9
    log(f"{ms:.3f} ms/step ({ms_ev:.3f} ms in events, {launches} launches, "
        f"{1e3 * ms_ev / hops:.2f} us per anti-diagonal)")
    line = {
        "metric": f"two-sided (GPTQ-2D) rounding, matrix entries/sec/GPU (n={n})",
        "value": round(n * n / (ms / 1e3), 1),
        "unit": "entries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic (seeded Y ~ N(0,1), bases triu(I + 0.1 N(0,1)))",
        "config": {"workload": f"gptq2d_two_sided_rounding_n{n}", "n": n},
        "roofline": {
            "kernel": ("g2d_rows_kernel (one persistent launch, a wave per row)" if persistent
                       else "g2d_diag_kernel (one launch per anti-diagonal)"),
            "bound": "hbm",
            "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": round(gptq2d_bytes(n) / launches, 1),
            "avg_launch_ms": round(ms_ev / launches, 5),
            "us_per_antidiagonal": round(1e3 * ms_ev / hops, 3),
            "note": "a chain of 2n-1 dependent anti-diagonals; the working set (3 n^2 "
                    "float64) stays in the caches, so the latency of each link (a "
                    "value handed from one row's wave to the next, or a launch), not "
                    "HBM, sets the time",
        },
    }
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the same problem (cpu_baseline)")
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            ref = oracle.two_sided_antidiagonal(y, rl, rr)
            dt = time.perf_counter() - t0
        got = Z.cpu().numpy()
        if not np.array_equal(ref, got):
            raise RuntimeError("GPU result differs from the oracle")
        line["cpu_baseline"] = {"value": round(n * n / dt, 1), "unit": "entries/s",
                                "cores": 1, "kind": "oracle",
                                "sample": f"the whole n={n} rounding ({dt:.1f} s, BLAS limited to "
                                          "one thread)"}
    print(json.dumps(line), flush=True)


def bench_w4a16(args):
    """Y = X W_hat^T with the packed 4-bit weights of the attention projection
    (4096 x 4096, g128 asymmetric), X m x 4096 bf16."""
    import numpy as np
    import torch
    import oracle
    from post_weight_quantization_syrk_amd import gptq, synth

    m, d_in, d_out, g = args.m, 4096, 4096, 128
    dev = "cuda:0"
    torch.cuda.set_device(0)
    gptq.lib()
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(d_out, d_in), dtype=np.uint8)
    scales = oracle.fp16_rne(np.exp(rng.uniform(-6.0, -2.0, size=(d_out, d_in // g))))
    zeros = rng.integers(0, 16, size=(d_out, d_in // g)).astype(np.float64)
    qw = oracle.pack_rows(codes, 4)
    s16, z16 = oracle.fp16_bits(scales), oracle.fp16_bits(zeros)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, d_in), dtype=np.float32))
    X = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    Q = torch.from_numpy(qw.astype(np.uint32).view(np.int32)).to(dev)
    S = torch.from_numpy(s16.view(np.int16)).to(dev)
    Z = torch.from_numpy(z16.view(np.int16)).to(dev)
    Y = torch.empty((m, d_out), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        gptq.gptq_w4a16_matmul(X, Q, S, Z, group_size=g, sym=False, Y=Y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        gptq.gptq_w4a16_matmul(X, Q, S, Z, group_size=g, sym=False, Y=Y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_ev = e0.elapsed_time(e1) / args.steps
    flops = 2.0 * m * d_in * d_out
    tf = flops / (ms_ev / 1e3) / 1e12
    log(f"w4a16 m={m}: {ms:.4f} ms/call ({ms_ev:.4f} ms in events), {tf:.1f} TFLOP/s")
    line = {
        "metric": f"W4A16 dequantized product, output elements/sec/GPU (m={m}, 4096x4096 g128)",
        "value": round(m * d_out / (ms / 1e3), 1),
        "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded codes, binary16 scales and zeros, X ~ N(0,1) bf16)",
        "config": {"workload": f"w4a16_m{m}_4096x4096_g128", "m": m, "d_in": d_in,
                   "d_out": d_out, "group_size": g},
        "roofline": {
            "kernel": "w4a16_kernel", "bound": "mfma", "achieved": round(tf, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "traffic": None, "algorithmic_flops_per_launch": flops,
            "avg_launch_ms": round(ms_ev, 5),
        },
    }
    if not args.no_cpu_baseline:
        rows = min(m, 256)
        x64 = synth.as_f64(xb[:rows], "bf16")
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        t0 = time.perf_counter()
        oracle.dequant_matmul(x64, qw, s16, z16, bits=4, group_size=g, sym=False)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(rows * d_out / dt, 1), "unit": "elements/s",
                                "cores": cores, "kind": "oracle",
                                "sample": f"{rows} of {m} rows of X, the whole weight "
                                          f"dequantized ({dt:.2f} s)"}
    print(json.dumps(line), flush=True)


def bench_shared(args):
    """The feed-forward gate and up projections (11008 x 4096 each, bf16) from one
    Hessian of 131072 tokens, 3-bit symmetric g64: one step = zero H, H += 2 X^T X,
    prepare, gptq_quantize_layers on both matrices, pack."""
    import torch
    from post_weight_quantization_syrk_amd import gptq, synth

    wl = synth.FFN_GATE
    dev = "cuda:0"
    torch.cuda.set_device(0)
    gptq.lib()
    d_out, d_in, n = wl.d_out, wl.d_in, wl.n_tokens
    log(f"generating inputs: X {n}x{d_in} bf16, gate and up {d_out}x{d_in} bf16")
    xb = synth.x_full(wl)
    X = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
    del xb
    Ws = [torch.from_numpy(synth.w_matrix(wl, tensor=t).view("int16")).to(dev).view(torch.bfloat16)
          for t in (0, 7)]
    H = torch.zeros((d_in, d_in), dtype=torch.float32, device=dev)
    U = torch.empty((d_in, d_in), dtype=torch.float32, device=dev)
    dead = torch.empty(d_in, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    rows = 2 * d_out
    ng = d_in // wl.group_size
    xcode = gptq.GPTQ_BF16 if wl.x_dtype == "bf16" else gptq.GPTQ_F32
    ws_h = torch.empty(gptq.gptq_hessian_workspace(d_in, n, xcode), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(gptq.gptq_prepare_workspace(d_in), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(gptq.gptq_quantize_workspace(rows, d_in, wl.block), dtype=torch.uint8,
                       device=dev)
    qweight = torch.empty((rows, d_in * wl.bits // 32), dtype=torch.int32, device=dev)
    s16 = torch.empty((rows, ng), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    stages = ["hessian", "prepare", "quantize", "pack"]
    out = {}

    def step(ev=None):
        H.zero_()
        if ev: ev[0].record(stream)
        gptq.gptq_hessian_accumulate(H, X, ws=ws_h)
        if ev: ev[1].record(stream)
        gptq.gptq_prepare_hinv(H, wl.damp, U, dead, status, ws=ws_p, check=False)
        if ev: ev[2].record(stream)
        c, sc, z, _, _ = gptq.gptq_quantize_layers(Ws, U, dead, bits=wl.bits,
                                                   group_size=wl.group_size, sym=wl.sym,
                                                   block=wl.block, want_loss=False, ws=ws_q)
        if ev: ev[3].record(stream)
        gptq.gptq_pack(c, sc, None, bits=wl.bits, group_size=wl.group_size, sym=wl.sym,
                       qweight=qweight, scales_f16=s16)
        if ev: ev[4].record(stream)
        out["c"] = c

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("factorization failed during warmup")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = {st: sum(events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps))
                / args.steps for i, st in enumerate(stages)}
    # for comparison: the two matrices quantized by separate calls
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for W in Ws:
        gptq.gptq_quantize_layer(W, U, dead, bits=wl.bits, group_size=wl.group_size, sym=wl.sym,
                                 block=wl.block, want_loss=False)
    e1.record(stream)
    torch.cuda.synchronize()
    sep_ms = e0.elapsed_time(e1)
    log(f"{ms_step:.3f} ms/step; stages " + ", ".join(f"{k} {v:.3f} ms" for k, v in stage_ms.items())
        + f"; separate quantize calls {sep_ms:.3f} ms")
    syrk_flops = float(n) * d_in * (d_in + 1)
    tf = syrk_flops / (stage_ms["hessian"] / 1e3) / 1e12
    line = {
        "metric": "GPTQ weights quantized/sec/GPU (FFN gate+up 2x11008x4096 sharing one Hessian, "
                  "131072 tokens)",
        "value": round(rows * d_in / (ms_step / 1e3), 1),
        "unit": "weights/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; stands in for a 7B model's FFN weights and calibration tokens)",
        "config": {"workload": "ffn_gate_up_2x11008x4096_131072tok_3bit_sym_g64",
                   "d_out": [d_out, d_out], "d_in": d_in, "tokens": n, "bits": wl.bits,
                   "group_size": wl.group_size, "sym": wl.sym, "block": wl.block},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "quantize_separate_calls_ms": round(sep_ms, 4),
        "roofline": {
            "kernel": "gptq_hessian_accumulate = syrk_bf16_kernel + splitk_reduce_kernel<256>",
            "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": syrk_flops,
            "avg_launch_ms": round(stage_ms["hessian"], 4),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(wl, synth, n_mats=2)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profiler", action="store_true",
                    help="skip the profiled quantize call that times the trailing update's "
                         "kernels (for runs under an external profiler)")
    ap.add_argument("--workload", choices=["gptq", "gptq2d", "w4a16", "ffn_shared"],
                    default="gptq")
    ap.add_argument("--m", type=int, default=4096, help="rows of X for --workload w4a16")
    ap.add_argument("--layer", choices=["attn7b", "l70b_sq", "l70b_up", "small"],
                    default="attn7b",
                    help="layer of the default workload: the 7B attention projection (4096 x "
                         "4096, 262144 tokens), the 70B-shaped 8192 x 8192 / 28672 x 8192 "
                         "layers (65536 tokens), or the small fp32 layer (256 x 256, 2048 "
                         "tokens with 4 outlier channels; the oracle runs it whole)")
    ap.add_argument("--n", type=int, default=1024, help="matrix size for --workload gptq2d")
    ap.add_argument("--act-order", action="store_true",
                    help="columns in activation order (gptq_act_order + the *_perm calls)")
    ap.add_argument("--static-groups", action="store_true",
                    help="with --act-order: static groups (parameters from the original W)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the quantization path runs on a single MI355X "
              "here; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "gptq2d":
        bench_gptq2d(args)
        return
    if args.workload == "w4a16":
        bench_w4a16(args)
        return
    if args.workload == "ffn_shared":
        bench_shared(args)
        return

    import torch
    from post_weight_quantization_syrk_amd import gptq, synth

    wl = {"attn7b": synth.ATTN7B, "l70b_sq": synth.L70B_SQ, "l70b_up": synth.L70B_UP,
          "small": synth.SMALL}[args.layer]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    gptq.lib()
    d_out, d_in, n = wl.d_out, wl.d_in, wl.n_tokens
    log(f"generating inputs: X {n}x{d_in} {wl.x_dtype}, W {d_out}x{d_in} {wl.w_dtype}")
    t0 = time.time()

    def to_dev(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(a.view("int16")).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    xb = synth.x_full(wl)
    X = to_dev(xb, wl.x_dtype)
    del xb
    W = to_dev(synth.w_matrix(wl), wl.w_dtype)
    log(f"inputs resident in HBM ({time.time() - t0:.1f}s)")

    H = torch.zeros((d_in, d_in), dtype=torch.float32, device=dev)
    U = torch.empty((d_in, d_in), dtype=torch.float32, device=dev)
    dead = torch.empty(d_in, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    ng = d_in // wl.group_size
    codes = torch.empty((d_out, d_in), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, ng), dtype=torch.float32, device=dev)
    zeros = torch.empty((d_out, ng), dtype=torch.float32, device=dev)
    qweight = torch.empty((d_out, d_in * wl.bits // 32), dtype=torch.int32, device=dev)
    s16 = torch.empty((d_out, ng), dtype=torch.int16, device=dev)
    z16 = torch.empty((d_out, ng), dtype=torch.int16, device=dev)
    xcode = gptq.GPTQ_BF16 if wl.x_dtype == "bf16" else gptq.GPTQ_F32
    ws_h = torch.empty(gptq.gptq_hessian_workspace(d_in, n, xcode), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(gptq.gptq_prepare_workspace(d_in), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(gptq.gptq_quantize_workspace(d_out, d_in, wl.block), dtype=torch.uint8,
                       device=dev)
    stream = torch.cuda.current_stream()
    order = args.act_order
    stages = (["hessian", "act_order", "prepare", "quantize", "pack"] if order
              else ["hessian", "prepare", "quantize", "pack"])
    if order:
        perm = torch.empty(d_in, dtype=torch.int32, device=dev)
        g_idx = torch.empty(d_in, dtype=torch.int32, device=dev)
        ws_a = torch.empty(gptq.gptq_act_order_workspace(d_in, n), dtype=torch.uint8, device=dev)
        ws_q = torch.empty(gptq.gptq_quantize_perm_workspace(d_out, d_in, wl.block),
                           dtype=torch.uint8, device=dev)

    def step(ev=None):
        k = 0
        H.zero_()
        if ev: ev[k].record(stream); k += 1
        gptq.gptq_hessian_accumulate(H, X, ws=ws_h)
        if ev: ev[k].record(stream); k += 1
        if order:
            gptq.gptq_act_order(X, d_in, perm=perm, ws=ws_a)
            if ev: ev[k].record(stream); k += 1
            gptq.gptq_prepare_hinv_perm(H, perm, wl.damp, U, dead, status, ws=ws_p, check=False)
            if ev: ev[k].record(stream); k += 1
            gptq.gptq_quantize_layer_perm(W, U, dead, perm, static_groups=args.static_groups,
                                          bits=wl.bits, group_size=wl.group_size, sym=wl.sym,
                                          block=wl.block, codes=codes, scales=scales, zeros=zeros,
                                          g_idx=g_idx, want_loss=False, ws=ws_q)
        else:
            gptq.gptq_prepare_hinv(H, wl.damp, U, dead, status, ws=ws_p, check=False)
            if ev: ev[k].record(stream); k += 1
            gptq.gptq_quantize_layer(W, U, dead, bits=wl.bits, group_size=wl.group_size,
                                     sym=wl.sym, block=wl.block, codes=codes, scales=scales,
                                     zeros=zeros, want_loss=False, ws=ws_q)
        if ev: ev[k].record(stream); k += 1
        gptq.gptq_pack(codes, scales, zeros, bits=wl.bits, group_size=wl.group_size, sym=wl.sym,
                       qweight=qweight, scales_f16=s16, zeros_f16=z16)
        if ev: ev[k].record(stream); k += 1

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("factorization failed during warmup")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    stage_ms = {s: sum(events[k][i].elapsed_time(events[k][i + 1]) for k in range(args.steps))
                / args.steps for i, s in enumerate(stages)}
    if int(status.item()) != 0:
        raise RuntimeError("factorization failed")
    log(f"{ms_step:.3f} ms/step; stages " + ", ".join(f"{k} {v:.3f} ms" for k, v in stage_ms.items()))

    weights = d_out * d_in
    value = weights / (ms_step / 1e3)
    syrk_flops = float(n) * d_in * (d_in + 1)
    trail_flops = float(d_out) * d_in * (d_in - wl.block)
    syrk_tflops = syrk_flops / (stage_ms["hessian"] / 1e3) / 1e12
    # bf16 X: the bf16 matrix peak; fp32 X: the fp32 matrix peak
    syrk_peak = PEAK_BF16_TFLOPS if wl.x_dtype == "bf16" else PEAK_FP32_TFLOPS
    syrk_kernel = "syrk_bf16_kernel" if wl.x_dtype == "bf16" else "syrk_f32_kernel"
    roofline = {
        "kernel": (f"gptq_hessian_accumulate = {syrk_kernel} + splitk_reduce_kernel "
                   f"(H += 2 X^T X)"),
        "timing": ("HIP events on the library's stream around the whole call (both kernels), "
                   "averaged over the timed steps"),
        "bound": "mfma",
        "achieved": round(syrk_tflops, 2),
        "peak": syrk_peak,
        "unit": "TFLOP/s",
        "frac": round(syrk_tflops / syrk_peak, 4),
        "traffic": traffic_from_profile() if args.layer == "attn7b" else None,
        "algorithmic_flops_per_launch": syrk_flops,
        "avg_launch_ms": round(stage_ms["hessian"], 4),
    }
    upd_tflops = (syrk_flops + trail_flops) / ((stage_ms["hessian"] + stage_ms["quantize"]) / 1e3) / 1e12
    rl = roofline_bound_ms(wl)
    # the far trailing update's own rate: its kernels (operand split, which
    # shares a launch with the column loop's diagonal blocks, + far updates)
    # timed by the profiler over one more quantize call
    trail_ms = None
    if not order and d_in > wl.block and not args.no_profiler:
        try:
            trail_ms = device_kernel_ms(
                lambda: gptq.gptq_quantize_layer(W, U, dead, bits=wl.bits,
                                                 group_size=wl.group_size, sym=wl.sym,
                                                 block=wl.block, codes=codes, scales=scales,
                                                 zeros=zeros, want_loss=False, ws=ws_q),
                ("trailing3_kernel", "uprep_kernel"))
        except Exception as e:  # the profiler is optional here
            log(f"trailing kernels not timed: {e}")
    trailing = None
    if trail_ms:
        far_flops = far_update_flops(d_out, d_in, wl.block)
        t_tf = far_flops / (trail_ms / 1e3) / 1e12
        trailing = {"kernels": "uprep_kernel (U^T split into parts, with the column loop's "
                               "diagonal blocks of U and W's working copy in the same launch) "
                               "+ trailing3_kernel (far updates; the near updates within a "
                               "group run inside colloop_kernel)",
                    "ms": round(trail_ms, 4), "algorithmic_flops": far_flops,
                    "achieved": round(t_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(t_tf / PEAK_BF16_TFLOPS, 4),
                    "timing": "torch profiler device times over one quantize call"}
    line = {
        "metric": f"GPTQ weights quantized/sec/GPU ({d_out}x{d_in}, {n} tokens)",
        "value": round(value, 1),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.x_dtype,
        "data": {"attn7b": "synthetic (seeded; stands in for a 7B model's weights and 128x2048 "
                           "calibration tokens)",
                 "small": "synthetic (seeded; fp32 layer with 4 outlier input channels x20)"}.get(
                     args.layer, "synthetic (seeded; stands in for a 70B model's layer weights and "
                                 "65536 calibration tokens)"),
        "config": {"workload": wl.name, "d_out": d_out, "d_in": d_in, "tokens": n,
                   "bits": wl.bits, "group_size": wl.group_size, "sym": wl.sym,
                   "block": wl.block, "damp": wl.damp, "act_order": bool(order),
                   "static_groups": bool(order and args.static_groups)},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "secondary": {"metric": "SYRK+update TFLOP/s", "value": round(upd_tflops, 2),
                      "unit": "TFLOP/s",
                      "note": "(n d(d+1) + d_out d_in (d_in-128)) / (hessian + quantize stage "
                              "time); the quantize stage also holds the column loop"},
        "roofline": roofline,
        "e2e_roofline_frac": round(rl["total"] / ms_step, 4),
        "roofline_bound_ms": {k: round(v, 4) for k, v in rl.items()},
        "trailing_gemm": trailing,
    }
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(wl, synth, act_order=order,
                                            static_groups=bool(order and args.static_groups))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

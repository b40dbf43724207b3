#!/usr/bin/env python3
"""Benchmark of the ConvRot W8A8 linear on one MI355X.

Headline workload: one ConvRot W8A8 linear at the MLP up/gate shape
M=2048 tokens, K=4096, N=12288, group 256 (bf16 activations N(0,1) with 1 %
outlier channels x20, int8 per-row weights).  One step = one call of
convrot_w8a8_linear (rotate + quantize the activations, int8 GEMM, bf16
epilogue) with all inputs resident in HBM.  Steps cycle through several
buffer sets whose total exceeds twice the 256 MB Infinity Cache, so every
step reads its operands from HBM.

Order: the per-kernel timings of the roofline (GEMM alone, rotate-quantize
alone, each after its own 50 ms of warm-up launches) run first, then the W
untimed warm-up steps and the K timed steps of the headline, then seven
more runs of at least 10 ms of steps (median and min), the parity check
against the oracle, and the extras.

Prints ONE JSON line on stdout: TOPS (2*M*N*K per step / step time), plus
tokens/s, the GEMM kernel's roofline position (timed live with HIP events on
the launch stream), the rotate-quantize kernel's HBM bandwidth (also fused
with the preceding RMSNorm), the parity of the benchmarked buffers against
the oracle (every activation code of the input), and the CPU oracle timed
on a bounded sample on this host (all threads and one, per stage).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-extras]
                       [--profile {gemm,gemm_tiles,gemm_bf16,rq,rq_large,rq_g16,rmsnorm_rq,copy,linear}]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, ops/s * 1e-12
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20
M, K, N, GROUP = 2048, 4096, 12288, 256


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text):
    """Source text without comments and blank lines: what the compiler sees
    of a kernel, so that editing a comment does not retire its counters."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


GEMM_SOURCES = ["w8a8_quantized_linear_amd/csrc/gemm_i8.hip"]
RQ_SOURCES = ["w8a8_quantized_linear_amd/csrc/rotate_quant.hip",
              "w8a8_quantized_linear_amd/csrc/rotate_quant_fast.hip"]
# Rotate-quantize passes whose HBM fraction is the graded figure: the
# 34 x 256-token stack's activations (K 4096 and the down projection's
# K 12288) and the MLP down projection's input at M=2048.
RQ_PASSES = [(8704, 4096), (8704, 12288), (2048, 12288)]
# The stack's RMSNorm input (hidden size 4096), normalised and quantized in one pass.
RMSNORM_PASS = (8704, 4096)
# A group-16 pass at the vision MLP width (4304 is not a multiple of 256).
RQ_G16_PASS = (16384, 4304)


def load_traffic(name, sources):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(sources):
        return None
    return rec.get("traffic_bytes_per_launch")


def load_mfma_busy():
    """MFMA busy per SIMD over the engine cycles for the headline GEMM
    (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over SQ_CYCLES / 32 engines),
    from the committed rocprofv3 counter summary of every tile plan, or None
    when the GEMM source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "gemm_i8_tiles_lds_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(GEMM_SOURCES):
        return None
    for r in rec.get("records", []):
        if (r["M"], r["N"], r["K"], r["weight_bits"]) == (M, N, K, 8):
            return round(r["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (r["SQ_CYCLES"] / 32), 4)
    return None


class Timer:
    """Average duration of repeated launches, from HIP events recorded on the
    current stream (the one the library launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, reps, warm=3, warm_s=0.05):
        """Seconds per launch of fn over reps launches, after warm-up
        launches for at least warm_s seconds: the device needs tens of
        milliseconds of load to reach its steady clock (after an idle spell,
        e.g. the host-side parity check, a pass timed at once measured up to
        20 % slower)."""
        torch = self.torch
        t0 = time.perf_counter()
        i = 0
        while True:
            for _ in range(warm):
                fn(i)
                i += 1
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= warm_s:
                break
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(reps):
            fn(i)
        e.record()
        e.synchronize()
        return s.elapsed_time(e) / 1e3 / reps  # seconds per launch


def build_sets(torch, cr, wl, nsets):
    x, w = wl.config_inputs("C3u")
    dev = torch.device("cuda")
    w_dev = torch.from_numpy(w).to(dev)
    wq0, ws0 = cr.quantize_weight(w_dev, group=GROUP, bits=8)
    del w_dev
    x0 = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    sets = []
    for i in range(nsets):
        xi = x0.clone()
        wqi = wq0.clone()
        wsi = ws0.clone()
        yi = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsp = cr.workspace(M, K, dev)
        sets.append((xi, wqi, wsi, yi, wsp))
    return x, w, sets


def host_cpu():
    """The host the CPU baseline runs on: model name, logical CPUs, and the
    CPUs this process may run on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_allowed": allowed}


def cpu_baseline(x, w, target_s=12.0, target_1t_s=3.0):
    """The CPU oracle as it stands, on the host cores: rotate+quantize a
    sample of tokens, naive int32 GEMM against all N rows, bf16 epilogue.
    Weight preparation is offline (not timed), as on the GPU side.  The
    value is the whole linear on all threads; the record adds the time of
    each stage on the same sample (rotation alone, quantization as the
    rest of the rotate-quantize call, GEMM, epilogue) and the whole linear
    on one thread over a smaller sample (the cost is linear in tokens)."""
    import oracle
    from w8a8_quantized_linear_amd import workloads as wl
    wq, ws = oracle.quantize_weight_i8(w, GROUP)
    threads = oracle.num_threads()
    ms = 16
    t0 = time.perf_counter()
    oracle.w8a8_linear(np.ascontiguousarray(x[:ms]), wq, ws, GROUP)
    t_probe = time.perf_counter() - t0
    ms = int(min(M, max(16, ms * target_s / max(t_probe, 1e-3))))
    # repeat the sample until about target_s of CPU work has been timed
    reps = max(1, min(8, int(round(target_s / max(t_probe * ms / 16, 1e-3)))))
    xs = np.ascontiguousarray(x[:ms])
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.w8a8_linear(xs, wq, ws, GROUP)
    t = (time.perf_counter() - t0) / reps

    # Stages, once each, on the same sample and threads.
    stages = {}
    x64 = wl.bf16_bits_to_float(xs).astype(np.float64)
    t0 = time.perf_counter()
    oracle.rotate_rows(x64, GROUP)
    stages["rotation"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    xq, xsc = oracle.rotate_quant(xs, GROUP)
    stages["quantize"] = max(0.0, time.perf_counter() - t0 - stages["rotation"])
    t0 = time.perf_counter()
    acc = oracle.gemm_i8(xq, wq)
    stages["gemm"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.epilogue(acc, xsc, ws)
    stages["epilogue"] = time.perf_counter() - t0

    # One thread, on a smaller sample.
    oracle.set_num_threads(1)
    try:
        m1 = 2
        t0 = time.perf_counter()
        oracle.w8a8_linear(np.ascontiguousarray(x[:m1]), wq, ws, GROUP)
        tp = time.perf_counter() - t0
        m1 = int(min(ms, max(2, m1 * target_1t_s / max(tp, 1e-3))))
        t0 = time.perf_counter()
        oracle.w8a8_linear(np.ascontiguousarray(x[:m1]), wq, ws, GROUP)
        t1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    return {
        "value": 2.0 * ms * N * K / t / 1e12,
        "unit": "TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {ms} of {M} tokens, full K={K} x N={N} (GEMM cost is linear in tokens), "
                  f"{reps} repetition(s), {t * reps:.1f} s in total; weights quantized by the oracle "
                  f"beforehand (untimed)",
        "tokens_per_s": ms / t,
        "seconds": t * reps,
        "host": host_cpu(),
        "threads": threads,
        "compile_flags": " ".join(["gcc", *oracle.CFLAGS]),
        "stage_seconds": {k: round(v, 4) for k, v in stages.items()},
        "stage_sample_tokens": ms,
        "one_thread": {"tokens": m1, "seconds": round(t1, 3), "tokens_per_s": m1 / t1,
                       "tops": 2.0 * m1 * N * K / t1 / 1e12},
    }


def check_parity(torch, cr, x, w, y_dev, xq_dev, xs_dev, wq_dev, ws_dev):
    """Parity of the benchmarked buffers against the oracle: every activation
    code and scale of the input (M x K), the weight codes and scales of 1024
    sampled rows, the int32 accumulators of the GPU's own codes on 64 tokens
    x 1024 rows (exact or not), and the bf16 output on those pairs against
    the oracle's (relative L2).  The oracle decides codes on the exact
    rotation, so a few codes per million may differ by one at rounding
    boundaries."""
    import oracle
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(M, 64, replace=False))
    rows = np.sort(rng.choice(N, 1024, replace=False))
    xq_ref, xs_ref = oracle.rotate_quant(np.ascontiguousarray(x), GROUP)
    wq_ref, ws_ref = oracle.quantize_weight_i8(np.ascontiguousarray(w[rows]), GROUP)
    y_ref = oracle.epilogue(oracle.gemm_i8(xq_ref[toks], wq_ref), xs_ref[toks], ws_ref)
    y = y_dev.view(torch.int16).cpu().numpy().view(np.uint16)[np.ix_(toks, rows)]
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xq_g = xq_dev.cpu().numpy()
    xs_g = xs_dev.cpu().numpy()
    wq_g = wq_dev.cpu().numpy()[rows]
    ws_g = ws_dev.cpu().numpy()[rows]
    # The GEMM on the GPU's own codes, all N, accumulators kept.
    acc = torch.empty((M, N), dtype=torch.int32, device=xq_dev.device)
    _ok(cr, cr.convrot_gemm_i8(xq_dev, xs_dev, wq_dev, 8, ws_dev, M, N, K, acc, None))
    torch.cuda.synchronize()
    acc_g = acc.cpu().numpy()[np.ix_(toks, rows)]
    del acc
    dx = xq_g.astype(np.int16) - xq_ref
    dw = wq_g.astype(np.int16) - wq_ref
    rel = lambda a, b: float(np.max(np.abs(a.astype(np.float64) - b) / np.where(b == 0, 1, np.abs(b))))
    return {
        "sample": f"activation codes: all {M} x {K}; weight codes: {rows.size} rows x {K}; "
                  f"output and accumulators: {toks.size} tokens x {rows.size} rows",
        "rel_l2": float(np.linalg.norm(f(y) - f(y_ref)) / np.linalg.norm(f(y_ref))),
        "code_mismatch_frac": float(np.count_nonzero(dx)) / dx.size,
        "code_mismatch_count": int(np.count_nonzero(dx)),
        "code_max_abs_diff": int(np.abs(dx).max()),
        "weight_code_mismatch_frac": float(np.count_nonzero(dw)) / dw.size,
        "weight_code_mismatch_count": int(np.count_nonzero(dw)),
        "scale_max_rel_diff": rel(xs_g, xs_ref),
        "weight_scale_max_rel_diff": rel(ws_g, ws_ref),
        "acc_exact": bool(np.array_equal(acc_g, oracle.gemm_i8(xq_g[toks], wq_g))),
    }


def extras_w4a8(torch, cr, wl, timer):
    """The int4-weight linear, M=4096 K=4096 N=12288, operands cycled through
    buffer sets larger than 2x the MALL."""
    cfg = wl.CONFIGS["C5"]
    lin = cfg.linears[0]
    x, w = wl.config_inputs("C5")
    dev = torch.device("cuda")
    wq4, ws = cr.quantize_weight(torch.from_numpy(w).to(dev), bits=4)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    per = cfg.M * lin.K * 2 + lin.N * lin.K // 2 + 2 * cfg.M * lin.N
    n = max(2, -(-2 * MALL_BYTES // per) + 1)
    sets = [(xd.clone(), wq4.clone(), ws.clone(), torch.empty((cfg.M, lin.N), dtype=torch.bfloat16, device=dev),
             cr.workspace(cfg.M, lin.K, dev)) for _ in range(n)]
    t = timer.time(lambda i: cr.w4a8_linear(*sets[i % n][:3], out=sets[i % n][3], ws=sets[i % n][4]), 100)
    ops = 2.0 * cfg.M * lin.N * lin.K
    del sets
    return {"workload": "W4A8 M=4096 K=4096 N=12288", "tops": ops / t / 1e12, "us": t * 1e6,
            "tokens_per_s": cfg.M / t, "pct_int8_peak": ops / t / 1e12 / PEAK_INT8_TOPS, "buffer_sets": n}


def extras_configs(torch, cr, wl, timer):
    """The other single-linear workloads, one convrot_w8a8_linear call per
    launch: M=16 K=512 N=256 (latency-bound; its buffers stay in the MALL),
    M=512 K=4096 N=4096, and the MLP down shape M=2048 K=12288 N=4096 with
    operands cycled through buffer sets larger than 2x the MALL."""
    dev = torch.device("cuda")
    res = {}
    for key in ("C1", "C2", "C3d"):
        cfg = wl.CONFIGS[key]
        lin = cfg.linears[0]
        x, w = wl.config_inputs(key)
        wq, ws = cr.quantize_weight(torch.from_numpy(w).to(dev), group=GROUP, bits=8)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        per = cfg.M * lin.K * 2 + lin.N * lin.K + 2 * cfg.M * lin.N
        n = min(64, max(2, -(-2 * MALL_BYTES // per) + 1))
        sets = [(xd.clone(), wq.clone(), ws.clone(), torch.empty((cfg.M, lin.N), dtype=torch.bfloat16, device=dev),
                 cr.workspace(cfg.M, lin.K, dev)) for _ in range(n)]
        t = timer.time(lambda i: cr.w8a8_linear(*sets[i % n][:3], group=GROUP, out=sets[i % n][3],
                                                ws=sets[i % n][4]), 200)
        ops = 2.0 * cfg.M * lin.N * lin.K
        res[key] = {"M": cfg.M, "K": lin.K, "N": lin.N, "us": round(t * 1e6, 2), "tops": round(ops / t / 1e12, 1),
                    "tokens_per_s": round(cfg.M / t, 1), "buffer_sets": n}
        del sets, wq, ws, xd
    return res


def extras_shards(torch, cr, wl, timer, x, w):
    """One GPU's share of the headline linear under 8-way sharding, from
    the headline's own inputs (cold buffer sets, one convrot_w8a8_linear
    per launch): tensor-parallel over N (all 2048 tokens, 1536 of the 12288
    weight rows) and data-parallel over M (256 of the 2048 tokens, all
    rows).  Neither needs any exchange for the linear itself."""
    dev = torch.device("cuda")
    res = {}
    for key, m0, m1, n0, n1 in (("tp8_N1536", 0, M, 0, N // 8), ("dp8_M256", 0, M // 8, 0, N)):
        xs = np.ascontiguousarray(x[m0:m1])
        wsl = np.ascontiguousarray(w[n0:n1])
        mm, nn = m1 - m0, n1 - n0
        wq, ws = cr.quantize_weight(torch.from_numpy(wsl).to(dev), group=GROUP, bits=8)
        xd = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
        per = mm * K * 2 + nn * K + 2 * mm * nn
        n = min(64, max(2, -(-2 * MALL_BYTES // per) + 1))
        sets = [(xd.clone(), wq.clone(), ws.clone(), torch.empty((mm, nn), dtype=torch.bfloat16, device=dev),
                 cr.workspace(mm, K, dev)) for _ in range(n)]
        t = timer.time(lambda i: cr.w8a8_linear(*sets[i % n][:3], group=GROUP, out=sets[i % n][3],
                                                ws=sets[i % n][4]), 200)
        ops = 2.0 * mm * nn * K
        res[key] = {"M": mm, "K": K, "N": nn, "us": round(t * 1e6, 2), "tops": round(ops / t / 1e12, 1),
                    "tokens_per_s": round(mm / t, 1), "buffer_sets": n}
        del sets, wq, ws, xd
    return res


def _ok(cr, rc):
    if rc != 0:
        raise RuntimeError(f"convrot status {rc}: {cr.convrot_status_string(rc)}")


def extras_stack(torch, cr, wl, timer):
    """32-layer synthetic decoder linear stack at M=8704, weights generated on
    device.  Three ways of running each layer's seven linears:
    - per linear: 7 rotate-quantize passes and 7 GEMM launches;
    - shared input: q/k/v and gate/up each share one rotate-quantize and one
      multi-output GEMM launch (4 passes, 4 launches);
    - shared input with the RMSNorm fused: as above, with the norms in front
      of q/k/v and gate/up folded into their rotate-quantize passes (so this
      variant does the two norms' work too)."""
    cfg = wl.CONFIGS["C4"]
    dev = torch.device("cuda")
    acts = [torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16) for a in wl.stack_activations()]
    layers = []
    for layer in range(cfg.layers):
        ws_ = []
        for li, lin in enumerate(cfg.linears):
            wd = wl.make_weight_device(lin.N, lin.K, wl.C4_WEIGHT_SEED_BASE + layer * 16 + li, dev)
            ws_.append(cr.quantize_weight(wd))
            del wd
        layers.append(ws_)
    outs = {lin.name: torch.empty((cfg.M, lin.N), dtype=torch.bfloat16, device=dev) for lin in cfg.linears}
    wsp = cr.workspace(cfg.M, 12288, dev)
    nws = [torch.from_numpy(wl.make_norm_weight(4096, 41, seed=s)).to(dev) for s in (4, 6)]
    xq = torch.empty((cfg.M, 4096), dtype=torch.int8, device=dev)
    xs = torch.empty((cfg.M,), dtype=torch.float32, device=dev)
    ops = 0.0
    for lin in cfg.linears:
        ops += 2.0 * cfg.M * lin.N * lin.K
    ops *= cfg.layers
    names = [lin.name for lin in cfg.linears]
    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

    def per_linear(_):
        for layer in range(cfg.layers):
            for li, lin in enumerate(cfg.linears):
                wq, wsc = layers[layer][li]
                cr.w8a8_linear(acts[wl.C4_INPUT_OF[lin.name]], wq, wsc, out=outs[lin.name], ws=wsp)

    def shared(_):
        for layer in range(cfg.layers):
            for gi, grp in enumerate(groups):
                cr.linear_multi(acts[gi], [layers[layer][names.index(n)] for n in grp],
                                outs=[outs[n] for n in grp], ws=wsp)

    def fused_norm(_):
        for layer in range(cfg.layers):
            for gi, grp in enumerate(groups):
                a = acts[gi]
                M, K = a.shape
                if gi in (0, 2):
                    _ok(cr, cr.convrot_rmsnorm_rotate_quant(a, nws[gi // 2], 1e-6, M, K, GROUP, xq, xs))
                    desc = [(layers[layer][names.index(n)][0], layers[layer][names.index(n)][1],
                             outs[n].shape[1], None, outs[n]) for n in grp]
                    _ok(cr, cr.convrot_gemm_i8_multi(xq, xs, 8, M, K, desc))
                else:
                    wq, wsc = layers[layer][names.index(grp[0])]
                    cr.w8a8_linear(a, wq, wsc, out=outs[grp[0]], ws=wsp)

    res = {"workload": "32-layer linear stack, M=8704 (34 x 256 tokens), 224 W8A8 linears"}
    for key, fn in (("per_linear", per_linear), ("shared_input", shared), ("shared_input_fused_norm", fused_norm)):
        t = timer.time(fn, 3, warm=1)
        res[key] = {"ms_per_pass": t * 1e3, "tokens_per_s": cfg.M / t, "tops": ops / t / 1e12,
                    "pct_int8_peak": ops / t / 1e12 / PEAK_INT8_TOPS}
    res.update(res["per_linear"])
    return res


def extras_dequant(torch, cr, wl, timer):
    """Weight-only (dequant) path at the headline shape: the bf16 GEMM with
    the dequantized weight resident, the dequantize kernel alone, and both
    (convrot_dequant_linear); torch's bf16 matmul (the vendor library) on the
    same buffers for context.  Operands cycle past 2x the MALL."""
    dev = torch.device("cuda")
    per = 2 * (M * K + N * K + M * N)
    n = max(2, -(-2 * MALL_BYTES // per) + 1)
    g = torch.Generator(device=dev).manual_seed(77)
    xs = [torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16) for _ in range(n)]
    wqs, wss = [], []
    for i in range(n):
        w = torch.randn((N, K), generator=g, device=dev) * 0.02
        wq, wsc = cr.quantize_weight(w)
        wqs.append(wq)
        wss.append(wsc)
        del w
    whs = [cr.dequantize_weight(wqs[i], wss[i], K) for i in range(n)]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    wsp = torch.empty((cr.convrot_dequant_workspace_size(N, K),), dtype=torch.uint8, device=dev)
    flops = 2.0 * M * N * K
    t_g = timer.time(lambda i: cr.gemm_bf16(xs[i % n], whs[i % n], out=ys[i % n]), 50)
    t_d = timer.time(lambda i: cr.convrot_dequantize_weight(wqs[i % n], 8, wss[i % n], N, K, GROUP, whs[i % n]), 50)
    t_l = timer.time(lambda i: cr.dequant_linear(xs[i % n], wqs[i % n], wss[i % n], out=ys[i % n], ws=wsp), 50)
    t_t = timer.time(lambda i: torch.matmul(xs[i % n], whs[i % n].t(), out=ys[i % n]), 50)
    dq_bytes = N * K + 4 * N + 2 * N * K
    res = {"workload": "weight-only path, M=2048 K=4096 N=12288 (bf16 activations, int8 weights dequantized to bf16)",
           "gemm_bf16": {"us": round(t_g * 1e6, 2), "tflops": round(flops / t_g / 1e12, 1),
                         "frac": round(flops / t_g / 1e12 / PEAK_BF16_TFLOPS, 4), "peak": PEAK_BF16_TFLOPS},
           "dequantize_weight": {"us": round(t_d * 1e6, 2), "bytes": dq_bytes,
                                 "achieved_gbs": round(dq_bytes / t_d / 1e9, 1)},
           "dequant_linear": {"us": round(t_l * 1e6, 2), "tflops": round(flops / t_l / 1e12, 1)},
           "torch_matmul_bf16": {"us": round(t_t * 1e6, 2), "tflops": round(flops / t_t / 1e12, 1)}}
    del xs, wqs, wss, whs, ys, wsp
    return res


def extras_vision(torch, cr, wl, timer):
    """Group-16 linears of a ConvRot vision block (widths 1152 and 4304 are
    not multiples of 256): qkv 1152->3456, proj 1152->1152, fc1 1152->4304,
    fc2 4304->1152 at M=4096 patches, each with its own group-16
    rotate-quantize; plus the group-16 rotate-quantize alone at M=16384."""
    dev = torch.device("cuda")
    Mv = 4096
    lins = (("qkv", 1152, 3456), ("proj", 1152, 1152), ("fc1", 1152, 4304), ("fc2", 4304, 1152))
    g = torch.Generator(device=dev).manual_seed(16)
    acts = {k: torch.randn((Mv, k), generator=g, device=dev).to(torch.bfloat16) for k in (1152, 4304)}
    ws_, outs = [], []
    for name, k, n in lins:
        w = torch.randn((n, k), generator=g, device=dev) * 0.02
        ws_.append(cr.quantize_weight(w, group=16))
        outs.append(torch.empty((Mv, n), dtype=torch.bfloat16, device=dev))
    wsp = cr.workspace(Mv, 4304, dev)
    ops = sum(2.0 * Mv * k * n for _, k, n in lins)

    def block(_):
        for (name, k, n), (wq, wsc), y in zip(lins, ws_, outs):
            cr.w8a8_linear(acts[k], wq, wsc, group=16, out=y, ws=wsp)

    t_b = timer.time(block, 30)
    Mr, Kr = RQ_G16_PASS
    per = Mr * (3 * Kr + 4)
    n = max(2, -(-2 * MALL_BYTES // per) + 1)
    xs = [torch.randn((Mr, Kr), generator=g, device=dev).to(torch.bfloat16) for _ in range(n)]
    qs = [torch.empty((Mr, Kr), dtype=torch.int8, device=dev) for _ in range(n)]
    ss = [torch.empty((Mr,), dtype=torch.float32, device=dev) for _ in range(n)]
    t_r = timer.time(lambda i: cr.convrot_rotate_quant(xs[i % n], Mr, Kr, 16, qs[i % n], ss[i % n]), 200, warm=50)
    res = {"workload": "vision block linears, group 16, M=4096 patches (qkv, proj, fc1, fc2)",
           "us_per_block": round(t_b * 1e6, 1), "tops": round(ops / t_b / 1e12, 1),
           "rotate_quant_g16": {"M": Mr, "K": Kr, "us": round(t_r * 1e6, 2), "bytes": per,
                                "achieved_gbs": round(per / t_r / 1e9, 1),
                                "frac": round(per / t_r / 1e9 / PEAK_HBM_GBS, 4),
                                "traffic": load_traffic("rotate_quant_g16_M16384_K4304", RQ_SOURCES)}}
    del xs, qs, ss, acts, ws_, outs, wsp
    return res


def _stream_probe():
    """The same-bytes streaming helper (tests/gpu_probe/stream_rq.hip, built
    by __graft_entry__.build), or None."""
    import ctypes
    path = os.path.join(ROOT, "tests", "gpu_probe", "libstream_rq.so")
    if not os.path.exists(path):
        return None
    fn = ctypes.CDLL(path).stream_rq_launch
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                   ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def stream_same_bytes(torch, xs, m, k, timer):
    """The same-bytes streaming helper over the input buffers xs (bf16
    [m, k] each, cycled), into output buffers of its own: the faster of its
    two launch shapes, or None when the helper is not built."""
    probe = _stream_probe()
    if probe is None:
        return None
    dev = torch.device("cuda")
    n = len(xs)
    per = m * (3 * k + 4)
    qs = [torch.empty((m, k), dtype=torch.int8, device=dev) for _ in range(n)]
    ss = [torch.empty((m,), dtype=torch.float32, device=dev) for _ in range(n)]
    blocks = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream().cuda_stream

    def sweep(mode):
        def run(i):
            rc = probe(xs[i % n].data_ptr(), qs[i % n].data_ptr(), ss[i % n].data_ptr(), m, k, mode, blocks, stream)
            if rc:
                raise RuntimeError(f"stream_rq_launch: {rc}")
        return timer.time(run, 200, warm=50)

    ts = {"chunk_per_thread": sweep(0), f"resident_grid_{blocks}": sweep(1)}
    best = min(ts, key=ts.get)
    del qs, ss
    return {"us": round(ts[best] * 1e6, 2), "bytes": per, "shape": best,
            "achieved": round(per / ts[best] / 1e9, 1), "frac": round(per / ts[best] / 1e9 / PEAK_HBM_GBS, 4),
            "us_by_shape": {a: round(b * 1e6, 2) for a, b in ts.items()}}


def rq_passes(torch, cr, timer):
    """Rotate-quantize bandwidth on the large passes, each cycled through
    enough buffer sets to exceed 2x the MALL (inputs N(0,1) bf16).  Beside
    each, two plain streaming passes over the same input buffers:
    - torch's vectorized elementwise kernel (x + 0 on the bf16 bits read as
      int32 words) into a buffer of the same size, 2 bytes read and 2
      written per value with no arithmetic: the rate a plain elementwise
      kernel reaches at that size;
    - the same-bytes helper (tests/gpu_probe/stream_rq.hip): exactly the
      pass's 3K + 4 bytes per row, 16-byte nontemporal loads and stores as in
      the quantizer, no arithmetic, one 16-value chunk per thread or a
      resident grid walking the chunks; the faster of the two is reported."""
    dev = torch.device("cuda")
    res = []
    for (m, k) in RQ_PASSES:
        per = m * (3 * k + 4)
        n = max(2, -(-2 * MALL_BYTES // per) + 1)
        g = torch.Generator(device=dev).manual_seed(m + k)
        xs = [torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16) for _ in range(n)]
        qs = [torch.empty((m, k), dtype=torch.int8, device=dev) for _ in range(n)]
        ss = [torch.empty((m,), dtype=torch.float32, device=dev) for _ in range(n)]
        t = timer.time(lambda i: cr.convrot_rotate_quant(xs[i % n], m, k, GROUP, qs[i % n], ss[i % n]), 200, warm=50)
        del qs, ss
        ys = [torch.empty((m, k // 2), dtype=torch.int32, device=dev) for _ in range(n)]
        t_ref = timer.time(lambda i: torch.add(xs[i % n].view(torch.int32), 0, out=ys[i % n]), 200, warm=50)
        ref_bytes = 4 * m * k
        rec = {"M": m, "K": k, "us": round(t * 1e6, 2), "bytes": per,
               "achieved": round(per / t / 1e9, 1), "frac": round(per / t / 1e9 / PEAK_HBM_GBS, 4),
               "elementwise_same_input": {"us": round(t_ref * 1e6, 2), "bytes": ref_bytes,
                                          "achieved": round(ref_bytes / t_ref / 1e9, 1)}}
        del ys
        same = stream_same_bytes(torch, xs, m, k, timer)
        if same is not None:
            rec["stream_same_bytes"] = same
        res.append(rec)
        del xs
    return res


def rmsnorm_rq_pass(torch, cr, wl, timer):
    """Fused RMSNorm + rotate-quantize on the decoder stack's norm input
    (M=8704 tokens, K=4096), with and without the optional bf16 norm output,
    beside the plain rotate-quantize of the same shape; buffer sets cycled
    past 2x the MALL as in rq_passes."""
    dev = torch.device("cuda")
    m, k = RMSNORM_PASS
    per = {"fused": m * (3 * k + 4) + 4 * k, "fused_y": m * (5 * k + 4) + 4 * k, "plain": m * (3 * k + 4)}
    n = max(2, -(-2 * MALL_BYTES // per["fused_y"]) + 1)
    g = torch.Generator(device=dev).manual_seed(m + k + 1)
    xs = [torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16) for _ in range(n)]
    qs = [torch.empty((m, k), dtype=torch.int8, device=dev) for _ in range(n)]
    ss = [torch.empty((m,), dtype=torch.float32, device=dev) for _ in range(n)]
    ys = [torch.empty((m, k), dtype=torch.bfloat16, device=dev) for _ in range(n)]
    nw = torch.from_numpy(wl.make_norm_weight(k, k // 100, seed=4)).to(dev)
    runs = {
        "fused": lambda i: cr.convrot_rmsnorm_rotate_quant(xs[i % n], nw, 1e-6, m, k, GROUP, qs[i % n], ss[i % n]),
        "fused_y": lambda i: cr.convrot_rmsnorm_rotate_quant(xs[i % n], nw, 1e-6, m, k, GROUP, qs[i % n],
                                                             ss[i % n], ys[i % n]),
        "plain": lambda i: cr.convrot_rotate_quant(xs[i % n], m, k, GROUP, qs[i % n], ss[i % n]),
    }
    res = {"M": m, "K": k, "bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "traffic": load_traffic("rmsnorm_rotate_quant_M8704_K4096", RQ_SOURCES)}
    for name, fn in runs.items():
        t = timer.time(fn, 200, warm=50)
        res[name] = {"us": round(t * 1e6, 2), "bytes": per[name], "achieved": round(per[name] / t / 1e9, 1),
                     "frac": round(per[name] / t / 1e9 / PEAK_HBM_GBS, 4)}
    del xs, qs, ss, ys
    return res


def _mfma_probe(torch):
    """The MFMA-rate helper (tests/gpu_probe/mfma_rate.hip, built by
    __graft_entry__.build): a launcher for blocks x 256 threads."""
    import ctypes
    path = os.path.join(ROOT, "tests", "gpu_probe", "libmfma_rate.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    for fn in (lib.mfma_rate_launch, lib.mfma_rate_launch_bf16):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")

    def run(iters, bf16=False):
        fn = lib.mfma_rate_launch_bf16 if bf16 else lib.mfma_rate_launch
        rc = fn(blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc:
            raise RuntimeError(f"mfma rate launch failed: {rc}")
    return run, out, blocks


MFMA_LOOP_ITERS = 10000


def mfma_loop(torch, timer):
    """Context for the roofline: the int8 rate of waves that do nothing but
    v_mfma_i32_32x32x32_i8 (no memory traffic), two workgroups of four
    waves per CU, about 2 ms per launch, timed like the kernels above."""
    probe = _mfma_probe(torch)
    if probe is None:
        return {"error": "tests/gpu_probe/libmfma_rate.so not built"}
    run, out, blocks = probe
    run(1)
    s1 = out.clone()
    run(2)
    consistent = bool(torch.equal(out, s1 * 2))
    t = timer.time(lambda i: run(MFMA_LOOP_ITERS), 5, warm=1)
    ops = blocks * 4 * MFMA_LOOP_ITERS * 8 * 65536
    res = {"workload": f"{blocks} workgroups x 4 waves x {MFMA_LOOP_ITERS} x 8 v_mfma_i32_32x32x32_i8",
           "us": round(t * 1e6, 1), "tops": round(ops / t / 1e12, 1),
           "frac": round(ops / t / 1e12 / PEAK_INT8_TOPS, 4), "work_doubles_with_iters": consistent}
    # the same loop on v_mfma_f32_32x32x16_bf16 (32768 flops each), for the
    # weight-only path's bf16 matmul
    t16 = timer.time(lambda i: run(MFMA_LOOP_ITERS, bf16=True), 5, warm=1)
    flops = blocks * 4 * MFMA_LOOP_ITERS * 8 * 32768
    res["bf16"] = {"us": round(t16 * 1e6, 1), "tflops": round(flops / t16 / 1e12, 1),
                   "frac": round(flops / t16 / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return res


def device_info(torch):
    """Device name, architecture, CUs, HBM, the peak shader clock and the HIP
    runtime version (from the runtime itself), torch's build."""
    import ctypes
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "gcn_arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1), "hip": torch.version.hip, "torch": torch.__version__}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (hip_runtime_api.h): peak clock in kHz
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, torch.cuda.current_device()) == 0:
            info["peak_clock_mhz"] = v.value / 1000
        if hip.hipRuntimeGetVersion(ctypes.byref(v)) == 0:
            info["hip_runtime_version"] = v.value
    except OSError:
        pass
    return info


def vendor_int_mm(torch, cr, wl, timer):
    """torch._int_mm (the vendor library's int8 GEMM, int32 output; run only)
    at the headline shape on cold operands, for context.  The weight is
    stored [N, K] as the library's is and passed transposed (its fastest
    layout here: a [K, N] copy ran about 35 % slower)."""
    dev = torch.device("cuda")
    per = M * K + N * K + 4 * M * N
    n = max(2, -(-2 * MALL_BYTES // per) + 1)
    a = [torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev) for _ in range(n)]
    b = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev) for _ in range(n)]
    c = [torch.empty((M, N), dtype=torch.int32, device=dev) for _ in range(n)]
    t = timer.time(lambda i: torch._int_mm(a[i % n], b[i % n].t(), out=c[i % n]), 50)
    del a, b, c
    return {"workload": "torch._int_mm int8 x int8 -> int32, M=2048 K=4096 N=12288 (no epilogue)",
            "us": round(t * 1e6, 2), "tops": round(2.0 * M * N * K / t / 1e12, 1)}


def copy_peak(torch, timer):
    """Measured streaming bandwidth of a 1 GiB device-to-device pass (read +
    write bytes), for context.  Two ways: torch's copy_ (the runtime's copy
    kernel) and an elementwise kernel that reads and writes the same bytes
    (x + 0 on int32 words), which streams about a fifth faster here."""
    a = torch.zeros((1 << 28,), dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    t_copy = timer.time(lambda i: b.copy_(a), 10)
    t_ew = timer.time(lambda i: torch.add(a, 0, out=b), 10)
    del a, b
    return {"copy_": round(2 * (1 << 30) / t_copy / 1e9, 1),
            "elementwise": round(2 * (1 << 30) / t_ew / 1e9, 1)}


# GEMM shapes whose tile plans the counter runs cover (M, N, K, weight bits).
# int8 weights: the headline shape (256x384, eight waves), M=2048, N=6144
# (256x192), the MLP down shape (256x128, three stages), the attention shape
# M=512 (64x128, four stages) and M=6144, N=8192 (256x256).  int4 weights:
# M=2048, N=12288 (256x192), the MLP down shape, M=512 and M=4096, N=12288
# (256x256).  Each plan also runs at a second K, so that counts which grow
# with K (the main loop) separate from those which do not (set-up and
# epilogue).
GEMM_TILE_SHAPES = [(2048, 12288, 4096, 8), (2048, 12288, 8192, 8), (2048, 6144, 4096, 8), (2048, 6144, 8192, 8),
                    (2048, 4096, 12288, 8), (2048, 4096, 4096, 8), (512, 4096, 4096, 8), (512, 4096, 8192, 8),
                    (6144, 8192, 4096, 8), (6144, 8192, 8192, 8),
                    (2048, 12288, 4096, 4), (2048, 12288, 8192, 4), (2048, 4096, 12288, 4), (2048, 4096, 4096, 4),
                    (512, 4096, 4096, 4), (512, 4096, 8192, 4), (4096, 12288, 4096, 4), (4096, 12288, 8192, 4)]


# Warm-up launches ahead of the profiled ones in --profile gemm_tiles (of the
# first shape, about 50 ms) and --profile mfma_rate (about 60 ms): counters
# taken on a device fresh from idle read a lower clock than the bench's
# steady state.
PROFILE_WARM_GEMM = 500
PROFILE_WARM_MFMA = 20


def profile_mode(mode, torch, cr, wl):
    """Short runs for rocprofv3 counter collection (a handful of launches)."""
    dev = torch.device("cuda")
    if mode == "gemm_tiles":
        g = torch.Generator(device=dev).manual_seed(3)
        first = True
        for (m, n, k, bits) in GEMM_TILE_SHAPES:
            xq = torch.randint(-127, 128, (m, k), dtype=torch.int8, device=dev, generator=g)
            if bits == 8:
                wq = torch.randint(-127, 128, (n, k), dtype=torch.int8, device=dev, generator=g)
            else:
                wq = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=dev, generator=g)
            xs = torch.rand(m, device=dev, generator=g) * 0.01
            ws = torch.rand(n, device=dev, generator=g) * 0.01
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            if first:  # the device's clock settles under tens of ms of load
                for _ in range(PROFILE_WARM_GEMM):
                    _ok(cr, cr.convrot_gemm_i8(xq, xs, wq, bits, ws, m, n, k, None, y))
                first = False
            for _ in range(3):
                _ok(cr, cr.convrot_gemm_i8(xq, xs, wq, bits, ws, m, n, k, None, y))
            torch.cuda.synchronize()
            log(f"profile mode gemm_tiles: W{bits} M={m} N={n} K={k}, 3 launches")
            del xq, wq, xs, ws, y
        return
    if mode == "mfma_rate":
        probe = _mfma_probe(torch)
        if probe is None:
            raise SystemExit("bench.py: tests/gpu_probe/libmfma_rate.so not built")
        run, _, blocks = probe
        for _ in range(PROFILE_WARM_MFMA + 3):
            run(MFMA_LOOP_ITERS)
        torch.cuda.synchronize()
        log(f"profile mode mfma_rate: {PROFILE_WARM_MFMA} warm-up and 3 launches of {blocks} x 4 waves x "
            f"{MFMA_LOOP_ITERS} x 8 MFMAs")
        return
    if mode == "copy":
        n = 1 << 30
        a = torch.empty((n,), dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n} bytes")
        return
    if mode == "rq_large":
        m, k = RQ_PASSES[1]
        xd = torch.randn((m, k), device=dev).to(torch.bfloat16)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xs = torch.empty((m,), dtype=torch.float32, device=dev)
        for _ in range(3):
            cr.convrot_rotate_quant(xd, m, k, GROUP, xq, xs)
        torch.cuda.synchronize()
        log(f"profile mode rq_large M={m} K={k}: 3 launches")
        return
    if mode == "rq_g16":
        m, k = RQ_G16_PASS
        xd = torch.randn((m, k), device=dev).to(torch.bfloat16)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xs = torch.empty((m,), dtype=torch.float32, device=dev)
        for _ in range(3):
            cr.convrot_rotate_quant(xd, m, k, 16, xq, xs)
        torch.cuda.synchronize()
        log(f"profile mode rq_g16 M={m} K={k} group 16: 3 launches")
        return
    if mode == "gemm_bf16":
        g = torch.Generator(device=dev).manual_seed(5)
        xb = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        wb = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            cr.gemm_bf16(xb, wb, out=yb)
        torch.cuda.synchronize()
        log(f"profile mode gemm_bf16 M={M} K={K} N={N}: 3 launches")
        return
    if mode == "rmsnorm_rq":
        m, k = RMSNORM_PASS
        xd = torch.randn((m, k), device=dev).to(torch.bfloat16)
        nw = torch.from_numpy(wl.make_norm_weight(k, k // 100, seed=4)).to(dev)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xs = torch.empty((m,), dtype=torch.float32, device=dev)
        for _ in range(3):
            cr.convrot_rmsnorm_rotate_quant(xd, nw, 1e-6, m, k, GROUP, xq, xs)
        torch.cuda.synchronize()
        log(f"profile mode rmsnorm_rq M={m} K={k}: 3 launches")
        return
    x, w, sets = build_sets(torch, cr, wl, 1)
    xd, wq, ws, y, wsp = sets[0]
    xq, xs = cr.rotate_quant(xd)
    for _ in range(3):
        if mode == "gemm":
            cr.convrot_gemm_i8(xq, xs, wq, 8, ws, M, N, K, None, y)
        elif mode == "rq":
            cr.convrot_rotate_quant(xd, M, K, GROUP, xq, xs)
        else:
            cr.w8a8_linear(xd, wq, ws, out=y, ws=wsp)
    torch.cuda.synchronize()
    log(f"profile mode {mode}: 3 launches")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The device reaches its steady clock only after tens of milliseconds of
    # this load: 20 warm-up steps measured 112.7 us per step, 500 (about
    # 55 ms) 105.7 us, on the same box.
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--profile", choices=["gemm", "gemm_tiles", "gemm_bf16", "rq", "rq_large", "rq_g16", "rmsnorm_rq", "mfma_rate",
                                          "copy", "linear"], default=None)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (each ConvRot linear runs on a single MI355X); "
              "multi-GPU runs are not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import w8a8_quantized_linear_amd as cr
    from w8a8_quantized_linear_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    cr.load()

    if args.profile:
        profile_mode(args.profile, torch, cr, wl)
        return

    per_set = M * K * 2 + N * K + N * 4 + M * N * 2 + cr.convrot_workspace_size(M, K)
    nsets = max(2, -(-2 * MALL_BYTES // per_set) + 1)
    log(f"building {nsets} buffer sets of {per_set / 2**20:.1f} MiB")
    x, w, sets = build_sets(torch, cr, wl, nsets)
    timer = Timer(torch)

    def step(i):
        xd, wq, ws, y, wsp = sets[i % nsets]
        cr.w8a8_linear(xd, wq, ws, group=GROUP, out=y, ws=wsp)

    ops = 2.0 * M * N * K
    # Per-kernel durations, live, on the launch stream (each after its own
    # 50 ms of warm-up launches).  They run before the headline region, so
    # the headline's steps start on a device that has been under this load.
    q = [cr.rotate_quant(s[0]) for s in sets]
    t_gemm = timer.time(lambda i: cr.convrot_gemm_i8(q[i % nsets][0], q[i % nsets][1], sets[i % nsets][1], 8,
                                                     sets[i % nsets][2], M, N, K, None, sets[i % nsets][3]),
                        max(200, args.steps))
    t_rq = timer.time(lambda i: cr.convrot_rotate_quant(sets[i % nsets][0], M, K, GROUP, q[i % nsets][0],
                                                        q[i % nsets][1]), max(200, args.steps))
    # resident (hot) variant of the whole step, for reference
    t_hot = timer.time(lambda i: cr.w8a8_linear(sets[0][0], sets[0][1], sets[0][2], out=sets[0][3],
                                                ws=sets[0][4]), max(200, args.steps))
    gemm_tops = ops / t_gemm / 1e12
    rq_bytes = M * (3 * K + 4)
    rq_gbs = rq_bytes / t_rq / 1e9
    # the same bytes moved by a plain streaming pass over the same inputs
    rq_same = stream_same_bytes(torch, [s[0] for s in sets], M, K, timer)

    # The headline: W untimed warm-up steps, then exactly K timed steps.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_step = start.elapsed_time(end) / 1e3 / args.steps
    log(f"timed {args.steps} steps: {t_step * 1e6:.1f} us/step (host wall {wall * 1e3:.1f} ms)")
    tops = ops / t_step / 1e12

    # Seven more timed runs (after the headline region, so they do not
    # affect it), each of at least 10 ms of steps: median and min per step.
    rep_steps = max(args.steps, int(np.ceil(0.010 / max(t_step, 1e-6))))
    reps = []
    for r in range(7):
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record()
        for i in range(rep_steps):
            step(i)
        s1.record()
        s1.synchronize()
        reps.append(s0.elapsed_time(s1) / rep_steps)
    reps.sort()

    last = sets[(args.steps - 1) % nsets]
    parity = check_parity(torch, cr, x, w, last[3], *q[(args.steps - 1) % nsets], last[1], last[2])
    # Every buffer set holds the same inputs, so every set's output must
    # equal the checked one bit for bit.
    parity["buffer_sets_identical"] = all(torch.equal(s_[3].view(torch.int16), last[3].view(torch.int16))
                                          for s_ in sets)
    log(f"parity (sampled, vs oracle): {parity}")

    out = {
        "metric": "W8A8 ConvRot linear TOPS & tokens/s (M=2048,K=4096,N=12288); % int8 MFMA peak",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "ConvRot W8A8 linear, MLP up/gate shape: M=2048 tokens, K=4096, N=12288, "
                               "group 256, bf16 N(0,1) activations with 1% outlier channels x20, int8 per-row "
                               "weights; operands cycled through buffer sets larger than 2x the MALL",
                   "M": M, "K": K, "N": N, "group": GROUP, "buffer_sets": nsets},
        "tokens_per_s": round(M / t_step, 1),
        "pct_int8_peak": round(tops / PEAK_INT8_TOPS, 4),
        "hot_tops": round(ops / t_hot / 1e12, 2),
        "step_repeats": {"runs": len(reps), "steps_each": rep_steps, "median_ms": round(reps[len(reps) // 2], 5),
                         "min_ms": round(reps[0], 5), "max_ms": round(reps[-1], 5),
                         "median_tops": round(ops / (reps[len(reps) // 2] * 1e-3) / 1e12, 2),
                         "max_tops": round(ops / (reps[0] * 1e-3) / 1e12, 2)},
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_i8_w8_kernel (eight-wave 256x384 int8 MFMA GEMM + bf16 epilogue)",
            "achieved": round(gemm_tops, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOPS",
            "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
            "traffic": load_traffic("gemm_i8_C3u", GEMM_SOURCES),
            "mfma_busy_counter": load_mfma_busy(),
            "avg_launch_us": round(t_gemm * 1e6, 3),
            "algorithmic_ops_per_launch": ops,
        },
        "rotate_quant": {
            "bound": "hbm",
            "achieved": round(rq_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(rq_gbs / PEAK_HBM_GBS, 4),
            "avg_launch_us": round(t_rq * 1e6, 3),
            "algorithmic_bytes_per_launch": rq_bytes,
            "traffic": load_traffic("rotate_quant_C3u", RQ_SOURCES),
            "stream_same_bytes": rq_same,
        },
        "parity": parity,
        "device": device_info(torch),
    }
    log("rotate-quantize on the large passes")
    out["rotate_quant_large"] = {"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "passes": rq_passes(torch, cr, timer),
                                 "traffic": load_traffic("rotate_quant_M8704_K12288", RQ_SOURCES),
                                 "copy_peak_measured": copy_peak(torch, timer)}
    log("fused RMSNorm + rotate-quantize M=8704 K=4096")
    out["rmsnorm_rotate_quant"] = rmsnorm_rq_pass(torch, cr, wl, timer)
    if not args.no_extras:
        log("extras: MFMA-only loop for context")
        out["mfma_loop"] = mfma_loop(torch, timer)
        if "tops" in out["mfma_loop"]:
            # the int8 rate the device sustains with no data to move, beside
            # the GEMM's (peak and frac stay priced at the published 5.0 POP/s)
            out["roofline"]["mfma_loop_tops"] = out["mfma_loop"]["tops"]
            out["roofline"]["frac_of_mfma_loop"] = round(gemm_tops / out["mfma_loop"]["tops"], 4)
        log("extras: vendor int8 GEMM for context")
        try:
            out["vendor_int_mm"] = vendor_int_mm(torch, cr, wl, timer)
        except RuntimeError as e:  # not every torch build exposes an int8 GEMM
            out["vendor_int_mm"] = {"error": str(e)[:200]}
        log("extras: single linears M=16 / 512 / 2048 (K 12288)")
        out["other_linears"] = extras_configs(torch, cr, wl, timer)
        log("extras: one GPU's share of the headline linear under 8-way sharding")
        out["shards"] = extras_shards(torch, cr, wl, timer, x, w)
        log("extras: W4A8 M=4096 K=4096 N=12288")
        out["w4a8"] = extras_w4a8(torch, cr, wl, timer)
        log("extras: weight-only path M=2048 K=4096 N=12288")
        out["dequant_path"] = extras_dequant(torch, cr, wl, timer)
        if "bf16" in out.get("mfma_loop", {}):
            g = out["dequant_path"]["gemm_bf16"]
            g["frac_of_mfma_loop"] = round(g["tflops"] / out["mfma_loop"]["bf16"]["tflops"], 4)
        log("extras: vision block, group 16")
        out["vision_g16"] = extras_vision(torch, cr, wl, timer)
        log("extras: 32-layer stack M=8704")
        out["stack"] = extras_stack(torch, cr, wl, timer)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

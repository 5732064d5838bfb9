"""Benchmark of the fused attention forward on one MI355X.

One step is one fa_fwd launch over the whole workload (inputs resident in
HBM).  Default workload: the wide-logit run B=2, H=16, N=8192, d=128,
non-causal (the throughput target).  Prints ONE JSON line with the metric,
the roofline of the kernel (MFMA-bound, BF16 dense peak), the CPU oracle
baseline, and per-run / per-variant timings.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense BF16 flop/clk/CU (the 2.5 PF spec)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fa_fwd_wide.json")
# Sources that define the forward kernel (the one whose HBM counters are
# stored): a change to any of them makes the stored traffic stale.
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_107_amd", "csrc", f)
                  for f in ("fa_kernel.hpp", "fa_internal.h", "fa_kernels_d64.hip",
                            "fa_kernels_d128.hip", "fa_kernels_d256.hip")] + \
                 [os.path.join(ROOT, "exact_attention_107_amd", "build.py")]


def workload_label(run, inp) -> str:
    """What the run is, with its sizes and input distribution."""
    if inp.get("cu_seqlens") is not None:
        shape = (f"{len(inp['lengths'])} packed sequences of {run.len_lo}..{run.len_hi} tokens "
                 f"(T={inp['T']}) H={inp['H']} d={inp['d']}")
    else:
        shape = f"B={inp['B']} H={inp['H']} N={inp['N']} d={inp['d']}"
    dist = f"Q,K~N(0,{run.sigma_qk:g}^2)"
    if run.boost_frac > 0:
        dist += f" with {run.boost_frac:.0%} of K rows x8"
    return f"{run.name}: {shape} causal={inp['causal']} {dist}, V~N(0,1)"


def fwd_rows(fa, torch, inp) -> int:
    """Rows per workgroup that fa_fwd picks for the input's shape on this GPU."""
    cu = inp.get("cu_seqlens")
    n = int(cu[-1]) if cu is not None else inp["N"]
    return fa.fwd_tile_rows(inp["B"], inp["H"], n, inp["d"], inp["causal"], cu is not None,
                            torch.cuda.get_device_properties(0).multi_processor_count)


def kernel_fingerprint() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def settle_clock(launch, seconds: float, torch) -> int:
    """Repeat `launch` for about `seconds` of wall time before anything is
    timed: the GPU leaves its idle clock over the first tens of
    milliseconds of load, which a short warmup alone does not cover.
    Returns the number of launches (reported in the JSON line)."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            launch()
        torch.cuda.synchronize()
        n += 5
    return n


def time_launches(launch, steps: int, warmup: int, torch):
    """Warmup, then `steps` launches bracketed by synchronisation; per-launch
    HIP events on the launch stream give the kernel's average duration."""
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record()
        launch()
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in ev]
    return wall * 1e3 / steps, float(np.mean(per)), float(np.median(per)), float(np.min(per))


def cpu_baseline(inp, target_s: float, gpu_out=None):
    """The oracle on a bounded row sample of the same workload, all host cores.
    With ``gpu_out = (o, lse, torch)`` (the timed launch's outputs) the same
    rows are also compared with the GPU result."""
    import oracle
    from exact_attention_107_amd.workloads import flops
    threads = oracle.default_threads()
    lengths = np.asarray(inp["lengths"])
    B, H = len(lengths), inp["H"]
    rng = np.random.Generator(np.random.PCG64(0))

    def rows_of(count):
        b = rng.integers(B, size=count)
        n = lengths[b]
        i = (rng.random(count) * n).astype(np.int64)
        h = rng.integers(H, size=count)
        return np.stack([b, h, i], axis=1).astype(np.int64)

    def credited(rows):
        # 4 * (visible keys) * d per row: the per-row share of 4 n^2 d (halved causal)
        n = lengths[rows[:, 0]].astype(np.float64)
        vis = (rows[:, 2] + 1).astype(np.float64) if inp["causal"] else n
        return float(np.sum(4.0 * vis * inp["d"]))

    calib = rows_of(max(threads * 4, 64))
    t0 = time.perf_counter()
    oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=inp["causal"],
                     cu_seqlens=inp["cu_seqlens"], rows=calib, nthreads=threads)
    dt = time.perf_counter() - t0
    count = int(min(max(len(calib) * target_s / max(dt, 1e-3), len(calib)), 2_000_000))
    rows = rows_of(count)
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=inp["causal"],
                                      cu_seqlens=inp["cu_seqlens"], rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    f = credited(rows)
    total = flops(lengths, H, inp["d"], inp["causal"])
    parity = None
    if gpu_out is not None:
        parity = sampled_parity(inp, rows, o_ref, lse_ref, *gpu_out)
    return {
        "value": f / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{count} random query rows of the {inp['name']} run "
                  f"({f / total * 100:.3f}% of its credited flops), fp64, {dt:.1f} s wall",
        "seconds": dt, "full_run_seconds_extrapolated": dt * total / f,
    }, parity


def sampled_parity(inp, rows, o_ref, lse_ref, o, lse, torch):
    """The timed launch's O and LSE on the oracle's sample rows, with the
    forward's tolerances (bf16 O: max 2e-2, mean 2e-3; fp32 LSE: max 1e-3)."""
    from exact_attention_107_amd.workloads import bf16_to_f32
    r = torch.from_numpy(rows).cuda()
    b, h, i = r[:, 0], r[:, 1], r[:, 2]
    if inp["cu_seqlens"] is None:
        og, lg = o[b, i, h], lse[b, h, i]
    else:
        tok = torch.from_numpy(inp["cu_seqlens"].astype(np.int64)).cuda()[b] + i
        og, lg = o[tok, h], lse[h, tok]
    og = bf16_to_f32(og.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    lg = lg.cpu().numpy().astype(np.float64)
    do, dl = np.abs(og - o_ref), np.abs(lg - lse_ref)
    res = {"kind": "oracle rows of the CPU baseline sample", "rows": int(len(rows)),
           "max_abs_o": float(do.max()), "mean_abs_o": float(do.mean()), "max_abs_lse": float(dl.max()),
           "tol": {"max_abs_o": 2e-2, "mean_abs_o": 2e-3, "max_abs_lse": 1e-3}}
    res["pass"] = bool(res["max_abs_o"] <= 2e-2 and res["mean_abs_o"] <= 2e-3 and res["max_abs_lse"] <= 1e-3)
    return res


def split_kv_runs(torch, fa):
    """Few-head runs: fa_fwd alone vs fa_fwd_splitkv at the library's suggested
    split count (both kernels inside the timed launch), and the merge kernel
    alone against the HBM roofline."""
    from exact_attention_107_amd.workloads import RUNS, flops, make_inputs
    res = {}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for name in ("few_heads", "few_heads_causal"):
        r = RUNS[name]
        log(f"[bench] split-KV run {name}")
        ri = make_inputs(r)
        q, k, v = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((r.B, r.H, r.N), dtype=torch.float32, device="cuda")
        S = fa.num_splits(r.B, r.H, r.N, r.d, r.causal, cus)
        op = torch.empty((S, r.B, r.N, r.H, r.d), dtype=torch.float32, device="cuda")
        lp = torch.empty((S, r.B, r.H, r.N), dtype=torch.float32, device="cuda")
        f = flops(ri["lengths"], r.H, r.d, r.causal)

        def plain():
            fa.fwd(q, k, v, causal=r.causal, scale=ri["scale"], out=o, lse=lse)

        def split():
            fa.fwd_splitkv(q, k, v, causal=r.causal, scale=ri["scale"], splits=S, out=o, lse=lse,
                           o_part=op, lse_part=lp)

        def merge():
            fa.merge(op, lp, out=o, lse=lse)

        _, ms_plain, _, _ = time_launches(plain, 20, 3, torch)
        _, ms_split, _, _ = time_launches(split, 20, 3, torch)
        _, ms_merge, _, _ = time_launches(merge, 20, 3, torch)
        rows = r.B * r.N * r.H
        merge_bytes = rows * (S * (r.d * 4 + 4) + r.d * 2 + 4)
        res[name] = {
            "shape": f"B={r.B} H={r.H} N={r.N} d={r.d} causal={r.causal}", "splits": S,
            "fa_fwd_ms": round(ms_plain, 4), "fa_fwd_tflops": round(f / ms_plain / 1e9, 1),
            "splitkv_ms": round(ms_split, 4), "splitkv_tflops": round(f / ms_split / 1e9, 1),
            "merge_ms": round(ms_merge, 4),
            "merge_roofline": {"bound": "hbm", "achieved": round(merge_bytes / ms_merge / 1e6, 1),
                               "peak": 8000.0, "unit": "GB/s",
                               "frac": round(merge_bytes / ms_merge / 1e6 / 8000.0, 4),
                               "bytes_per_launch": merge_bytes},
        }
        del q, k, v, o, lse, op, lp
    return res


def backward_run(torch, fa, name, steps=10, warmup=2):
    """fa_bwd (prep, dK/dV and dQ kernels) on one run, after one forward that
    provides O and LSE.  Credited flops: 10 n^2 d per (sequence, head), halved
    causal (five n x n x d products); the kernels execute 14 n^2 d (S and dP
    are recomputed by both the dK/dV and the dQ kernel), which is what the
    MFMA roofline counts."""
    from exact_attention_107_amd.workloads import RUNS, bwd_flops, make_grad, make_inputs
    r = RUNS[name]
    log(f"[bench] backward run {name}")
    ri = make_inputs(r)
    q, k, v = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
    do = to_dev(make_grad(ri["q"].shape, r.seed + 5000), torch)
    cu = None if ri["cu_seqlens"] is None else torch.from_numpy(ri["cu_seqlens"]).to("cuda")
    o, lse = fa.fwd(q, k, v, causal=r.causal, scale=ri["scale"], cu_seqlens=cu)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws_floats = fa.bwd_workspace_floats(1, r.H, ri["T"]) if cu is not None else fa.bwd_workspace_floats(r.B, r.H, r.N)
    ws = torch.empty(ws_floats, dtype=torch.float32, device="cuda")

    def launch():
        fa.bwd(q, k, v, o, lse, do, causal=r.causal, scale=ri["scale"], cu_seqlens=cu, dq=dq, dk=dk, dv=dv,
               workspace=ws)

    ms_step, ms, ms_med, ms_min = time_launches(launch, steps, warmup, torch)
    f = bwd_flops(ri["lengths"], r.H, r.d, r.causal)
    executed = f * 14.0 / 10.0
    shape = (f"{len(ri['lengths'])} packed sequences, T={ri['T']} H={r.H} d={r.d} causal={r.causal}"
             if cu is not None else f"B={r.B} H={r.H} N={r.N} d={r.d} causal={r.causal}")
    res = {"shape": shape, "ms": round(ms, 4),
           "ms_per_step": round(ms_step, 4), "tflops_credited": round(f / ms / 1e9, 1),
           "roofline": {"bound": "mfma", "achieved": round(executed / ms / 1e9, 1), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(executed / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                        "per_launch": "14*B*H*N^2*d executed MFMA flops (halved causal) / mean HIP-event "
                                      "duration of the three backward kernels"}}
    del q, k, v, do, o, lse, dq, dk, dv, ws, cu
    return res, f, ms_step


PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS  # dense E4M3 MFMA rate is twice BF16's


def fp8_setup(torch, fa, r, ri):
    """Device inputs of one FP8 run, quantised per (sequence, head); returns
    (q, launch of the forward, quantisation of q into its codes, (o, lse))."""
    q, k, v = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    if ri["cu_seqlens"] is not None:
        cu = torch.from_numpy(ri["cu_seqlens"]).cuda()
        q8, dq = fa.quantize_fp8_packed(q, cu)
        k8, dk = fa.quantize_fp8_packed(k, cu)
        vt8, dv = fa.quantize_fp8_packed(v, cu, transpose=True)
        lse = torch.empty((r.H, ri["T"]), dtype=torch.float32, device="cuda")

        def launch():
            fa.fwd_fp8_packed(q8, k8, vt8, dq, dk, dv, cu, causal=r.causal, scale=ri["scale"], out=o, lse=lse)

        def quant():
            fa.quantize_fp8_packed(q, cu, out=q8, descale=dq)
        return q, launch, quant, (o, lse)
    q8, dq = fa.quantize_fp8(q)
    k8, dk = fa.quantize_fp8(k)
    vt8, dv = fa.quantize_fp8(v, transpose=True)
    lse = torch.empty((r.B, r.H, r.N), dtype=torch.float32, device="cuda")

    def launch():
        fa.fwd_fp8(q8, k8, vt8, dq, dk, dv, causal=r.causal, scale=ri["scale"], out=o, lse=lse)

    def quant():
        fa.quantize_fp8(q, out=q8, descale=dq)
    return q, launch, quant, (o, lse)


def fp8_runs(torch, fa):
    """FP8 (E4M3) forward on the headline shape and others (d = 256, the
    packed causal batch): inputs are quantised per (sequence, head) once,
    outside the timed launches; the quantisation of one tensor is timed on
    its own."""
    from exact_attention_107_amd.workloads import RUNS, flops, make_inputs
    res = {}
    for name in ("wide", "long_causal", "mid", "wide_d256", "varlen_causal"):
        r = RUNS[name]
        log(f"[bench] fp8 run {name}")
        ri = make_inputs(r)
        q, launch, quant, _ = fp8_setup(torch, fa, r, ri)
        f = flops(ri["lengths"], r.H, r.d, r.causal)

        _, ms, _, _ = time_launches(launch, 30, 30, torch)
        _, msq, _, _ = time_launches(quant, 10, 3, torch)
        tf = f / ms / 1e9
        shape = (f"packed B={r.B} T={ri['T']} H={r.H} d={r.d} causal={r.causal}" if ri["cu_seqlens"] is not None
                 else f"B={r.B} H={r.H} N={r.N} d={r.d} causal={r.causal}")
        res[name] = {"shape": shape, "ms": round(ms, 4),
                     "tflops": round(tf, 1),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4)},
                     "quantize_one_tensor_ms": round(msq, 4)}
        del q, launch, quant
    return res


def masked_runs(torch, fa):
    """fa_fwd_masked: a causal sliding window of 1024 keys with ALiBi slopes
    on B=1 H=16 N=16384 d=128 (credited flops: 4 d per visible (query, key)
    pair), and the plain causal mask through the masked path next to fa_fwd."""
    from exact_attention_107_amd.workloads import Run, flops, make_inputs
    r = Run("masked", 1, 16, 16384, 128, False, 1009)
    log("[bench] masked runs")
    ri = make_inputs(r)
    q, k, v = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((r.B, r.H, r.N), dtype=torch.float32, device="cuda")
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / r.H) for h in range(r.H)], dtype=torch.float32,
                          device="cuda")
    W = 1024
    pairs = sum(min(i + 1, W + 1) for i in range(r.N))
    f_window = 4.0 * r.d * r.H * r.B * pairs
    f_causal = flops(ri["lengths"], r.H, r.d, True)
    res = {"shape": f"B={r.B} H={r.H} N={r.N} d={r.d}"}
    for name, kw, f in (("window1024_alibi", dict(window_left=W, window_right=0, alibi_slopes=slopes), f_window),
                        ("causal_masked_path", dict(window_left=-1, window_right=0), f_causal)):
        def launch():
            fa.fwd_masked(q, k, v, scale=ri["scale"], out=o, lse=lse, **kw)
        _, ms, _, _ = time_launches(launch, 20, 20, torch)
        res[name] = {"ms": round(ms, 4), "tflops": round(f / ms / 1e9, 1)}

    def causal():
        fa.fwd(q, k, v, causal=True, scale=ri["scale"], out=o, lse=lse)
    _, ms, _, _ = time_launches(causal, 20, 20, torch)
    res["causal_fa_fwd"] = {"ms": round(ms, 4), "tflops": round(f_causal / ms / 1e9, 1)}
    del q, k, v, o, lse
    return res


def other_pass(torch, fa, which, workload, steps, warmup, settle_s=0.0):
    """One kernel family alone on one workload, for profiling: the FP8
    forward (inputs quantised once, outside the timed launches), the split-KV
    forward with the library's split count (split kernel and merge in each
    launch), or the masked forward's sliding window with ALiBi."""
    from exact_attention_107_amd.workloads import Run, RUNS, flops, make_inputs
    if which == "masked":
        r = Run("masked", 1, 16, 16384, 128, False, 1009)
    else:
        r = RUNS[workload]
    ri = make_inputs(r)
    q, k, v = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((r.B, r.H, r.N), dtype=torch.float32, device="cuda")
    f = flops(ri["lengths"], r.H, r.d, r.causal)
    label = f"{r.name}: B={r.B} H={r.H} N={r.N} d={r.d} causal={r.causal}"
    res = {}
    if which == "fp8":
        _, launch, _, _ = fp8_setup(torch, fa, r, ri)
    elif which == "split":
        S = fa.num_splits(r.B, r.H, r.N, r.d, r.causal, torch.cuda.get_device_properties(0).multi_processor_count)
        op = torch.empty((S, r.B, r.N, r.H, r.d), dtype=torch.float32, device="cuda")
        lp = torch.empty((S, r.B, r.H, r.N), dtype=torch.float32, device="cuda")
        res["splits"] = S

        def launch():
            fa.fwd_splitkv(q, k, v, causal=r.causal, scale=ri["scale"], splits=S, out=o, lse=lse, o_part=op,
                           lse_part=lp)
    elif which == "pingpong":
        label += ", the two query tiles of a workgroup half a key tile apart"

        def launch():
            fa.fwd(q, k, v, causal=r.causal, scale=ri["scale"], out=o, lse=lse, pingpong=True)
    else:
        W = 1024
        slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / r.H) for h in range(r.H)], dtype=torch.float32,
                              device="cuda")
        f = 4.0 * r.d * r.H * r.B * sum(min(i + 1, W + 1) for i in range(r.N))
        label += f", window of {W} keys to the left, causal, ALiBi slopes 2^(-8(h+1)/H)"

        def launch():
            fa.fwd_masked(q, k, v, scale=ri["scale"], out=o, lse=lse, window_left=W, window_right=0,
                          alibi_slopes=slopes)
    log(f"[bench] {which} pass on {label}")
    if settle_s > 0:
        res["clock_settle_launches"] = settle_clock(launch, settle_s, torch)
    ms_step, ms, _, _ = time_launches(launch, steps, warmup, torch)
    res.update({"ms": round(ms, 5), "tflops": round(f / ms / 1e9, 1)})
    return res, f, ms_step, ms, label


def reference_copy(torch, mib: int) -> None:
    """One plain device copy of `mib` MiB: a dispatch of known bytes to scale
    the HBM byte counters by."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def quant_pass(torch, fa, workload, steps, warmup, settle_s=0.0):
    """The per-(sequence, head) E4M3 quantisation an FP8 forward needs, for
    profiling: Q and K in their own layout and V transposed, one step = the
    three calls."""
    from exact_attention_107_amd.workloads import RUNS, make_inputs
    r = RUNS[workload]
    ri = make_inputs(r)
    q, k, v = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
    cu = torch.from_numpy(ri["cu_seqlens"]).cuda() if ri["cu_seqlens"] is not None else None
    if cu is None:
        outs = [fa.quantize_fp8(x, transpose=t) for x, t in ((q, False), (k, False), (v, True))]
    else:
        outs = [fa.quantize_fp8_packed(x, cu, transpose=t) for x, t in ((q, False), (k, False), (v, True))]

    def launch():
        for (x, t), (c, d) in zip(((q, False), (k, False), (v, True)), outs):
            if cu is None:
                fa.quantize_fp8(x, transpose=t, out=c, descale=d)
            else:
                fa.quantize_fp8_packed(x, cu, transpose=t, out=c, descale=d)
    label = f"{r.name}: B={r.B} H={r.H} N={ri['N']} d={r.d}{' packed' if cu is not None else ''}, Q and K " \
            "in their layout, V transposed"
    log(f"[bench] quant pass on {label}")
    res = {}
    if settle_s > 0:
        res["clock_settle_launches"] = settle_clock(launch, settle_s, torch)
    ms_step, ms, _, _ = time_launches(launch, steps, warmup, torch)
    nbytes = 3 * q.numel() * 2
    res.update({"ms": round(ms, 5), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_bf16_per_step": nbytes})
    return res, ms_step, label


def rescale_rates(torch, fa):
    """How often the conditional rescale fires (counting instance of the
    kernel, one launch per run and rule): the share of wave-steps (64 keys x 32
    rows) whose O accumulator is rescaled, and of rows whose reference max moves,
    over every key tile after each wave's first."""
    from exact_attention_107_amd.workloads import RUNS, make_inputs
    res = {}
    for name in ("wide", "mid", "long_causal", "varlen_causal"):
        log(f"[bench] rescale counts {name}")
        ri = make_inputs(RUNS[name])
        q, k, v = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
        cu = torch.from_numpy(ri["cu_seqlens"]).cuda() if ri["cu_seqlens"] is not None else None
        res[name] = {}
        for rule, mode in (("strict", fa.RESCALE_STRICT), ("threshold", fa.RESCALE_THRESHOLD)):
            c = fa.rescale_counts(q, k, v, causal=ri["causal"], scale=ri["scale"], cu_seqlens=cu,
                                  rescale_mode=mode)
            res[name][rule] = {"step_rescale_rate": round(c["step_rescale_rate"], 5),
                               "row_move_rate": round(c["row_move_rate"], 5), "steps": c["steps"]}
        del q, k, v
    return res


def device_clock(arch: str):
    """Max engine clock and CU count that rocminfo reports for the GPU agent."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    name = arch.split(":")[0]
    for block in txt.split("Agent ")[1:]:
        if re.search(r"Name:\s+" + re.escape(name) + r"\s", block):
            clk = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", block)
            cus = re.search(r"Compute Unit:\s+(\d+)", block)
            return {"max_sclk_mhz": int(clk.group(1)) if clk else None,
                    "compute_units": int(cus.group(1)) if cus else None}
    return None


def traffic_for(fingerprint: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_fingerprint") != fingerprint:
        return None
    return t.get("bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="wide")
    ap.add_argument("--extra", type=int, default=1, help="also time the other runs and variants")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd", "fp8", "split", "masked", "pingpong", "quant"),
                    default="fwd",
                    help="time only one other kernel family on --workload (for profiling): bwd = the "
                         "backward pass, fp8 = the FP8 forward, split = the split-KV forward and merge, "
                         "masked = the 1024-key sliding window with ALiBi (fixed shape), pingpong = the "
                         "two-query-tile ping-pong schedule of the forward (d = 128, dense), quant = the "
                         "FP8 quantisation of Q, K and V^T")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed launches before the warmup, so that the timed steps "
                         "run at the clock the GPU holds under this load (0: none)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "reference dispatch for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward here is a single-GPU "
              "kernel with no collectives; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from exact_attention_107_amd import fa
    from exact_attention_107_amd.workloads import RUNS, flops, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    fa.load()
    props = torch.cuda.get_device_properties(0)
    if args.which == "bwd":
        res, f, ms_step = backward_run(torch, fa, args.workload, args.steps, args.warmup)
        print(json.dumps({
            "metric": "attention bwd TFLOP/s (bf16, credited 10*B*H*N^2*d, halved causal)",
            "value": res["tflops_credited"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{args.workload}: {res['shape']}"}, "roofline": res["roofline"],
            "kernel_fingerprint": kernel_fingerprint()}), flush=True)
        return 0
    if args.which == "quant":
        if args.copy_mb:
            reference_copy(torch, args.copy_mb)
        res, ms_step, label = quant_pass(torch, fa, args.workload, args.steps, args.warmup, args.settle_s)
        print(json.dumps({
            "metric": "FP8 quantisation of Q, K, V^T, GB/s (bf16 bytes of the three inputs per step)",
            "value": res["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8-e4m3", "data": "synthetic", "config": {"workload": label}, "result": res,
            "kernel_fingerprint": kernel_fingerprint()}), flush=True)
        return 0
    if args.which in ("fp8", "split", "masked", "pingpong"):
        res, f, ms_step, ms_kernel, label = other_pass(torch, fa, args.which, args.workload, args.steps,
                                                       args.warmup, args.settle_s)
        print(json.dumps({
            "metric": f"attention {args.which} forward TFLOP/s (credited 4*B*H*N^2*d, halved causal)",
            "value": round(f / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp8-e4m3" if args.which == "fp8" else "bf16", "data": "synthetic",
            "config": {"workload": label}, "result": res, "kernel_fingerprint": kernel_fingerprint()}), flush=True)
        return 0
    run = RUNS[args.workload]
    log(f"[bench] generating {run.name} inputs")
    inp = make_inputs(run)
    inp["name"] = run.name
    q, k, v = (to_dev(inp[x], torch) for x in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda() if inp["cu_seqlens"] is not None else None
    o = torch.empty_like(q)
    lse_shape = (inp["H"], inp["T"]) if cu is not None else (inp["B"], inp["H"], inp["N"])
    lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda")
    f = flops(inp["lengths"], inp["H"], inp["d"], inp["causal"])

    def launch():
        fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu, out=o, lse=lse)

    if args.copy_mb:
        reference_copy(torch, args.copy_mb)
    settle_launches = settle_clock(launch, args.settle_s, torch) if args.settle_s > 0 else 0
    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup "
        f"({settle_launches} launches to settle the clock first)")
    ms_step, ms_kernel, ms_med, ms_min = time_launches(launch, args.steps, args.warmup, torch)
    value = f / (ms_step * 1e-3) / 1e12
    achieved = f / (ms_kernel * 1e-3) / 1e12
    log(f"[bench] {run.name}: {ms_step:.4f} ms/step, kernel {ms_kernel:.4f} ms, {achieved:.1f} TFLOP/s")

    fp = kernel_fingerprint()
    out = {
        "metric": "attention fwd TFLOP/s (bf16, causal & non-causal) and % of MFMA BF16 peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": workload_label(run, inp),
            "B": inp["B"], "H": inp["H"], "N": inp["N"], "d": inp["d"], "causal": inp["causal"],
            "flops_per_step": f, "tile_rows": fwd_rows(fa, torch, inp), "tile_keys": fa.tile_keys(inp["d"]),
        },
        "clock_settle": {"seconds": args.settle_s, "launches": settle_launches,
                         "note": "untimed launches before the warmup steps"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(fp),
            "kernel_ms_mean": round(ms_kernel, 5), "kernel_ms_median": round(ms_med, 5),
            "kernel_ms_min": round(ms_min, 5),
            "per_launch": "4*B*H*N^2*d flops (halved if causal) / mean HIP-event duration",
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""),
                   "rocminfo": device_clock(getattr(props, "gcnArchName", "gfx950")),
                   "peak_formula": "256 CU x 2.4 GHz x 4096 dense BF16 flop/clk/CU (spec)"},
        "kernel_fingerprint": fp,
    }

    if args.extra:
        runs = {}
        for name in ("mid", "mid_causal", "long_causal", "varlen_causal", "wide_d64", "wide_d256", "few_heads",
                     "few_heads_causal"):
            r = RUNS[name]
            log(f"[bench] run {name}")
            ri = make_inputs(r)
            rq, rk, rv = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
            rcu = torch.from_numpy(ri["cu_seqlens"]).cuda() if ri["cu_seqlens"] is not None else None
            ro = torch.empty_like(rq)
            rl_shape = (ri["H"], ri["T"]) if rcu is not None else (ri["B"], ri["H"], ri["N"])
            rl = torch.empty(rl_shape, dtype=torch.float32, device="cuda")
            rf = flops(ri["lengths"], ri["H"], ri["d"], ri["causal"])

            def rlaunch():
                fa.fwd(rq, rk, rv, causal=ri["causal"], scale=ri["scale"], cu_seqlens=rcu, out=ro, lse=rl)

            _, kms, _, _ = time_launches(rlaunch, 50, 50, torch)  # clocks settle as for the headline
            runs[name] = {"ms": round(kms, 4), "tflops": round(rf / (kms * 1e-3) / 1e12, 1),
                          "pct_of_peak": round(100 * rf / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
                          "tile_rows": fwd_rows(fa, torch, ri)}
            del rq, rk, rv, ro, rl
        out["runs"] = runs
        variants = {}
        for em, en in ((fa.EXP_HW, "hw"), (fa.EXP_POLY, "poly"), (fa.EXP_MIXED, "mixed")):
            for rm, rn in ((fa.RESCALE_ALWAYS, "always"), (fa.RESCALE_STRICT, "strict"),
                           (fa.RESCALE_THRESHOLD, "threshold")):
                def vlaunch():
                    fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], out=o, lse=lse,
                           exp_mode=em, rescale_mode=rm)
                _, kms, _, _ = time_launches(vlaunch, 50, 30, torch)
                variants[f"{en}/{rn}"] = {"ms": round(kms, 4),
                                          "tflops": round(f / (kms * 1e-3) / 1e12, 1)}
        out["variants"] = variants
        # the two-group ping-pong schedule (fa_fwd_pingpong, d = 128): same
        # arithmetic, the workgroup's halves half a key tile apart
        pingpong = {}
        for name in ("wide", "mid", "mid_causal", "long_causal", "varlen_causal"):
            r = RUNS[name]
            ri = make_inputs(r) if name != run.name else inp
            rq, rk, rv = (to_dev(ri[x], torch) for x in ("q", "k", "v"))
            rcu = torch.from_numpy(ri["cu_seqlens"]).cuda() if ri["cu_seqlens"] is not None else None
            ro = torch.empty_like(rq)
            rl_shape = (ri["H"], ri["T"]) if rcu is not None else (ri["B"], ri["H"], ri["N"])
            rl = torch.empty(rl_shape, dtype=torch.float32, device="cuda")
            rf = flops(ri["lengths"], ri["H"], ri["d"], ri["causal"])
            res = {"in_step": 0.0, "pingpong": 0.0}
            for _ in range(3):  # alternate the two schedules; best of three each
                for sched, pp in (("in_step", False), ("pingpong", True)):
                    def plaunch():
                        fa.fwd(rq, rk, rv, causal=ri["causal"], scale=ri["scale"], cu_seqlens=rcu, out=ro, lse=rl,
                               pingpong=pp)
                    _, kms, _, _ = time_launches(plaunch, 30, 20, torch)
                    res[sched] = max(res[sched], round(rf / (kms * 1e-3) / 1e12, 1))
            pingpong[name] = res
            del rq, rk, rv, ro, rl
        out["pingpong_tflops"] = pingpong
        out["split_kv"] = split_kv_runs(torch, fa)
        out["backward"] = {name: backward_run(torch, fa, name)[0]
                           for name in ("mid", "mid_causal", "bwd_long", "bwd_long_causal", "varlen_causal",
                                        "wide_d256")}
        out["fp8"] = fp8_runs(torch, fa)
        out["masked"] = masked_runs(torch, fa)
        out["rescale_rates"] = rescale_rates(torch, fa)

    if not args.no_cpu_baseline:
        launch()  # the variants above reused o and lse: restore the timed launch's outputs
        torch.cuda.synchronize()
        log("[bench] CPU oracle baseline")
        out["cpu_baseline"], out["parity"] = cpu_baseline(inp, args.cpu_seconds, (o, lse, torch))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path
through the C ABI binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import bf16_to_f32

# Tolerances on bf16 O and fp32 LSE against the fp64 oracle.
TOL_O_MAX = 2e-2
TOL_O_MEAN = 2e-3
TOL_LSE_MAX = 1e-3


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> float64 numpy (exact widening)."""
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_to_f32(bits).astype(np.float64)


def run_gpu(inp, **kw):
    q, k, v = (to_dev(inp[x]) for x in ("q", "k", "v"))
    cu = None
    if inp.get("cu_seqlens") is not None:
        cu = torch.from_numpy(inp["cu_seqlens"]).to("cuda")
    o, lse = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu, **kw)
    torch.cuda.synchronize()
    return o, lse


def metrics(o, lse, o_ref, lse_ref):
    do = np.abs(np.asarray(o, np.float64) - o_ref)
    dl = np.abs(np.asarray(lse, np.float64) - lse_ref)
    return {
        "max_o": float(do.max()) if do.size else 0.0,
        "mean_o": float(do.mean()) if do.size else 0.0,
        "max_lse": float(dl.max()) if dl.size else 0.0,
        "finite": bool(np.all(np.isfinite(o)) and np.all(np.isfinite(lse))),
    }


def assert_within(m, what=""):
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_o"] <= TOL_O_MAX, f"{what}: max|dO| {m['max_o']:.3e} > {TOL_O_MAX}"
    assert m["mean_o"] <= TOL_O_MEAN, f"{what}: mean|dO| {m['mean_o']:.3e} > {TOL_O_MEAN}"
    assert m["max_lse"] <= TOL_LSE_MAX, f"{what}: max|dLSE| {m['max_lse']:.3e} > {TOL_LSE_MAX}"


def full_parity(inp, **kw):
    """Every element of O and LSE against the oracle (small sizes)."""
    o, lse = run_gpu(inp, **kw)
    o_ref, lse_ref = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"],
                                      causal=inp["causal"], cu_seqlens=inp.get("cu_seqlens"))
    return metrics(from_dev(o), lse.cpu().numpy(), o_ref, lse_ref), (o, lse)


def sample_rows(inp, count: int, seed: int = 0) -> np.ndarray:
    """(b, h, i) rows: tile boundaries, sequence ends, and random rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(inp["lengths"])
    B, H = len(lengths), inp["H"]
    rows = []
    for b in range(B):
        n = int(lengths[b])
        if n == 0:
            continue
        for i in {0, 1, 63, 64, 127, 128, 255, 256, n // 2, n - 2, n - 1}:
            if 0 <= i < n:
                rows.append((b, int(rng.integers(H)), i))
    while len(rows) < count:
        b = int(rng.integers(B))
        n = int(lengths[b])
        if n:
            rows.append((b, int(rng.integers(H)), int(rng.integers(n))))
    return np.array(rows, dtype=np.int64)


def gather_rows(inp, o: torch.Tensor, lse: torch.Tensor, rows: np.ndarray):
    rows_t = torch.from_numpy(rows)
    b, h, i = rows_t[:, 0], rows_t[:, 1], rows_t[:, 2]
    if inp.get("cu_seqlens") is None:
        osel = o[b.cuda(), i.cuda(), h.cuda()]
        lsel = lse[b.cuda(), h.cuda(), i.cuda()]
    else:
        cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int64))
        tok = (cu[b] + i).cuda()
        osel = o[tok, h.cuda()]
        lsel = lse[h.cuda(), tok]
    return from_dev(osel), lsel.cpu().numpy().astype(np.float64)


def sampled_parity(inp, o, lse, count=384, seed=0):
    rows = sample_rows(inp, count, seed)
    o_ref, lse_ref = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"],
                                      causal=inp["causal"], cu_seqlens=inp.get("cu_seqlens"),
                                      rows=rows)
    og, lg = gather_rows(inp, o, lse, rows)
    return metrics(og, lg, o_ref, lse_ref)


def every_row_parity(inp, o: torch.Tensor, lse: torch.Tensor):
    """Every row of a full-size output against the fp64 oracle in its
    whole-matrix form (oracle.matrix), one (sequence, head) at a time.
    Returns the metrics over all elements and the worst head."""
    from oracle import matrix
    o_bits = o.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    lse_h = lse.cpu().numpy().astype(np.float64)
    cu = inp.get("cu_seqlens")
    max_o = max_l = 0.0
    sum_o = 0.0
    count = 0
    finite = True
    worst = None
    for b, h, o_ref, l_ref in matrix.iter_heads(inp["q"], inp["k"], inp["v"], scale=inp["scale"],
                                                causal=inp["causal"], cu_seqlens=cu):
        if cu is None:
            og = bf16_to_f32(o_bits[b, :, h, :]).astype(np.float64)
            lg = lse_h[b, h, :]
        else:
            t0, t1 = int(cu[b]), int(cu[b + 1])
            og = bf16_to_f32(o_bits[t0:t1, h, :]).astype(np.float64)
            lg = lse_h[h, t0:t1]
        if og.size == 0:
            continue
        do = np.abs(og - o_ref)
        dl = np.abs(lg - l_ref)
        finite = finite and bool(np.all(np.isfinite(og)) and np.all(np.isfinite(lg)))
        mo, ml = float(do.max()), float(dl.max())
        if worst is None or mo > worst[2]:
            worst = (b, h, mo)
        max_o, max_l = max(max_o, mo), max(max_l, ml)
        sum_o += float(do.sum())
        count += do.size
    return {"max_o": max_o, "mean_o": sum_o / max(count, 1), "max_lse": max_l, "finite": finite,
            "elements": count, "worst_head": worst}

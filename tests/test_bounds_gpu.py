"""Loads at the end of an allocation (needs an MI355X).

Q, K, V (for the backward also O and dO; for the FP8 forward the E4M3 codes)
are views at the start of a larger device buffer whose part past the
tensor's end holds NaN.  A tail tile covers rows past the sequence; the
kernels must read those rows as zeros and never the bytes behind them, or
P = 0 times NaN makes the output NaN.  Every result must equal, bit for bit,
the result on the same tensors followed by zeros, and match the oracle.
The last sequence (dense: the last batch entry; packed: the last packed
sequence) ends at the end of the tensor, with N mod 64 in {1, 20, 33, 63}.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import Run, make_grad, make_inputs
from gpu_helpers import assert_within, from_dev, metrics

pytestmark = pytest.mark.gpu

TAIL_ROWS = 160            # more than two 64-row tiles past the end
BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F
REMS = [1, 20, 33, 63]


def _tail_view(arr: np.ndarray, fill: int, row_elems: int, dtype) -> torch.Tensor:
    """Device copy of `arr` at the start of a buffer followed by TAIL_ROWS
    rows of `fill` (raw bits)."""
    flat = np.ascontiguousarray(arr).reshape(-1)
    if arr.dtype == np.uint16:
        buf = torch.empty(flat.size + TAIL_ROWS * row_elems, dtype=torch.int16, device="cuda")
        buf[flat.size:] = fill - (1 << 16) if fill >= (1 << 15) else fill
        buf[:flat.size] = torch.from_numpy(flat.view(np.int16)).cuda()
    else:
        buf = torch.empty(flat.size + TAIL_ROWS * row_elems, dtype=torch.uint8, device="cuda")
        buf[flat.size:] = fill
        buf[:flat.size] = torch.from_numpy(flat).cuda()
    return buf[:flat.size].view(dtype).view(arr.shape)


def _inputs(d, r, packed, causal, seed):
    n = 128 + r
    if packed:
        return make_inputs(Run("tail", 2, 2, 0, d, causal, seed), lengths=[77, n])
    return make_inputs(Run("tail", 2, 2, n, d, causal, seed))


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("r", REMS)
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_reads_nothing_past_the_end(d, r, packed, causal):
    inp = _inputs(d, r, packed, causal, seed=900 + r)
    H = inp["H"]
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda() if packed else None
    nan_t = [_tail_view(inp[x], BF16_NAN, H * d, torch.bfloat16) for x in ("q", "k", "v")]
    zero_t = [_tail_view(inp[x], 0, H * d, torch.bfloat16) for x in ("q", "k", "v")]
    o_ref, l_ref = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=causal,
                                    cu_seqlens=inp["cu_seqlens"])
    # d = 128: fa_fwd picks 128-row tiles at this size; the 256-row instance
    # (fa_fwd_variant with the default exp and rescale) is checked too
    tiles = [{}] + ([dict(exp_mode=fa.EXP_HW, rescale_mode=fa.RESCALE_STRICT)] if d == 128 else [])
    for kw in tiles:
        o1, l1 = fa.fwd(*nan_t, causal=causal, scale=inp["scale"], cu_seqlens=cu, **kw)
        o0, l0 = fa.fwd(*zero_t, causal=causal, scale=inp["scale"], cu_seqlens=cu, **kw)
        torch.cuda.synchronize()
        what = f"d={d} N%64={r} packed={packed} causal={causal} {'fixed tile' if kw else 'fa_fwd'}"
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all(), what
        assert _same(o1, o0) and torch.equal(l1, l0), what
        assert_within(metrics(from_dev(o1), l1.cpu().numpy(), o_ref, l_ref), what)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("r", [1, 33])
def test_splitkv_and_masked_read_nothing_past_the_end(d, r):
    inp = _inputs(d, r, False, False, seed=950 + r)
    H = inp["H"]
    nan_t = [_tail_view(inp[x], BF16_NAN, H * d, torch.bfloat16) for x in ("q", "k", "v")]
    zero_t = [_tail_view(inp[x], 0, H * d, torch.bfloat16) for x in ("q", "k", "v")]
    outs = []
    for t in (nan_t, zero_t):
        s = fa.fwd_splitkv(*t, causal=False, scale=inp["scale"], splits=2)
        m = fa.fwd_masked(*t, window_left=40, window_right=-1, scale=inp["scale"])
        outs.append((s[0], s[1], m[0], m[1]))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.isfinite(a.float()).all()
        assert _same(a, b)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("r", REMS)
@pytest.mark.parametrize("packed", [False, True])
def test_bwd_reads_nothing_past_the_end(d, r, packed):
    inp = _inputs(d, r, packed, True, seed=970 + r)
    H = inp["H"]
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda() if packed else None
    do = make_grad(inp["q"].shape, 5970 + r)
    zq, zk, zv = (_tail_view(inp[x], 0, H * d, torch.bfloat16) for x in ("q", "k", "v"))
    o, lse = fa.fwd(zq, zk, zv, causal=True, scale=inp["scale"], cu_seqlens=cu)
    torch.cuda.synchronize()
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    grads = []
    for fill in (BF16_NAN, 0):
        t = [_tail_view(a, fill, H * d, torch.bfloat16) for a in (inp["q"], inp["k"], inp["v"], o_bits, do)]
        grads.append(fa.bwd(t[0], t[1], t[2], t[3], lse, t[4], causal=True, scale=inp["scale"],
                            cu_seqlens=cu))
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), *grads):
        assert torch.isfinite(a.float()).all(), f"{name} d={d} N%64={r} packed={packed}"
        assert _same(a, b), f"{name} d={d} N%64={r} packed={packed}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("r", [1, 33, 63])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_reads_nothing_past_the_end(d, r, causal):
    from oracle import fp8 as ofp8
    inp = _inputs(d, r, False, causal, seed=990 + r)
    H = inp["H"]
    q8, dq = ofp8.quantize(inp["q"])
    k8, dk = ofp8.quantize(inp["k"])
    vt8, dv = ofp8.quantize(inp["v"], transpose=True)
    scales = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (dq, dk, dv)]
    vt = torch.from_numpy(np.ascontiguousarray(vt8)).cuda()
    outs = []
    for fill in (E4M3_NAN, 0):
        tq = _tail_view(q8, fill, H * d, torch.uint8)
        tk = _tail_view(k8, fill, H * d, torch.uint8)
        outs.append(fa.fwd_fp8(tq, tk, vt, *scales, causal=causal, scale=inp["scale"]))
    torch.cuda.synchronize()
    (o1, l1), (o0, l0) = outs
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert _same(o1, o0) and torch.equal(l1, l0)

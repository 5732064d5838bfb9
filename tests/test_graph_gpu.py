"""The library's launches captured in HIP graphs (torch.cuda.CUDAGraph) and
replayed (needs an MI355X).

None of the entry points allocates, frees, synchronises or records a memset
when the caller passes every buffer, so each one can be captured.  Every test
captures one call, then replays the graph several times with eager work in
between (new input values copied into the captured buffers, outputs filled
with NaN) and a synchronisation after each replay; every replay must equal
the eager call on the same inputs bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import Run, make_grad, make_inputs
from gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _replays(sources, load, outputs, eager, call):
    """sources: input sets; load(src) copies one into the captured input
    buffers; eager(src) -> reference outputs; call() is the captured call
    writing `outputs`."""
    refs = [eager(s) for s in sources]
    load(sources[0])
    call()                      # warm-up outside the capture (first-use set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep, i in enumerate([0, 1, 0, 1]):
        load(sources[i])
        for t in outputs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, refs[i]):
            assert _same(got, want), f"replay {rep} (input set {i})"


def _dense(seed, B=2, H=3, N=700, d=128, causal=False):
    inp = make_inputs(Run("g", B, H, N, d, causal, seed))
    return {x: to_dev(inp[x]) for x in ("q", "k", "v")}, inp["scale"]


@pytest.mark.parametrize("causal", [False, True])
def test_graph_forward_dense(causal):
    srcs = [_dense(s, causal=causal)[0] for s in (501, 502)]
    scale = 1.0 / np.sqrt(128)
    q, k, v = (torch.empty_like(srcs[0][x]) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((2, 3, 700), dtype=torch.float32, device="cuda")

    def load(s):
        q.copy_(s["q"]); k.copy_(s["k"]); v.copy_(s["v"])
    _replays(srcs, load, [o, lse], lambda s: fa.fwd(s["q"], s["k"], s["v"], causal=causal, scale=scale),
             lambda: fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse))


def test_graph_forward_packed():
    lengths = [1, 0, 300, 129, 64]
    srcs = []
    for s in (503, 504):
        inp = make_inputs(Run("gp", len(lengths), 2, 0, 128, True, s, varlen=True), lengths=lengths)
        srcs.append({x: to_dev(inp[x]) for x in ("q", "k", "v")})
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], np.int32)).cuda()
    scale = inp["scale"]
    q, k, v = (torch.empty_like(srcs[0][x]) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((2, q.shape[0]), dtype=torch.float32, device="cuda")

    def load(s):
        q.copy_(s["q"]); k.copy_(s["k"]); v.copy_(s["v"])
    _replays(srcs, load, [o, lse],
             lambda s: fa.fwd(s["q"], s["k"], s["v"], causal=True, scale=scale, cu_seqlens=cu),
             lambda: fa.fwd(q, k, v, causal=True, scale=scale, cu_seqlens=cu, out=o, lse=lse))


def test_graph_splitkv_static_and_workspace():
    """The allocation-free split-KV entry point (its partials in the static
    scratch) and the workspace one, each captured; both equal the eager
    workspace call."""
    srcs = [_dense(s, B=1, H=2, N=3000)[0] for s in (505, 506)]
    scale = 1.0 / np.sqrt(128)
    S = 3
    q, k, v = (torch.empty_like(srcs[0][x]) for x in ("q", "k", "v"))

    def load(s):
        q.copy_(s["q"]); k.copy_(s["k"]); v.copy_(s["v"])

    def eager(s):
        return fa.fwd_splitkv(s["q"], s["k"], s["v"], scale=scale, splits=S)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 3000), dtype=torch.float32, device="cuda")
    _replays(srcs, load, [o, lse], eager,
             lambda: fa.fwd_splitkv_static(q, k, v, scale=scale, splits=S, out=o, lse=lse))
    op = torch.empty((S, 1, 3000, 2, 128), dtype=torch.float32, device="cuda")
    lp = torch.empty((S, 1, 2, 3000), dtype=torch.float32, device="cuda")
    _replays(srcs, load, [o, lse], eager,
             lambda: fa.fwd_splitkv(q, k, v, scale=scale, splits=S, out=o, lse=lse, o_part=op, lse_part=lp))


@pytest.mark.parametrize("causal", [False, True])
def test_graph_backward(causal):
    srcs = []
    for s in (507, 508):
        t, scale = _dense(s, B=1, H=2, N=500, causal=causal)
        t["do"] = to_dev(make_grad((1, 500, 2, 128), s + 5000))
        t["o"], t["lse"] = fa.fwd(t["q"], t["k"], t["v"], causal=causal, scale=scale)
        srcs.append(t)
    names = ("q", "k", "v", "o", "lse", "do")
    buf = {x: torch.empty_like(srcs[0][x]) for x in names}
    dq, dk, dv = (torch.empty_like(buf["q"]) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_floats(1, 2, 500), dtype=torch.float32, device="cuda")

    def load(s):
        for x in names:
            buf[x].copy_(s[x])
    _replays(srcs, load, [dq, dk, dv],
             lambda s: fa.bwd(s["q"], s["k"], s["v"], s["o"], s["lse"], s["do"], causal=causal, scale=scale),
             lambda: fa.bwd(buf["q"], buf["k"], buf["v"], buf["o"], buf["lse"], buf["do"], causal=causal,
                            scale=scale, dq=dq, dk=dk, dv=dv, workspace=ws))


def test_graph_fp8_and_masked():
    srcs = [_dense(s, B=1, H=2, N=600)[0] for s in (509, 510)]
    scale = 1.0 / np.sqrt(128)
    q, k, v = (torch.empty_like(srcs[0][x]) for x in ("q", "k", "v"))

    def load(s):
        q.copy_(s["q"]); k.copy_(s["k"]); v.copy_(s["v"])
    # FP8: quantisation and forward captured together
    q8, dq = fa.quantize_fp8(srcs[0]["q"])
    k8, dk = fa.quantize_fp8(srcs[0]["k"])
    vt8, dv = fa.quantize_fp8(srcs[0]["v"], transpose=True)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 600), dtype=torch.float32, device="cuda")

    def fp8_call(qq, kk, vv, out=None, l=None):
        fa.quantize_fp8(qq, out=q8, descale=dq)
        fa.quantize_fp8(kk, out=k8, descale=dk)
        fa.quantize_fp8(vv, transpose=True, out=vt8, descale=dv)
        return fa.fwd_fp8(q8, k8, vt8, dq, dk, dv, scale=scale, out=out, lse=l)

    def fp8_eager(s):
        a, b = fp8_call(s["q"], s["k"], s["v"])
        return a.clone(), b.clone()
    _replays(srcs, load, [o, lse], fp8_eager, lambda: fp8_call(q, k, v, o, lse))
    slopes = torch.tensor([0.5, 0.125], dtype=torch.float32, device="cuda")
    _replays(srcs, load, [o, lse],
             lambda s: fa.fwd_masked(s["q"], s["k"], s["v"], window_left=100, window_right=0,
                                     alibi_slopes=slopes, scale=scale),
             lambda: fa.fwd_masked(q, k, v, window_left=100, window_right=0, alibi_slopes=slopes, scale=scale,
                                   out=o, lse=lse))

"""Backward pass (fa_bwd), HIP path vs the fp64 oracle of the gradients,
through the C ABI (needs an MI355X).

The GPU forward's own O and LSE feed the GPU backward, as in training; the
oracle computes dQ, dK, dV from the definition in fp64.  Errors are measured
relative to each gradient's scale (the gradients' magnitudes shrink with the
sequence length, so absolute bounds would not mean the same at every size):
    rel_rms = ||g - ref||_2 / ||ref||_2,   rel_max = max|g - ref| / max|ref|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import RUNS, Run, make_grad, make_inputs
from gpu_helpers import from_dev, to_dev
from oracle.backward import attention_backward

pytestmark = pytest.mark.gpu

# bf16 P and dS feed the gradient products and bf16 rounds the outputs
# (relative 2^-9 each); see the backward section of the design notes.
GRAD_TOL_RMS = 1e-2
GRAD_TOL_MAX = 3e-2


def _inputs(d, causal, N, B=2, H=3, seed=61, sigma=1.0):
    inp = make_inputs(Run("bwd", B, H, N, d, causal, seed, sigma_qk=sigma))
    inp["do"] = make_grad(inp["q"].shape, seed + 5000)
    return inp


def _gpu(inp):
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"])
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=inp["causal"], scale=inp["scale"])
    torch.cuda.synchronize()
    return dq, dk, dv


def _grad_metrics(g, ref):
    diff = np.abs(g - ref)
    nref = float(np.linalg.norm(ref))
    return {
        "rel_rms": float(np.linalg.norm(diff)) / max(nref, 1e-300),
        "rel_max": float(diff.max()) / max(float(np.abs(ref).max()), 1e-300),
        "finite": bool(np.all(np.isfinite(g))),
    }


def _check(grads, refs, what):
    for name, g, ref in zip(("dQ", "dK", "dV"), grads, refs):
        g = from_dev(g) if isinstance(g, torch.Tensor) else g
        m = _grad_metrics(g, ref)
        print(f"{what} {name} {m}")
        assert m["finite"], f"{what} {name}: non-finite"
        if not np.any(ref):
            # exactly zero in exact arithmetic (one key: dS = P (dP - delta)
            # with dP and delta equal); fp32 leaves a rounding residue
            assert np.max(np.abs(g)) <= 1e-3, f"{what} {name}: expected zeros, got {np.max(np.abs(g))}"
            continue
        assert m["rel_rms"] <= GRAD_TOL_RMS, f"{what} {name}: rel_rms {m['rel_rms']:.3e}"
        assert m["rel_max"] <= GRAD_TOL_MAX, f"{what} {name}: rel_max {m['rel_max']:.3e}"


def _oracle(inp):
    return attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale=inp["scale"],
                              causal=inp["causal"])


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_ragged(d, causal):
    """Several key tiles and query blocks with ragged tails, every element."""
    inp = _inputs(d, causal, 300)
    _check(_gpu(inp), _oracle(inp), f"d={d} causal={causal}")


@pytest.mark.parametrize("N", [1, 31, 32, 33, 127, 128, 129, 255, 520])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_edge_lengths(N, causal):
    inp = _inputs(128, causal, N, B=1, H=2, seed=300 + N)
    _check(_gpu(inp), _oracle(inp), f"N={N} causal={causal}")


def test_bwd_wide_logits():
    """Scores of a few units (sigma 3 on Q and K): peaked softmax rows."""
    inp = _inputs(128, False, 400, B=1, H=2, seed=71, sigma=3.0)
    _check(_gpu(inp), _oracle(inp), "wide logits")


def test_bwd_zero_upstream_gradient():
    inp = _inputs(64, True, 200, B=1, H=2, seed=72)
    inp["do"] = np.zeros_like(inp["do"])
    for g in _gpu(inp):
        assert torch.count_nonzero(g.view(torch.int16)).item() == 0


def test_bwd_deterministic():
    inp = _inputs(128, True, 700, B=1, H=2, seed=73)
    a = _gpu(inp)
    b = _gpu(inp)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("N", [1, 33, 129, 160, 390])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d256_edge_lengths(N, causal):
    """d = 256 (two rows per direct load, one wave per SIMD; causal blocks
    above the diagonal run fully masked instead of being skipped)."""
    inp = _inputs(256, causal, N, B=1, H=2, seed=400 + N)
    _check(_gpu(inp), _oracle(inp), f"d=256 N={N} causal={causal}")


def test_bwd_rejects_other_head_dims():
    q = torch.zeros(1, 64, 1, 96, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError):
        fa.bwd(q, q.clone(), q.clone(), q.clone(), lse, q.clone())


@pytest.mark.parametrize("name", ["mid", "mid_causal", "wide_d256"])
def test_bwd_full_size_sampled_heads(name):
    """The benchmark's backward shapes at full size; two (b, h) heads are
    checked in full (each head's gradients depend on that head alone)."""
    run = RUNS[name]
    inp = make_inputs(run)
    inp["do"] = make_grad(inp["q"].shape, run.seed + 5000)
    dq, dk, dv = _gpu(inp)
    for b, h in ((0, 0), (run.B - 1, run.H - 1)):
        sl = {x: inp[x][b:b + 1, :, h:h + 1] for x in ("q", "k", "v", "do")}
        refs = attention_backward(sl["q"], sl["k"], sl["v"], sl["do"], scale=inp["scale"],
                                  causal=run.causal)
        grads = [from_dev(g[b:b + 1, :, h:h + 1]) for g in (dq, dk, dv)]
        _check(grads, refs, f"{name} b={b} h={h}")


# ---------------------------------------------------------------------------
# Packed sequences (cu_seqlens): each sequence is its own attention problem.

def _packed_inputs(lengths, d, causal, H=3, seed=81):
    r = Run("packed_bwd", len(lengths), H, 0, d, causal, seed, varlen=True)
    inp = make_inputs(r, lengths=lengths)
    inp["do"] = make_grad(inp["q"].shape, seed + 5000)
    return inp


def _gpu_packed(inp):
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "do"))
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], dtype=np.int32)).to("cuda")
    o, lse = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu)
    grads = fa.bwd(q, k, v, o, lse, do, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu)
    torch.cuda.synchronize()
    return grads


def _oracle_packed(inp):
    return attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], scale=inp["scale"],
                              causal=inp["causal"], cu_seqlens=inp["cu_seqlens"])


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_packed_small(d, causal):
    """Empty, one-token and ragged sequences in one packed batch, every element."""
    inp = _packed_inputs([1, 0, 5, 130, 257, 64, 300, 33], d, causal)
    _check(_gpu_packed(inp), _oracle_packed(inp), f"packed d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_packed_many_sequences(causal):
    """More than 64 sequences (the work decode walks them 64 at a time)."""
    rng = np.random.default_rng(82)
    lengths = [int(x) for x in rng.integers(0, 160, size=150)]
    inp = _packed_inputs(lengths, 64, causal, H=2, seed=83)
    _check(_gpu_packed(inp), _oracle_packed(inp), f"150 sequences causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_packed_equals_dense_bitwise(causal):
    """Each packed sequence gives bitwise the gradients of a dense run of it alone."""
    lengths = [37, 300, 129]
    inp = _packed_inputs(lengths, 128, causal, H=2, seed=84)
    packed = _gpu_packed(inp)
    cu = inp["cu_seqlens"]
    for b, n in enumerate(lengths):
        t0 = int(cu[b])
        one = {x: inp[x][None, t0:t0 + n] for x in ("q", "k", "v", "do")}
        one.update(causal=causal, scale=inp["scale"])
        dense = _gpu(one)
        for g_packed, g_dense in zip(packed, dense):
            assert torch.equal(g_packed[t0:t0 + n].view(torch.int16), g_dense[0].view(torch.int16))


def test_bwd_packed_workload_sampled():
    """The packed causal benchmark batch (32 sequences of 128..8192 tokens, 16
    heads) at full size; the two shortest sequences are checked in full for
    two heads each."""
    run = RUNS["varlen_causal"]
    inp = make_inputs(run)
    inp["do"] = make_grad(inp["q"].shape, run.seed + 5000)
    grads = _gpu_packed(inp)
    cu = inp["cu_seqlens"]
    lengths = np.diff(cu)
    for b in np.argsort(lengths, kind="stable")[:2]:
        t0, t1 = int(cu[b]), int(cu[b + 1])
        for h in (0, run.H - 1):
            sl = {x: inp[x][None, t0:t1, h:h + 1] for x in ("q", "k", "v", "do")}
            refs = attention_backward(sl["q"], sl["k"], sl["v"], sl["do"], scale=inp["scale"],
                                      causal=True)
            got = [from_dev(g[t0:t1, h:h + 1])[None] for g in grads]
            _check(got, refs, f"packed workload sequence {b} (n={t1 - t0}) h={h}")

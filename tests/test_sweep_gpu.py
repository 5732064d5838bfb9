"""Seeded random shapes through the forward, split-KV, masked and backward
entry points (needs an MI355X), each against the fp64 oracle element by
element.

The hand-picked cases fix one or two sizes at a time; here every draw mixes a
head dimension, a head count of 1-5, a batch of 1-3 (or 1-6 packed sequences,
empty and one-token ones included), lengths up to 420 (several query and key
tiles with a ragged tail), causal or not, unit or wide logits, key-range
counts and window edges.  The draws come from fixed seeds, so a failure names
its case and repeats.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import Run, make_grad, make_inputs
from gpu_helpers import assert_within, from_dev, metrics, to_dev
from oracle import mods as omods
from oracle.backward import attention_backward

pytestmark = pytest.mark.gpu

CASES = 40
MAX_N = 420
# gradient tolerances of the backward tests (bf16 P and dS, bf16 outputs)
GRAD_TOL_RMS = 1e-2
GRAD_TOL_MAX = 3e-2


def _draw(seed: int):
    """One random problem: the inputs dict (dense or packed) and a label."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d = int(rng.choice([64, 128, 256]))
    H = int(rng.integers(1, 6))
    causal = bool(rng.integers(2))
    sigma = float(rng.choice([1.0, 3.0]))
    if rng.integers(2):
        lengths = [int(x) for x in rng.integers(0, MAX_N, int(rng.integers(1, 7)))]
        if rng.integers(3) == 0:
            lengths[int(rng.integers(len(lengths)))] = int(rng.choice([0, 1]))
        if sum(lengths) == 0:
            lengths[0] = 1
        inp = make_inputs(Run(f"sweep{seed}", len(lengths), H, 0, d, causal, seed, sigma_qk=sigma,
                              varlen=True), lengths=lengths)
        label = f"seed={seed} d={d} H={H} causal={causal} sigma={sigma} packed lengths={lengths}"
    else:
        B, N = int(rng.integers(1, 4)), int(rng.integers(1, MAX_N))
        inp = make_inputs(Run(f"sweep{seed}", B, H, N, d, causal, seed, sigma_qk=sigma))
        label = f"seed={seed} d={d} H={H} causal={causal} sigma={sigma} B={B} N={N}"
    return inp, rng, label


def _dev(inp):
    q, k, v = (to_dev(inp[x]) for x in ("q", "k", "v"))
    cu = inp.get("cu_seqlens")
    return q, k, v, (torch.from_numpy(np.asarray(cu, np.int32)).cuda() if cu is not None else None)


def _tokens(inp):
    return int(inp["cu_seqlens"][-1]) if inp.get("cu_seqlens") is not None else int(inp["q"].shape[1])


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_forward(case):
    """fa_fwd (at d = 128 also the fixed 256-row tile, bitwise)."""
    inp, _, label = _draw(1000 + case)
    q, k, v, cu = _dev(inp)
    o, lse = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu)
    torch.cuda.synchronize()
    print(label, flush=True)
    ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=inp["causal"],
                              cu_seqlens=inp.get("cu_seqlens"))
    assert_within(metrics(from_dev(o), lse.cpu().numpy(), ro, rl), label)
    if inp["d"] == 128:
        o8, l8 = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu,
                        exp_mode=fa.EXP_HW, rescale_mode=fa.RESCALE_STRICT)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o8.view(torch.int16)) and torch.equal(lse, l8), label


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_splitkv(case):
    """fa_fwd_splitkv / fa_fwd_splitkv_packed with a random range count."""
    inp, rng, label = _draw(2000 + case)
    q, k, v, cu = _dev(inp)
    S = int(rng.integers(1, min(6, (_tokens(inp) + 63) // 64) + 1))
    label += f" splits={S}"
    print(label, flush=True)
    if cu is None:
        o, lse = fa.fwd_splitkv(q, k, v, causal=inp["causal"], scale=inp["scale"], splits=S)
    else:
        o, lse = fa.fwd_splitkv_packed(q, k, v, cu, causal=inp["causal"], scale=inp["scale"], splits=S)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=inp["causal"],
                              cu_seqlens=inp.get("cu_seqlens"))
    assert_within(metrics(from_dev(o), lse.cpu().numpy(), ro, rl), label)


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_masked(case):
    """fa_fwd_masked / fa_fwd_masked_packed with random window edges and,
    half the time, ALiBi slopes."""
    inp, rng, label = _draw(3000 + case)
    q, k, v, cu = _dev(inp)
    n = _tokens(inp)
    left = -1 if rng.integers(3) == 0 else int(rng.integers(0, n + 2))
    right = -1 if rng.integers(3) == 0 else int(rng.integers(0, n + 2))
    H = inp["H"]
    slopes = (np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], np.float32)
              if rng.integers(2) else None)
    label += f" window=({left}, {right}) alibi={slopes is not None}"
    print(label, flush=True)
    sl = torch.from_numpy(slopes).cuda() if slopes is not None else None
    if cu is None:
        o, lse = fa.fwd_masked(q, k, v, window_left=left, window_right=right, alibi_slopes=sl,
                               scale=inp["scale"])
        ro, rl = omods.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], left=left, right=right,
                                 slopes=slopes)
    else:
        o, lse = fa.fwd_masked_packed(q, k, v, cu, window_left=left, window_right=right, alibi_slopes=sl,
                                      scale=inp["scale"])
        ro, rl = omods.attention_packed(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], scale=inp["scale"],
                                        left=left, right=right, slopes=slopes)
    torch.cuda.synchronize()
    assert_within(metrics(from_dev(o), lse.cpu().numpy(), ro, rl), label)


@pytest.mark.parametrize("case", range(CASES // 2))
def test_sweep_backward(case):
    """fa_bwd (dense or packed) after fa_fwd: dQ, dK, dV against the fp64
    gradients."""
    inp, _, label = _draw(4000 + case)
    q, k, v, cu = _dev(inp)
    do_bits = make_grad(inp["q"].shape, 9000 + case)
    do = to_dev(do_bits)
    print(label, flush=True)
    o, lse = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu)
    grads = fa.bwd(q, k, v, o, lse, do, causal=inp["causal"], scale=inp["scale"], cu_seqlens=cu)
    torch.cuda.synchronize()
    refs = attention_backward(inp["q"], inp["k"], inp["v"], do_bits, scale=inp["scale"], causal=inp["causal"],
                              cu_seqlens=inp.get("cu_seqlens"))
    for name, g, ref in zip(("dQ", "dK", "dV"), grads, refs):
        g = from_dev(g)
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite"
        if not np.any(ref):
            assert np.max(np.abs(g)) <= 1e-3, f"{label} {name}: expected zeros"
            continue
        diff = np.abs(g - ref)
        rel_rms = float(np.linalg.norm(diff)) / float(np.linalg.norm(ref))
        rel_max = float(diff.max()) / float(np.abs(ref).max())
        assert rel_rms <= GRAD_TOL_RMS and rel_max <= GRAD_TOL_MAX, \
            f"{label} {name}: rel_rms {rel_rms:.3e} rel_max {rel_max:.3e}"


@pytest.mark.parametrize("case", range(CASES // 2))
def test_sweep_fp8(case):
    """fa_fwd_fp8 on dense draws: every element within the E4M3 error bound
    of the FP8 tests (quantisation as the oracle defines it)."""
    from test_fp8_gpu import _all_rows, _check_rows, _quantized, _run_fp8
    rng = np.random.Generator(np.random.PCG64(5000 + case))
    d = int(rng.choice([64, 128, 256]))
    B, H, N = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, MAX_N))
    causal = bool(rng.integers(2))
    sigma = float(rng.choice([1.0, 3.0]))
    inp = make_inputs(Run(f"sweep8_{case}", B, H, N, d, causal, 5000 + case, sigma_qk=sigma))
    label = f"fp8 seed={5000 + case} d={d} B={B} H={H} N={N} causal={causal} sigma={sigma}"
    print(label, flush=True)
    qz = _quantized(inp)
    o, lse = _run_fp8(*qz, inp["scale"], causal)
    _check_rows(inp, causal, *qz, o, lse, _all_rows(B, H, N), label)

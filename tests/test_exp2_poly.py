"""The FMA-polynomial exp2 of the kernel, checked on the CPU.

The FlashAttention V4 explainer (section 3.2) evaluates part of the
exponentials with a polynomial on the FMA units; the kernel's EXP_POLY and
EXP_MIXED variants do the same with a cubic minimax fit of 2^f on [0, 1).
These tests read the coefficients out of the kernel source, re-derive them
with the generator, and emulate the kernel's fp32 evaluation (clamp, floor,
Horner with fused multiply-adds, exponent-field add) to bound its error and
pin the special values the attention relies on.
"""
from __future__ import annotations

import os
import re
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_107_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_exp2_poly  # noqa: E402


def kernel_coefficients():
    src = open(os.path.join(CSRC, "fa_kernel.hpp")).read()
    body = re.search(r"float exp2_poly\(float x\) \{(.*?)\n\}", src, re.S).group(1)
    c3, c2 = (float(v) for v in re.search(
        r"__builtin_fmaf\(f, ([0-9.e+-]+)f, ([0-9.e+-]+)f\)", body).groups())
    c1 = float(re.search(r"__builtin_fmaf\(f, p, ([0-9.e+-]+)f\);\n\s*p = __builtin_fmaf\(f, p, 1\.0f\)",
                         body).group(1))
    return np.float32(c1), np.float32(c2), np.float32(c3)


def fma32(a, b, c):
    """fp32 fused multiply-add: the fp32 x fp32 product is exact in fp64."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(np.float32)


def exp2_poly_host(x):
    """Host emulation of the kernel's exp2_poly, step for step in fp32."""
    c1, c2, c3 = kernel_coefficients()
    x = np.maximum(np.asarray(x, np.float32), np.float32(-127.0))
    n = np.floor(x).astype(np.float32)
    f = (x - n).astype(np.float32)
    p = fma32(f, c3, c2)
    p = fma32(f, p, c1)
    p = fma32(f, p, np.float32(1.0))
    bits = p.view(np.int32).astype(np.int64) + (n.astype(np.int64) << 23)
    return bits.astype(np.int32).view(np.float32)


def test_coefficients_are_the_generators():
    c, err = gen_exp2_poly.remez_fixed_c0(3)
    ours = kernel_coefficients()
    for k in range(3):
        assert ours[k] == np.float32(c[k + 1]), f"c{k + 1}: kernel {ours[k]!r} vs derived {c[k + 1]!r}"
    assert err < 1e-4


def test_relative_error_over_the_score_range():
    # scaled scores minus the reference max lie in [-inf, tau = 8]; below
    # -126 the result is far under bf16's resolution of the row's largest term
    x = np.linspace(-126.0, 8.0, 1 << 22, dtype=np.float32)
    y = exp2_poly_host(x).astype(np.float64)
    rel = np.abs(y / np.exp2(x.astype(np.float64)) - 1.0)
    assert rel.max() < 1.2e-4          # the fit's 8.6e-5 plus fp32 rounding
    assert rel.max() < 2.0 ** -9       # below bf16's rounding of P


def test_special_values():
    ninf = np.float32(-np.inf)
    vals = exp2_poly_host(np.array([ninf, -1e30, -200.0, -127.5, -127.0], np.float32))
    assert np.all(vals == 0.0) and not np.any(np.signbit(vals))  # masked scores give +0
    ints = np.arange(-126, 9, dtype=np.float32)
    assert np.array_equal(exp2_poly_host(ints), np.exp2(ints))   # p(0) = 1: exact powers of two
    assert exp2_poly_host(np.float32(8.0)) == np.float32(256.0)  # the threshold bound 2^tau


def test_monotone_on_each_unit_interval():
    f = np.linspace(0.0, 1.0, 1 << 16, endpoint=False, dtype=np.float32)
    y = exp2_poly_host(f - np.float32(3.0))
    assert np.all(np.diff(y.astype(np.float64)) >= 0.0)


@pytest.mark.parametrize("x", [-0.75, -12.3, 3.999, 7.5])
def test_matches_exp2_pointwise(x):
    y = float(exp2_poly_host(np.float32(x)))
    assert abs(y / 2.0 ** float(np.float32(x)) - 1.0) < 1.2e-4

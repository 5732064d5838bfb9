"""Seeded synthetic inputs for the attention forward.

This module only draws random numbers and rounds them to bf16; it holds none
of the attention arithmetic, so both the HIP path's tests and the CPU oracle
can take their inputs from it.

The pages give no workload shapes; the runs below are the library's own test
and benchmark set (dense, causal, long causal, packed variable-length causal,
a wide-logit stress input, and few-head long sequences for the split of the
key sequence).  Every draw is numpy ``Generator(PCG64(seed))``
fp32 ``standard_normal`` (times sigma where stated), then rounded once to
bf16 round-to-nearest-even.  Tensor order is Q, K, V.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Run:
    """One benchmark/parity run."""
    name: str
    B: int            # batch, or number of packed sequences
    H: int
    N: int            # sequence length (dense) or total tokens (packed)
    d: int
    causal: bool
    seed: int
    sigma_qk: float = 1.0
    boost_frac: float = 0.0   # fraction of K rows per (b, h) scaled by 8
    varlen: bool = False
    len_lo: int = 0           # packed lengths drawn uniform in [len_lo, len_hi]
    len_hi: int = 0

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The library's run set.  ``N`` of the packed run is filled in from its seed.
RUNS = {
    "tiny": Run("tiny", 1, 1, 128, 64, False, 1001),
    "tiny_causal": Run("tiny_causal", 1, 1, 128, 64, True, 1001),
    "mid": Run("mid", 4, 16, 2048, 128, False, 1002),
    "mid_causal": Run("mid_causal", 4, 16, 2048, 128, True, 1002),
    "long_causal": Run("long_causal", 1, 32, 16384, 128, True, 1003),
    "varlen_causal": Run("varlen_causal", 32, 16, 0, 128, True, 1004,
                         varlen=True, len_lo=128, len_hi=8192),
    "wide": Run("wide", 2, 16, 8192, 128, False, 1005, sigma_qk=3.0, boost_frac=0.01),
    "wide_d64": Run("wide_d64", 2, 16, 4096, 64, False, 1005, sigma_qk=3.0, boost_frac=0.01),
    "wide_d256": Run("wide_d256", 2, 16, 4096, 256, False, 1005, sigma_qk=3.0, boost_frac=0.01),
    # few (batch, head) pairs over long sequences: too few query tiles to fill
    # the GPU, the shape the split of the key sequence is for
    "few_heads": Run("few_heads", 1, 4, 8192, 128, False, 1006),
    "few_heads_causal": Run("few_heads_causal", 1, 4, 16384, 128, True, 1007),
    # backward pass at the forward's long shape, N(0,1) inputs
    "bwd_long": Run("bwd_long", 2, 16, 8192, 128, False, 1008),
    "bwd_long_causal": Run("bwd_long_causal", 2, 16, 8192, 128, True, 1008),
}


def packed_lengths(rng: np.random.Generator, count: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=count).astype(np.int64)


def make_inputs(run: Run, *, B: int | None = None, H: int | None = None,
                N: int | None = None, lengths=None, seed: int | None = None):
    """Draw Q, K, V for ``run`` (optionally overriding sizes or the seed).

    Returns a dict with ``q, k, v`` (uint16 bf16 bits, ``[B, N, H, d]`` or
    ``[T, H, d]``), ``cu_seqlens`` (int32 or None), ``lengths`` and the scalar
    parameters.
    """
    B = run.B if B is None else B
    H = run.H if H is None else H
    d = run.d
    rng = np.random.Generator(np.random.PCG64(run.seed if seed is None else seed))
    if run.varlen or lengths is not None:
        if lengths is None:
            lengths = packed_lengths(rng, B, run.len_lo, run.len_hi)
        lengths = np.asarray(lengths, dtype=np.int64)
        B = len(lengths)
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        T = int(cu[-1])
        shape = (T, H, d)
    else:
        N = run.N if N is None else N
        lengths = np.full(B, N, dtype=np.int64)
        cu = None
        shape = (B, N, H, d)

    def draw(sigma):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        return x

    q = draw(run.sigma_qk)
    k = draw(run.sigma_qk)
    if run.boost_frac > 0:
        for b in range(B):
            n = int(lengths[b])
            cnt = int(math.floor(run.boost_frac * n))
            for h in range(H):
                idx = rng.choice(n, size=cnt, replace=False)
                if cu is None:
                    k[b, idx, h, :] *= np.float32(8.0)
                else:
                    k[int(cu[b]) + idx, h, :] *= np.float32(8.0)
    v = draw(1.0)
    return {
        "q": bf16_bits(q), "k": bf16_bits(k), "v": bf16_bits(v),
        "cu_seqlens": cu, "lengths": lengths, "B": B, "H": H,
        "N": int(shape[1]) if cu is None else int(lengths.max()),
        "T": int(np.prod(shape[:-2])) if cu is None else int(cu[-1]),
        "d": d, "scale": run.scale, "causal": run.causal,
    }


def make_grad(shape, seed: int) -> np.ndarray:
    """Upstream gradient dO for the backward pass: N(0,1) drawn from its own
    ``Generator(PCG64(seed))``, rounded once to bf16; returns the bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits(rng.standard_normal(size=tuple(shape), dtype=np.float32))


def bwd_flops(run_or_lengths, H: int, d: int, causal: bool) -> float:
    """Credited backward FLOPs: the five n x n x d products of the gradient
    (S recomputed, dP, dV, dK, dQ) = 10*n^2*d per (sequence, head), halved
    when causal -- 2.5 times the forward's credit."""
    return 2.5 * flops(run_or_lengths, H, d, causal)


def flops(run_or_lengths, H: int, d: int, causal: bool) -> float:
    """Credited FLOPs: 4*n^2*d per (sequence, head), halved when causal."""
    lengths = np.asarray(run_or_lengths, dtype=np.float64)
    f = 4.0 * H * d * float(np.sum(lengths * lengths))
    return f / 2 if causal else f

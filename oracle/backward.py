"""fp64 gradients of exact attention: the oracle of the backward pass.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the HIP backward is
checked against it; the product path never imports it.

The pages treat the backward pass only qualitatively: the attention weights
are recomputed from the saved statistics instead of being stored
(FlashAttention 1-4 post, summary table, FlashAttention-1 column;
"Understanding FlashAttention V4", section 2.2), and FlashAttention-4 keeps
its intermediates on chip and offers a deterministic mode (same page,
section 3.3).  None of them writes the gradient out.  The plainest reading,
taken here, is the exact gradient of the forward definition
O = softmax(scale * Q K^T) V with respect to Q, K and V for an upstream
gradient dO, written out per (sequence, head) with one materialised n x n
score matrix:

    S  = scale * Q K^T          (masked entries -inf when causal)
    P  = softmax_rows(S)
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))        (softmax Jacobian, row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

rowsum(P * dP) equals rowsum(dO * O); the GPU computes it that way from the
forward output, this oracle from P and dP (the two agree in exact arithmetic).
"""
from __future__ import annotations

import numpy as np

from . import _widen


def _one_head(Q, K, V, dO, scale, causal):
    n = Q.shape[0]
    S = (Q @ K.T) * scale
    if causal:
        S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    m = np.max(S, axis=1, keepdims=True)
    E = np.exp(S - m)
    P = E / np.sum(E, axis=1, keepdims=True)
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    return dQ, dK, dV


def attention_backward(q, k, v, do, *, scale: float, causal: bool, cu_seqlens=None):
    """dQ, dK, dV (float64, shaped like q) of exact attention.

    q, k, v, do  uint16 bf16 bit patterns (widened exactly) or float arrays,
                 ``[B, N, H, d]`` dense or ``[T, H, d]`` packed with
                 ``cu_seqlens`` (int32, ``B+1`` offsets).
    scale        the fp32 softmax scale, widened to double as given.
    """
    Q, K, V, dO = (_widen(x) for x in (q, k, v, do))
    if not (Q.shape == K.shape == V.shape == dO.shape):
        raise ValueError("q, k, v and do must have the same shape")
    sc = float(np.float32(scale))
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    if cu_seqlens is None:
        if Q.ndim != 4:
            raise ValueError("dense inputs are [B, N, H, d]")
        B, N, H, _ = Q.shape
        for b in range(B):
            for h in range(H):
                g = _one_head(Q[b, :, h], K[b, :, h], V[b, :, h], dO[b, :, h], sc, causal)
                dQ[b, :, h], dK[b, :, h], dV[b, :, h] = g
    else:
        if Q.ndim != 3:
            raise ValueError("packed inputs are [T, H, d]")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        H = Q.shape[1]
        for b in range(len(cu) - 1):
            t0, t1 = int(cu[b]), int(cu[b + 1])
            if t1 <= t0:
                continue
            for h in range(H):
                g = _one_head(Q[t0:t1, h], K[t0:t1, h], V[t0:t1, h], dO[t0:t1, h], sc, causal)
                dQ[t0:t1, h], dK[t0:t1, h], dV[t0:t1, h] = g
    return dQ, dK, dV

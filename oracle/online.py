"""The pages' tiled online-softmax recurrence, in fp64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): a second, independent
route to the same result, used to pin the definition oracle.

Follows the FlashAttention-1 derivation of the "FlashAttention 1-4 explained"
post (online softmax equation block): for each query block, walk the key/value
blocks carrying the running row max m, the running sum l and the unnormalised
output O,

    m_new = max(m, rowmax(S_ij))
    P~    = exp(S_ij - m_new)
    l_new = exp(m - m_new) * l + rowsum(P~)
    O_new = exp(m - m_new) * O + P~ V_j

and divide by l once at the end (the FlashAttention-2 deferred
normalisation).  ``rescale`` selects how the correction factor is applied:

* ``"always"``    every block, as written above;
* ``"strict"``    only rows whose max grew (FlashAttention-4 conditional
                  rescale, "only when m_new > m"); the skipped factor is
                  exactly 1, so the result is unchanged;
* ``"threshold"`` keep the stale reference max unless the block's max exceeds
                  it by more than ``tau`` (natural-log units), the "only when
                  overflow is possible" reading of the explainer's section 3.2.
                  O and l always share one reference, so the result is exact.
"""
from __future__ import annotations

import numpy as np


def _widen(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def online_attention(q, k, v, *, scale: float, causal: bool, Br: int, Bc: int,
                     rescale: str = "always", tau: float = 8.0):
    """One head.  q, k, v: ``[n, d]`` (uint16 bf16 bits, or float arrays).

    Returns ``(o [n, d], lse [n], n_rescaled_rows)`` in float64.
    """
    if rescale not in ("always", "strict", "threshold"):
        raise ValueError(rescale)
    to64 = (lambda a: _widen(a)) if np.asarray(q).dtype == np.uint16 else \
        (lambda a: np.asarray(a, dtype=np.float64))
    Q, K, V = to64(q), to64(k), to64(v)
    n, d = Q.shape
    sc = float(np.float32(scale))
    O = np.zeros((n, d))
    lse = np.zeros(n)
    rescaled = 0
    for i0 in range(0, n, Br):
        i1 = min(i0 + Br, n)
        Qi = Q[i0:i1]
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        Oi = np.zeros((i1 - i0, d))
        for j0 in range(0, n, Bc):
            j1 = min(j0 + Bc, n)
            S = (Qi @ K[j0:j1].T) * sc
            if causal:
                qi = np.arange(i0, i1)[:, None]
                kj = np.arange(j0, j1)[None, :]
                S = np.where(kj <= qi, S, -np.inf)
            rowmax = S.max(axis=1)
            if rescale == "threshold":
                grow = rowmax > m + tau
                # the first finite block always sets the reference
                grow |= np.isneginf(m) & np.isfinite(rowmax)
                m_new = np.where(grow, rowmax, m)
            else:
                m_new = np.maximum(m, rowmax)
                grow = m_new > m
            ref = np.where(np.isneginf(m_new), 0.0, m_new)
            P = np.exp(S - ref[:, None])
            alpha = np.exp(np.where(np.isneginf(m), -np.inf, m) - ref)
            if rescale == "always":
                l = alpha * l + P.sum(axis=1)
                Oi = alpha[:, None] * Oi + P @ V[j0:j1]
            else:
                # rows that keep their reference skip the correction
                a = np.where(grow, alpha, 1.0)
                l = a * l + P.sum(axis=1)
                Oi = a[:, None] * Oi + P @ V[j0:j1]
            rescaled += int(np.count_nonzero(grow & ~np.isneginf(m)))
            m = m_new
        O[i0:i1] = Oi / l[:, None]
        lse[i0:i1] = m + np.log(l)
    return O, lse, rescaled

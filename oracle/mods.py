"""Attention with a window mask and a linear position bias: the oracle of the
masked entry point.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

The pages mention only that FlashAttention-4 serves as a backend of PyTorch's
FlexAttention (FlashAttention 1-4 post, FlashAttention-4 section; the
reportify summary, notes [24] and [27]), whose user code rewrites scores
(a score modification) or hides key positions (a mask).  No particular
modification is named.  Two common ones are taken here, written out as
definitions:

* window mask: key j is visible to query i iff ``i - left <= j <= i + right``
  (a negative bound means unbounded on that side; ``right = 0`` with an
  unbounded left side is the causal mask);
* linear bias by distance (ALiBi): the scaled score gets ``slope_h * (j - i)``
  added, one slope per head.

    s_ij = scale * q_i . k_j + slope_h * (j - i)      for visible j
    O_i = softmax_j(s_ij) V,  LSE_i = ln sum_j exp(s_ij)

A row with no visible key gets O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np

from . import _widen


def visible(i, j, n, left, right):
    """Boolean visibility of key j to query i (broadcasting)."""
    ok = (j >= 0) & (j < n)
    if left >= 0:
        ok = ok & (j >= i - left)
    if right >= 0:
        ok = ok & (j <= i + right)
    return ok


def attention(q, k, v, *, scale: float, left: int = -1, right: int = -1, slopes=None, rows=None):
    """fp64 attention of dense ``[B, N, H, d]`` bf16 bit patterns (or floats)
    under the window mask and the optional per-head slopes ``[H]``.

    Returns ``(o [B, N, H, d], lse [B, H, N])``, or for ``rows`` (``(n, 3)``
    triples (b, h, i)) ``(o [n, d], lse [n])``.
    """
    Q, K, V = (_widen(x) for x in (q, k, v))
    B, N, H, d = Q.shape
    sc = float(np.float32(scale))
    sl = np.zeros(H) if slopes is None else np.asarray(slopes, np.float32).astype(np.float64)
    keys = np.arange(N)

    def one(b, h, i):
        s = (K[b, :, h] @ Q[b, i, h]) * sc + sl[h] * (keys - i)
        vis = visible(i, keys, N, left, right)
        if not vis.any():
            return np.zeros(d), -np.inf
        s = np.where(vis, s, -np.inf)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        return (e / l) @ V[b, :, h], m + np.log(l)

    if rows is None:
        o = np.zeros((B, N, H, d))
        lse = np.zeros((B, H, N))
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    o[b, i, h], lse[b, h, i] = one(b, h, i)
        return o, lse
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for r, (b, h, i) in enumerate(rows):
        o[r], lse[r] = one(b, h, i)
    return o, lse


def attention_packed(q, k, v, cu_seqlens, *, scale: float, left: int = -1, right: int = -1, slopes=None,
                     rows=None):
    """The same definition over packed sequences: ``q, k, v [T, H, d]`` with
    sequence b holding tokens ``cu[b] .. cu[b+1]-1``; positions i, j (window
    and bias) count from the sequence's first token, and a query sees only its
    own sequence's keys.

    Returns ``(o [T, H, d], lse [H, T])``, or for ``rows`` (``(n, 3)``
    triples (b, h, i), i within sequence b) ``(o [n, d], lse [n])``.
    """
    Q, K, V = (_widen(x) for x in (q, k, v))
    T, H, d = Q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n_seq = np.diff(cu)
    if cu[0] != 0 or np.any(n_seq < 0) or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    sc = float(np.float32(scale))
    sl = np.zeros(H) if slopes is None else np.asarray(slopes, np.float32).astype(np.float64)

    def one(b, h, i):
        t0, n = int(cu[b]), int(n_seq[b])
        keys = np.arange(n)
        s = (K[t0:t0 + n, h] @ Q[t0 + i, h]) * sc + sl[h] * (keys - i)
        vis = visible(i, keys, n, left, right)
        if not vis.any():
            return np.zeros(d), -np.inf
        s = np.where(vis, s, -np.inf)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        return (e / l) @ V[t0:t0 + n, h], m + np.log(l)

    if rows is None:
        o = np.zeros((T, H, d))
        lse = np.zeros((H, T))
        for b in range(len(n_seq)):
            for h in range(H):
                for i in range(int(n_seq[b])):
                    o[cu[b] + i, h], lse[h, cu[b] + i] = one(b, h, i)
        return o, lse
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for r, (b, h, i) in enumerate(rows):
        if not 0 <= i < n_seq[b]:
            raise ValueError("row index outside its sequence")
        o[r], lse[r] = one(b, h, i)
    return o, lse

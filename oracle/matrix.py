"""Exact attention forward in fp64 as whole-matrix products (torch CPU ops).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the product path
never imports it.

The same definition as :func:`oracle.attention` (the compute chain of
section 1.1 of the FlashAttention V4 explainer; the "standard attention"
equations of the FlashAttention 1-4 post), written with library matrix
products so that full-size outputs can be checked on every row in about a
minute of host time:

    for each sequence b and head h, and a block of query rows i:
        S   = (Q_i K^T) * scale           torch.matmul in float64
        S_ij = -inf where key j is hidden  (j >= n; causal: j > i; outside
                                            the key range)
        m_i = max_j S_ij
        E   = exp(S - m)                   (exp(-inf) = 0)
        l_i = sum_j E_ij
        O_i = (E / l) V                    torch.matmul in float64
        LSE_i = m_i + ln l_i

Query rows are independent, so taking them a block at a time changes no
result beyond the rounding order of the library's sums; rows that see no
key get O = 0 and LSE = -inf.  Inputs are the same bf16 bit patterns as the
C oracle's, widened exactly to float64; ``scale`` is the fp32 value widened.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _widen, all_rows

ROW_BLOCK = 1024


def _spans(q, cu_seqlens):
    """(start token, length) of every sequence, and the layout kind."""
    if cu_seqlens is None:
        if q.ndim != 4:
            raise ValueError("dense inputs are [B, N, H, d]")
        B, N = q.shape[0], q.shape[1]
        return [(b * N, N) for b in range(B)], False
    if q.ndim != 3:
        raise ValueError("packed inputs are [T, H, d]")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lengths = np.diff(cu)
    if cu[0] != 0 or np.any(lengths < 0) or int(cu[-1]) != q.shape[0]:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return [(int(cu[b]), int(lengths[b])) for b in range(len(lengths))], True


def _head(x, t0, n, h):
    """Rows t0 .. t0+n-1 of head h as a float64 torch tensor [n, d]."""
    flat = x.reshape(-1, x.shape[-2], x.shape[-1])
    return torch.from_numpy(_widen(flat[t0:t0 + n, h, :]))


def head_attention(qh, kh, vh, *, scale: float, causal: bool, rows=None, key_range=None,
                   row_block: int = ROW_BLOCK):
    """Attention of one (sequence, head): ``qh, kh, vh`` float64 ``[n, d]``.
    ``rows``: query indices (default all).  Returns float64 numpy
    ``o [len(rows), d]`` and ``lse [len(rows)]``."""
    n, d = kh.shape
    sc = float(np.float32(scale))
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    lo, hi = (0, n) if key_range is None else (max(0, int(key_range[0])), min(n, int(key_range[1])))
    o = np.zeros((len(rows), vh.shape[1]))
    lse = np.full(len(rows), -np.inf)
    if hi <= lo or len(rows) == 0:
        return o, lse
    keys = torch.arange(lo, hi)
    for r0 in range(0, len(rows), row_block):
        ri = torch.from_numpy(rows[r0:r0 + row_block])
        k_end = min(hi, int(ri.max()) + 1) if causal else hi
        if k_end <= lo:
            continue
        S = (qh[ri] @ kh[lo:k_end].T) * sc
        if causal:
            S = S.masked_fill(keys[None, :k_end - lo] > ri[:, None], float("-inf"))
        m = S.max(dim=1).values
        seen = torch.isfinite(m)
        E = torch.exp(S - torch.where(seen, m, torch.zeros_like(m))[:, None])
        l = E.sum(dim=1)
        ob = (E / torch.where(seen, l, torch.ones_like(l))[:, None]) @ vh[lo:k_end]
        o[r0:r0 + len(ri)] = ob.numpy()
        lse[r0:r0 + len(ri)] = torch.where(seen, m + torch.log(l), m).numpy()
    return o, lse


def iter_heads(q, k, v, *, scale: float, causal: bool, cu_seqlens=None, key_range=None):
    """Yields ``(b, h, o [n, d], lse [n])`` for every sequence and head, one
    head at a time (bounded memory for full-size checks)."""
    spans, _ = _spans(q, cu_seqlens)
    H = q.shape[-2]
    for b, (t0, n) in enumerate(spans):
        for h in range(H):
            if n == 0:
                yield b, h, np.zeros((0, q.shape[-1])), np.zeros(0)
                continue
            o, lse = head_attention(_head(q, t0, n, h), _head(k, t0, n, h), _head(v, t0, n, h),
                                    scale=scale, causal=causal, key_range=key_range)
            yield b, h, o, lse


def attention(q, k, v, *, scale: float, causal: bool, cu_seqlens=None, rows=None,
              key_range=None, **_unused):
    """Same arguments and results as :func:`oracle.attention` (layouts,
    ``rows`` triples, ``key_range``)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have the same shape")
    spans, packed = _spans(q, cu_seqlens)
    H, d = q.shape[-2], q.shape[-1]
    full = rows is None
    if full:
        rows = all_rows(len(spans), H, [n for _, n in spans])
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for b, h in {(int(b), int(h)) for b, h in rows[:, :2]}:
        sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
        t0, n = spans[b]
        if np.any(rows[sel, 2] >= n) or np.any(rows[sel, 2] < 0):
            raise ValueError("row index outside its sequence")
        ob, lb = head_attention(_head(q, t0, n, h), _head(k, t0, n, h), _head(v, t0, n, h),
                                scale=scale, causal=causal, rows=rows[sel, 2], key_range=key_range)
        o[sel] = ob
        lse[sel] = lb
    if not full:
        return o, lse
    o_full = np.zeros(q.shape)
    if not packed:
        B, N = q.shape[0], q.shape[1]
        lse_full = np.zeros((B, H, N))
        o_full[rows[:, 0], rows[:, 2], rows[:, 1], :] = o
        lse_full[rows[:, 0], rows[:, 1], rows[:, 2]] = lse
    else:
        lse_full = np.zeros((H, q.shape[0]))
        starts = np.array([t0 for t0, _ in spans], dtype=np.int64)
        tok = starts[rows[:, 0]] + rows[:, 2]
        o_full[tok, rows[:, 1], :] = o
        lse_full[rows[:, 1], tok] = lse
    return o_full, lse_full

"""FP8 (E4M3) forward: the oracle's side.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

The FlashAttention 1-4 post (FlashAttention-3 engineering notes and summary
table) runs the forward's matrix products on FP8 tensor cores and keeps the
backward in BF16; it gives no format details and no scaling policy.  The
readings taken here:

* FP8 is the OCP E4M3 format (the "fn" variant gfx950 computes on): 1 sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
  infinities, code 0x7f / 0xff is NaN, largest finite 448.
* Scaling is per (sequence, head): x = code_value * descale, with
  descale = amax / 448 over that head's values (amax = 0 gives descale 1 and
  all-zero codes).  Codes are x * (1 / descale) rounded to nearest, ties to
  even, every step in fp32 -- the quantisation decision is taken in the
  precision the kernel takes it in.
* V is also offered transposed, [B, H, d, Np] with rows padded by zero codes
  to Np = ceil(N / 64) * 64 (the layout the FP8 kernel reads); packed
  sequences take [H, d, Tp] with each sequence's keys padded to a multiple
  of 64 (see quantize_packed).
* The attention of the FP8 inputs is the exact attention of the dequantised
  values (code value times descale, exact in fp64).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64 values (NaN for 0x7f / 0xff)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


# the 127 finite non-negative codes in increasing order, and their values
_POS_CODES = np.arange(0x7f, dtype=np.uint8)
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """Round finite values with |x| <= 448 to the nearest E4M3 code, ties to
    the even code (the one whose mantissa LSB is 0)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values with |x| <= 448")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], code)  # exact values
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize(x_bits, *, transpose: bool = False):
    """Per-(b, h) E4M3 quantisation of a bf16 ``[B, N, H, d]`` tensor.

    Returns ``(codes, descale)``: codes ``[B, N, H, d]``, or when
    ``transpose`` ``[B, H, d, Np]`` with ``Np = ceil(N / 64) * 64`` and zero
    codes in the padding; descale ``[B, H]`` fp32 (= amax / 448).
    """
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    B, N, H, d = x.shape
    amax = np.max(np.abs(x), axis=(1, 3)).astype(np.float32)        # [B, H]
    safe = np.where(amax > 0, amax, np.float32(E4M3_MAX)).astype(np.float32)
    descale = np.where(amax > 0, (safe / np.float32(E4M3_MAX)).astype(np.float32),
                       np.float32(1.0)).astype(np.float32)         # fp32 division
    inv = (np.float32(1.0) / descale).astype(np.float32)             # fp32 reciprocal
    y = (x * inv[:, None, :, None]).astype(np.float32)              # fp32 product
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)                             # |y| <= 448 up to rounding
    codes = e4m3_encode(y)
    if transpose:
        np_ = (N + 63) // 64 * 64
        t = np.zeros((B, H, d, np_), dtype=np.uint8)
        t[..., :N] = codes.transpose(0, 2, 3, 1)
        codes = t
    return codes, descale


def attention(q8, k8, vt8, dq, dk, dv, *, scale: float, causal: bool, rows=None):
    """Exact attention (fp64) of dequantised E4M3 inputs.

    q8, k8  ``[B, N, H, d]`` codes; vt8 ``[B, H, d, >= N]`` codes (V
            transposed; columns past N are ignored);
    dq, dk, dv  ``[B, H]`` descales; rows None (all) or ``(n, 3)`` (b, h, i).
    Returns ``(o, lse)``: ``o [B, N, H, d]`` and ``lse [B, H, N]`` for all
    rows, else ``o [n, d]`` and ``lse [n]``.
    """
    B, N, H, d = q8.shape
    Q = e4m3_decode(q8) * np.asarray(dq, np.float64)[:, None, :, None]
    K = e4m3_decode(k8) * np.asarray(dk, np.float64)[:, None, :, None]
    Vt = e4m3_decode(vt8[..., :N]) * np.asarray(dv, np.float64)[:, :, None, None]   # [B, H, d, N]
    sc = float(np.float32(scale))
    full = rows is None
    if full:
        o = np.zeros((B, N, H, d))
        lse = np.zeros((B, H, N))
        for b in range(B):
            for h in range(H):
                S = (Q[b, :, h] @ K[b, :, h].T) * sc
                if causal:
                    S = np.where(np.tril(np.ones((N, N), dtype=bool)), S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                l = E.sum(axis=1, keepdims=True)
                o[b, :, h] = (E / l) @ Vt[b, h].T
                lse[b, h] = (m + np.log(l))[:, 0]
        return o, lse
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for r, (b, h, i) in enumerate(rows):
        nvis = i + 1 if causal else N
        s = (K[b, :nvis, h] @ Q[b, i, h]) * sc
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[r] = Vt[b, h][:, :nvis] @ (e / l)
        lse[r] = m + np.log(l)
    return o, lse


# ---------------------------------------------------------------------------
# Packed sequences (cu_seqlens): the same reading per sequence.  Sequence b
# holds tokens cu[b] .. cu[b+1]-1 of a [T, H, d] tensor and is its own
# attention problem; its scales are per (sequence, head).

def vt_stride_packed(T: int, B: int) -> int:
    """Row length (keys) of the packed V^T layout ``[H, d, Tp]``:
    ``Tp = ceil(T / 64) * 64 + 64 * B``, enough for every sequence's keys
    padded to a multiple of 64."""
    return (T + 63) // 64 * 64 + 64 * B


def padded_starts(cu_seqlens) -> np.ndarray:
    """Column where sequence b's keys start in a packed V^T row: the sum of
    ceil(n / 64) * 64 over the sequences before it."""
    n = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    padded = (n + 63) // 64 * 64
    return np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)


def _segments(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = np.diff(cu)
    if cu[0] != 0 or np.any(n < 0) or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return cu, n


def quantize_packed(x_bits, cu_seqlens, *, transpose: bool = False):
    """Per-(sequence, head) E4M3 quantisation of a packed bf16 ``[T, H, d]``.

    The steps of :func:`quantize`, with the amax of (b, h) taken over the
    sequence's own tokens.  Returns ``(codes, descale)``: codes ``[T, H, d]``,
    or when ``transpose`` ``[H, d, Tp]`` (``Tp = vt_stride_packed(T, B)``)
    with sequence b's keys at columns ``padded_starts[b] + i`` and zero codes
    elsewhere; descale ``[B, H]`` fp32.
    """
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    T, H, d = x.shape
    cu, n = _segments(cu_seqlens, T)
    B = len(n)
    seq = np.repeat(np.arange(B), n)                                  # sequence of each token
    amax = np.zeros((B, H), dtype=np.float32)
    absmax_tok = np.max(np.abs(x), axis=2)                            # [T, H]
    np.maximum.at(amax, seq, absmax_tok)                              # segment maxima
    safe = np.where(amax > 0, amax, np.float32(E4M3_MAX)).astype(np.float32)
    descale = np.where(amax > 0, (safe / np.float32(E4M3_MAX)).astype(np.float32),
                       np.float32(1.0)).astype(np.float32)
    inv = (np.float32(1.0) / descale).astype(np.float32)              # [B, H]
    y = (x * inv[seq][:, :, None]).astype(np.float32)
    codes = e4m3_encode(np.clip(y, -E4M3_MAX, E4M3_MAX))
    if transpose:
        Tp = vt_stride_packed(T, B)
        t = np.zeros((H, d, Tp), dtype=np.uint8)
        col = padded_starts(cu)[seq] + (np.arange(T) - cu[seq])      # column of each token
        t[:, :, col] = codes.transpose(1, 2, 0)
        codes = t
    return codes, descale


def attention_packed(q8, k8, vt8, dq, dk, dv, cu_seqlens, *, scale: float, causal: bool, rows=None):
    """Exact attention (fp64) of dequantised packed E4M3 inputs.

    q8, k8  ``[T, H, d]`` codes; vt8 ``[H, d, >= Tp]`` codes in the packed V^T
            layout; dq, dk, dv ``[B, H]`` descales of (sequence, head).
    rows None (all) or ``(n, 3)`` (b, h, i) with i counted within sequence b.
    Returns ``o [T, H, d]``, ``lse [H, T]`` for all rows, else ``o [n, d]``
    and ``lse [n]``.  A sequence sees only its own keys.
    """
    T, H, d = q8.shape
    cu, n = _segments(cu_seqlens, T)
    B = len(n)
    seq = np.repeat(np.arange(B), n)
    dq, dk, dv = (np.asarray(a, np.float64) for a in (dq, dk, dv))
    Q = e4m3_decode(q8) * dq[seq][:, :, None]                          # [T, H, d]
    K = e4m3_decode(k8) * dk[seq][:, :, None]
    col = padded_starts(cu)[seq] + (np.arange(T) - cu[seq])
    V = e4m3_decode(vt8[:, :, col]).transpose(2, 0, 1) * dv[seq][:, :, None]   # [T, H, d]
    sc = float(np.float32(scale))

    def one(b, h, i_rows):
        t0, nb = int(cu[b]), int(n[b])
        S = (Q[t0 + i_rows, h] @ K[t0:t0 + nb, h].T) * sc               # [len(i_rows), nb]
        if causal:
            S = np.where(np.arange(nb)[None, :] <= i_rows[:, None], S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        return (E / l) @ V[t0:t0 + nb, h], (m + np.log(l))[:, 0]

    if rows is None:
        o = np.zeros((T, H, d))
        lse = np.zeros((H, T))
        for b in range(B):
            if n[b] == 0:
                continue
            for h in range(H):
                ob, lb = one(b, h, np.arange(n[b]))
                o[cu[b]:cu[b + 1], h] = ob
                lse[h, cu[b]:cu[b + 1]] = lb
        return o, lse
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for r, (b, h, i) in enumerate(rows):
        if not 0 <= i < n[b]:
            raise ValueError("row index outside its sequence")
        ob, lb = one(b, h, np.array([i]))
        o[r], lse[r] = ob[0], lb[0]
    return o, lse

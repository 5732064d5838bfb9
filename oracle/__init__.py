"""fp64 CPU oracle for exact attention (forward).

TEST INFRASTRUCTURE ONLY: the checker that the fused HIP kernel is compared
against.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path never does, and nothing here is
shared with the HIP path.

The forward, written from the FlashAttention explainer pages:

* :func:`attention` -- the plain definition (compute chain of section 1.1;
  the "standard attention" equations of the FlashAttention 1-4 post): each
  score row is materialised, the row max is subtracted, exp, normalise, then
  P V.  Implemented in C (``oracle.c``), fp64, threaded over rows.
* :func:`oracle.online.online_attention` -- the tiled online-softmax
  recurrence of the FlashAttention-1 derivation, used only to cross-check the
  definition (the two agree to rounding in exact arithmetic).

and :func:`oracle.backward.attention_backward`, the exact gradients of the
same definition (numpy, fp64), for the backward pass.

Layouts: dense tensors are ``[B, N, H, d]`` uint16 (bf16 bit patterns);
packed variable-length tensors are ``[T, H, d]`` with ``cu_seqlens`` (int32,
``B+1`` entries).  LSE is ``[B, H, N]`` (dense) or ``[H, T]`` (packed).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (plain gcc, no fast-math)."""
    global _lib
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-pthread",
             _SRC, "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, LIB_PATH)
        _lib = None
    return LIB_PATH


def load_library(path: str | None = None):
    """Load the oracle library (``path`` lets tests load a rebuilt copy)."""
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
    else:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
    fn = lib.oracle_attention_rows
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    fr = lib.oracle_attention_rows_range
    fr.restype = ctypes.c_int
    fr.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _widen(x) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly; float arrays -> float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def all_rows(B: int, H: int, lengths) -> np.ndarray:
    """Every (b, h, i) triple, in the order the outputs are laid out."""
    out = []
    for b in range(B):
        n = int(lengths[b])
        bb = np.full((H, n), b, dtype=np.int64)
        hh = np.repeat(np.arange(H, dtype=np.int64)[:, None], n, axis=1)
        ii = np.repeat(np.arange(n, dtype=np.int64)[None, :], H, axis=0)
        out.append(np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1))
    if not out:
        return np.zeros((0, 3), dtype=np.int64)
    return np.concatenate(out, axis=0)


def attention(q, k, v, *, scale: float, causal: bool, cu_seqlens=None,
              rows=None, nthreads: int | None = None, lib=None, key_range=None):
    """Exact attention forward in fp64.

    q, k, v    uint16 arrays: ``[B, N, H, d]`` (dense) or ``[T, H, d]``
               (packed, with ``cu_seqlens``).
    scale      the fp32 softmax scale (widened to double as given).
    rows       None for every row, or an ``(n, 3)`` int array of
               ``(b, h, i)`` triples.
    key_range  None for every visible key, or ``(lo, hi)``: only keys
               ``lo <= j < hi`` (indices within the sequence) take part.  A
               row with no key left gets ``O = 0`` and ``LSE = -inf``.
    Returns ``(o, lse)`` as float64: full layouts (``o`` shaped like ``q``,
    ``lse`` ``[B, H, N]`` or ``[H, T]``) when ``rows`` is None, else
    ``o [n, d]`` and ``lse [n]``.
    """
    lib = lib if lib is not None else load_library()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have the same shape")
    if cu_seqlens is None:
        if q.ndim != 4:
            raise ValueError("dense inputs are [B, N, H, d]")
        B, N, H, d = q.shape
        lengths = [N] * B
        cu = None
        nmax = N
    else:
        if q.ndim != 3:
            raise ValueError("packed inputs are [T, H, d]")
        T, H, d = q.shape
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        B = cu.shape[0] - 1
        lengths = np.diff(cu.astype(np.int64))
        if cu[0] != 0 or np.any(lengths < 0) or int(cu[-1]) != T:
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
        nmax = int(lengths.max()) if B > 0 else 1
        N = max(nmax, 1)
    full = rows is None
    if full:
        rows = all_rows(B, H, lengths)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    if n > 0:
        common = (_ptr(q), _ptr(k), _ptr(v), B, H, max(nmax, 1), d,
                  ctypes.c_float(scale), int(bool(causal)),
                  _ptr(cu) if cu is not None else None, n, _ptr(rows))
        if key_range is None:
            rc = lib.oracle_attention_rows(*common, _ptr(o), _ptr(lse),
                                           int(nthreads or default_threads()))
        else:
            lo, hi = (int(x) for x in key_range)
            rc = lib.oracle_attention_rows_range(*common, lo, hi, _ptr(o), _ptr(lse),
                                                 int(nthreads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle attention rows failed with code {rc}")
    if not full:
        return o, lse
    # scatter into the tensor layouts
    o_full = np.zeros(q.shape, dtype=np.float64)
    if cu is None:
        lse_full = np.zeros((B, H, N), dtype=np.float64)
        o_full[rows[:, 0], rows[:, 2], rows[:, 1], :] = o
        lse_full[rows[:, 0], rows[:, 1], rows[:, 2]] = lse
    else:
        lse_full = np.zeros((H, q.shape[0]), dtype=np.float64)
        tok = cu[rows[:, 0]].astype(np.int64) + rows[:, 2]
        o_full[tok, rows[:, 1], :] = o
        lse_full[rows[:, 1], tok] = lse
    return o_full, lse_full


def merge(o_parts, lse_parts):
    """Combine attention results over disjoint key ranges into the result
    over their union, in fp64.

    ``o_parts``: ``[S, ...rows..., d]`` normalised partial outputs;
    ``lse_parts``: ``[S, ...rows...]`` their log-sum-exps (``-inf`` for a
    range with no key).  Each part is a softmax over its own keys, so with
    ``LSE = ln sum_s exp(LSE_s)`` the union's weights are the parts' weights
    times ``exp(LSE_s - LSE)``: ``O = sum_s exp(LSE_s - LSE) O_s``.  This is
    the rescaling the FlashAttention-2 section of the FlashAttention 1-4 post
    applies when the key/value sequence is split.  Returns ``(o, lse)``.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError("o_parts must be lse_parts' shape plus a trailing d")
    m = np.max(lse_parts, axis=0)
    safe = np.where(np.isfinite(m), m, 0.0)          # no key anywhere: keep -inf
    w = np.exp(lse_parts - safe[None])                 # exp(-inf) = 0 for empty parts
    tot = np.sum(w, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = safe + np.log(tot)
        o = np.sum(w[..., None] * o_parts, axis=0) / tot[..., None]
    o = np.where((tot > 0)[..., None], o, 0.0)
    lse = np.where(tot > 0, lse, -np.inf)
    return o, lse

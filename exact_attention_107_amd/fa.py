"""Python binding of libfa.so: argument marshalling only.

Every step of the attention forward runs in the library's HIP kernel; this
module checks tensors, allocates the outputs with torch, passes raw device
pointers and torch's current HIP stream, and turns error codes into
exceptions.  If the library is not built, every call raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

# enum fa_exp_mode / fa_rescale_mode of include/fa.h
EXP_HW, EXP_POLY, EXP_MIXED = 0, 1, 2
RESCALE_ALWAYS, RESCALE_STRICT, RESCALE_THRESHOLD = 0, 1, 2
EXPORTS = ("fa_fwd", "fa_fwd_variant", "fa_strerror", "fa_tile_rows", "fa_tile_keys",
           "fa_fwd_splitkv", "fa_merge", "fa_split_range", "fa_num_splits", "fa_bwd",
           "fa_bwd_workspace_floats", "fa_fwd_fp8", "fa_quantize_fp8", "fa_fp8_vt_stride",
           "fa_fwd_masked", "fa_fwd_rescale_counts", "fa_fwd_splitkv_static", "fa_fwd_pingpong",
           "fa_fp8_vt_stride_packed", "fa_quantize_fp8_packed", "fa_fwd_fp8_packed", "fa_fwd_splitkv_packed",
           "fa_fwd_masked_packed", "fa_fwd_tile_rows")
FA_ERR_SCRATCH = 10
STATIC_SCRATCH_BYTES = 64 << 20   # FA_STATIC_SCRATCH_BYTES of include/fa.h

_lib = None

# The library reads cu_seqlens on the device and does not validate its
# contents (its kernels clamp every sequence to [0, T], so malformed offsets
# give wrong results, not out-of-range accesses).  With FA_CHECK_CU_SEQLENS=1
# in the environment every packed call first checks the offsets on the host
# (a copy and a synchronisation per call: for debugging, not for hot loops).
CHECK_CU_SEQLENS = os.environ.get("FA_CHECK_CU_SEQLENS", "") not in ("", "0")


def check_cu_seqlens(cu_seqlens: torch.Tensor, T: int) -> None:
    """Raise ValueError unless ``cu_seqlens`` (int32 ``[B+1]``, any device)
    starts at 0, never decreases and ends at ``T``."""
    c = cu_seqlens.detach().to("cpu", torch.int64)
    if c.dim() != 1 or c.numel() < 2:
        raise ValueError("cu_seqlens must be [B+1]")
    if int(c[0]) != 0 or int(c[-1]) != int(T) or bool((c[1:] < c[:-1]).any()):
        raise ValueError(f"cu_seqlens must start at 0, be non-decreasing and end at T = {T}")


class FaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"fa error {code}: {msg}")
        self.code = code


def load(path: str | None = None):
    """Load libfa.so and declare its C signatures (raises if not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    common = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32, vp, vp]
    lib.fa_fwd.argtypes = common
    lib.fa_fwd.restype = i32
    lib.fa_fwd_variant.argtypes = common + [i32, i32]
    lib.fa_fwd_variant.restype = i32
    lib.fa_strerror.argtypes = [i32]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_tile_rows.argtypes = [i32]
    lib.fa_tile_rows.restype = i32
    lib.fa_tile_keys.argtypes = [i32]
    lib.fa_tile_keys.restype = i32
    lib.fa_fwd_tile_rows.argtypes = [i32] * 7
    lib.fa_fwd_tile_rows.restype = i32
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32,
                                   i32, vp, vp, vp]
    lib.fa_fwd_splitkv.restype = i32
    lib.fa_fwd_splitkv_static.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32,
                                          i32, vp]
    lib.fa_fwd_splitkv_static.restype = i32
    lib.fa_merge.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.fa_merge.restype = i32
    lib.fa_split_range.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.fa_split_range.restype = i32
    lib.fa_num_splits.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_num_splits.restype = i32
    lib.fa_bwd.argtypes = [vp] * 9 + [i32, i32, i32, i32, ctypes.c_float, i32, vp, vp, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_workspace_floats.argtypes = [i32, i32, i32]
    lib.fa_bwd_workspace_floats.restype = ctypes.c_longlong
    lib.fa_fwd_fp8.argtypes = [vp] * 8 + [i32, i32, i32, i32, ctypes.c_float, i32, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.fa_quantize_fp8.restype = i32
    lib.fa_fp8_vt_stride.argtypes = [i32]
    lib.fa_fp8_vt_stride.restype = i32
    lib.fa_fp8_vt_stride_packed.argtypes = [i32, i32]
    lib.fa_fp8_vt_stride_packed.restype = i32
    lib.fa_quantize_fp8_packed.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.fa_quantize_fp8_packed.restype = i32
    lib.fa_fwd_fp8_packed.argtypes = [vp] * 9 + [i32, i32, i32, i32, ctypes.c_float, i32, vp]
    lib.fa_fwd_fp8_packed.restype = i32
    lib.fa_fwd_splitkv_packed.argtypes = [vp] * 6 + [i32, i32, i32, i32, ctypes.c_float, i32, i32, vp, vp, vp]
    lib.fa_fwd_splitkv_packed.restype = i32
    lib.fa_fwd_masked_packed.argtypes = [vp] * 6 + [i32, i32, i32, i32, ctypes.c_float, i32, i32, vp, vp]
    lib.fa_fwd_masked_packed.restype = i32
    lib.fa_fwd_masked.argtypes = [vp] * 5 + [i32, i32, i32, i32, ctypes.c_float, i32, i32, vp, vp]
    lib.fa_fwd_masked.restype = i32
    lib.fa_fwd_pingpong.argtypes = common
    lib.fa_fwd_pingpong.restype = i32
    lib.fa_fwd_rescale_counts.argtypes = common + [i32, vp]
    lib.fa_fwd_rescale_counts.restype = i32
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().fa_strerror(int(code)).decode()


def _check(t: torch.Tensor, name: str, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
        scale: float | None = None, cu_seqlens: torch.Tensor | None = None,
        exp_mode: int | None = None, rescale_mode: int | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
        stream: torch.cuda.Stream | None = None, counts: torch.Tensor | None = None,
        pingpong: bool = False):
    """Exact attention forward on the GPU.

    q, k, v     bf16, ``[B, N, H, d]`` (dense) or ``[T, H, d]`` with
                ``cu_seqlens`` (int32, ``[B+1]``, on the same device).
    scale       defaults to ``1/sqrt(d)``, rounded to fp32.
    exp_mode, rescale_mode   None for the library default (``fa_fwd``), else
                one of the EXP_* / RESCALE_* constants (``fa_fwd_variant``).
    out, lse    optional preallocated outputs (``o`` like q; ``lse`` fp32
                ``[B, H, N]`` or ``[H, T]``).
    counts      optional int64 ``[4]`` device tensor: run the counting
                instance (``fa_fwd_rescale_counts``, d = 128, hardware exp2,
                ``rescale_mode`` strict or threshold), which adds its rescale
                statistics to it.
    pingpong    run ``fa_fwd_pingpong`` (d = 128; the two halves of each
                workgroup half a key tile apart; bitwise fa_fwd's result).
    Returns ``(o, lse)``.  The kernel is queued on ``stream`` (default: the
    current stream); nothing is synchronised.
    """
    lib = load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, name, torch.bfloat16, dev)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, N, H, d]")
        B, N, H, d = q.shape
        lse_shape = (B, H, N)
        cu_ptr = None
    else:
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if q.dim() != 3 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("packed q must be [T, H, d] with cu_seqlens [B+1]")
        N, H, d = q.shape
        B = cu_seqlens.numel() - 1
        lse_shape = (H, N)
        cu_ptr = cu_seqlens.data_ptr()
        if CHECK_CU_SEQLENS:
            check_cu_seqlens(cu_seqlens, N)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
    else:
        _check(lse, "lse", torch.float32, dev)
        if tuple(lse.shape) != lse_shape:
            raise ValueError(f"lse must be {lse_shape}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            int(B), int(H), int(N), int(d), ctypes.c_float(scale), int(bool(causal)),
            cu_ptr, ctypes.c_void_p(s.cuda_stream))
    if counts is not None:
        _check(counts, "counts", torch.int64, dev)
        if counts.numel() != 4:
            raise ValueError("counts must hold 4 int64 values")
        if exp_mode not in (None, EXP_HW):
            raise ValueError("the counting instance evaluates exp2 in hardware (exp_mode EXP_HW)")
    if pingpong and (counts is not None or exp_mode is not None or rescale_mode is not None):
        raise ValueError("pingpong runs the default variant only (no counts, exp_mode or rescale_mode)")
    with torch.cuda.device(dev):
        if pingpong:
            rc = lib.fa_fwd_pingpong(*args)
        elif counts is not None:
            rc = lib.fa_fwd_rescale_counts(*args, int(RESCALE_STRICT if rescale_mode is None else rescale_mode),
                                           counts.data_ptr())
        elif exp_mode is None and rescale_mode is None:
            rc = lib.fa_fwd(*args)
        else:
            rc = lib.fa_fwd_variant(*args, int(EXP_HW if exp_mode is None else exp_mode),
                                    int(RESCALE_STRICT if rescale_mode is None else rescale_mode))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def rescale_counts(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                   scale: float | None = None, cu_seqlens: torch.Tensor | None = None,
                   rescale_mode: int = RESCALE_STRICT) -> dict:
    """How often the conditional rescale fires (``fa_fwd_rescale_counts``).

    Returns the four counters of the C ABI by name plus the two rates:
    ``step_rescale_rate`` (wave-steps whose O accumulator was rescaled) and
    ``row_move_rate`` (rows whose reference max moved), over every key tile
    after each wave's first.
    """
    c = torch.zeros(4, dtype=torch.int64, device=q.device)
    fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu_seqlens, rescale_mode=rescale_mode, counts=c)
    steps, rescaled, moved, rows = (int(x) for x in c.cpu().tolist())
    return {"steps": steps, "rescaled_steps": rescaled, "rows_moved": moved, "rows": rows,
            "step_rescale_rate": rescaled / steps if steps else 0.0,
            "row_move_rate": moved / rows if rows else 0.0}


def tile_rows(d: int) -> int:
    return int(load().fa_tile_rows(int(d)))


def tile_keys(d: int) -> int:
    return int(load().fa_tile_keys(int(d)))


def fwd_tile_rows(B: int, H: int, N: int, d: int, causal: bool = False, packed: bool = False,
                  num_cus: int = 0) -> int:
    """Rows per workgroup tile fa_fwd picks for a shape (packed: B sequences, N = T)."""
    return int(load().fa_fwd_tile_rows(int(B), int(H), int(N), int(d), int(bool(causal)),
                                       int(bool(packed)), int(num_cus)))


def split_range(N: int, d: int, causal: bool, num_splits: int, s: int, row: int) -> tuple[int, int]:
    """Keys ``[lo, hi)`` of range ``s`` of :func:`fwd_splitkv` for query ``row``."""
    lo, hi = ctypes.c_int(), ctypes.c_int()
    rc = load().fa_split_range(int(N), int(d), int(bool(causal)), int(num_splits), int(s), int(row),
                               ctypes.byref(lo), ctypes.byref(hi))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return lo.value, hi.value


def num_splits(B: int, H: int, N: int, d: int, causal: bool = False, num_cus: int = 0) -> int:
    """The library's suggested split count for :func:`fwd_splitkv`."""
    return int(load().fa_num_splits(int(B), int(H), int(N), int(d), int(bool(causal)), int(num_cus)))


def _dense_shape(q):
    if q.dim() != 4:
        raise ValueError("dense tensors are [B, N, H, d]")
    return tuple(int(x) for x in q.shape)


def fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                scale: float | None = None, splits: int | None = None,
                out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                o_part: torch.Tensor | None = None, lse_part: torch.Tensor | None = None,
                stream: torch.cuda.Stream | None = None):
    """Split-KV forward (``fa_fwd_splitkv``), dense ``[B, N, H, d]`` (packed: ``fwd_splitkv_packed``).

    ``splits`` defaults to the library's suggestion for this device.  The fp32
    workspaces ``o_part [S, B, N, H, d]`` and ``lse_part [S, B, H, N]`` are
    allocated with torch unless given.  Returns ``(o, lse)``.
    """
    lib = load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, name, torch.bfloat16, dev)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    B, N, H, d = _dense_shape(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if splits is None:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        splits = num_splits(B, H, N, d, causal, cus)
    S = int(splits)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    o_part = torch.empty((S, B, N, H, d), dtype=torch.float32, device=dev) if o_part is None else o_part
    lse_part = torch.empty((S, B, H, N), dtype=torch.float32, device=dev) if lse_part is None else lse_part
    for t, name, dt, shape in ((out, "out", torch.bfloat16, (B, N, H, d)),
                               (lse, "lse", torch.float32, (B, H, N)),
                               (o_part, "o_part", torch.float32, (S, B, N, H, d)),
                               (lse_part, "lse_part", torch.float32, (S, B, H, N))):
        _check(t, name, dt, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                B, H, N, d, ctypes.c_float(scale), int(bool(causal)), S,
                                o_part.data_ptr(), lse_part.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def _packed_qkv(q, k, v, cu_seqlens):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, name, torch.bfloat16, dev)
    if k.shape != q.shape or v.shape != q.shape or q.dim() != 3:
        raise ValueError("packed q, k and v must be [T, H, d] of one shape")
    T, H, d = (int(x) for x in q.shape)
    B = _packed_cu(cu_seqlens, dev, T)
    return dev, B, T, H, d


def fwd_splitkv_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                       splits: int, causal: bool = False, scale: float | None = None,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       o_part: torch.Tensor | None = None, lse_part: torch.Tensor | None = None,
                       stream: torch.cuda.Stream | None = None):
    """Split-KV forward over packed sequences (``fa_fwd_splitkv_packed``):
    ``q, k, v [T, H, d]``, ``cu_seqlens`` int32 ``[B+1]``; the fp32
    workspaces ``o_part [S, T, H, d]`` and ``lse_part [S, H, T]`` are
    allocated with torch unless given.  Returns ``(o [T, H, d], lse [H, T])``."""
    lib = load()
    dev, B, T, H, d = _packed_qkv(q, k, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    S = int(splits)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, T), dtype=torch.float32, device=dev) if lse is None else lse
    o_part = torch.empty((S, T, H, d), dtype=torch.float32, device=dev) if o_part is None else o_part
    lse_part = torch.empty((S, H, T), dtype=torch.float32, device=dev) if lse_part is None else lse_part
    for t, name, dt, shape in ((out, "out", torch.bfloat16, (T, H, d)), (lse, "lse", torch.float32, (H, T)),
                               (o_part, "o_part", torch.float32, (S, T, H, d)),
                               (lse_part, "lse_part", torch.float32, (S, H, T))):
        _check(t, name, dt, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_fwd_splitkv_packed(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                       cu_seqlens.data_ptr(), B, H, T, d, ctypes.c_float(scale), int(bool(causal)),
                                       S, o_part.data_ptr(), lse_part.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def fwd_masked_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                      window_left: int = -1, window_right: int = -1, alibi_slopes: torch.Tensor | None = None,
                      scale: float | None = None, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Window mask and ALiBi over packed sequences (``fa_fwd_masked_packed``):
    positions count from each sequence's first token.  Returns
    ``(o [T, H, d], lse [H, T])``."""
    lib = load()
    dev, B, T, H, d = _packed_qkv(q, k, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if alibi_slopes is not None:
        _check(alibi_slopes, "alibi_slopes", torch.float32, dev)
        if tuple(alibi_slopes.shape) != (H,):
            raise ValueError(f"alibi_slopes must be ({H},)")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, T), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, dev)
    _check(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (T, H, d) or tuple(lse.shape) != (H, T):
        raise ValueError(f"out must be {(T, H, d)} and lse {(H, T)}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_fwd_masked_packed(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                      cu_seqlens.data_ptr(), B, H, T, d, ctypes.c_float(scale), int(window_left),
                                      int(window_right),
                                      None if alibi_slopes is None else alibi_slopes.data_ptr(),
                                      ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def fwd_splitkv_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                       scale: float | None = None, splits: int | None = None,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       stream: torch.cuda.Stream | None = None):
    """``fa_fwd_splitkv_static``: the split-KV forward with its partials in
    the library's static per-GPU scratch (the C call allocates nothing; pass
    ``out`` and ``lse`` to allocate nothing here either).  Calls that overlap
    on one GPU race.  Returns ``(o, lse)``."""
    lib = load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, name, torch.bfloat16, dev)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    B, N, H, d = _dense_shape(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if splits is None:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        splits = num_splits(B, H, N, d, causal, cus)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, dev)
    _check(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (B, N, H, d) or tuple(lse.shape) != (B, H, N):
        raise ValueError(f"out must be {(B, N, H, d)} and lse {(B, H, N)}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       lse.data_ptr(), B, H, N, d, ctypes.c_float(scale),
                                       int(bool(causal)), int(splits), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def merge(o_part: torch.Tensor, lse_part: torch.Tensor, *, out: torch.Tensor | None = None,
          lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """``fa_merge``: combine fp32 partials ``o_part [S, B, N, H, d]`` and
    ``lse_part [S, B, H, N]`` into bf16 ``o`` and fp32 ``lse``."""
    lib = load()
    dev = o_part.device
    _check(o_part, "o_part", torch.float32, dev)
    _check(lse_part, "lse_part", torch.float32, dev)
    if o_part.dim() != 5:
        raise ValueError("o_part must be [S, B, N, H, d]")
    S, B, N, H, d = (int(x) for x in o_part.shape)
    if tuple(lse_part.shape) != (S, B, H, N):
        raise ValueError("lse_part must be [S, B, H, N]")
    out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, dev)
    _check(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (B, N, H, d) or tuple(lse.shape) != (B, H, N):
        raise ValueError("out must be [B, N, H, d] and lse [B, H, N]")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_merge(o_part.data_ptr(), lse_part.data_ptr(), S, B, H, N, d, out.data_ptr(),
                          lse.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def bwd_workspace_floats(B: int, H: int, N: int) -> int:
    return int(load().fa_bwd_workspace_floats(int(B), int(H), int(N)))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, causal: bool = False, scale: float | None = None,
        cu_seqlens: torch.Tensor | None = None,
        dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
        dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
        stream: torch.cuda.Stream | None = None):
    """Gradients of the attention forward (``fa_bwd``).

    Layouts as ``fwd``: dense ``[B, N, H, d]`` with ``lse [B, H, N]``, or
    packed ``[T, H, d]`` with ``cu_seqlens`` (int32 ``[B+1]``) and
    ``lse [H, T]``.  ``o`` and ``lse`` are the forward's outputs, ``dout``
    the upstream gradient.  Returns ``(dq, dk, dv)`` (bf16, shaped like q);
    the fp32 workspace is allocated with torch unless given.
    """
    lib = load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    if cu_seqlens is None:
        B, N, H, d = _dense_shape(q)
        lse_shape, ws_batch, cu_ptr = (B, H, N), B, None
    else:
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if q.dim() != 3 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("packed q must be [T, H, d] with cu_seqlens [B+1]")
        N, H, d = q.shape
        B = cu_seqlens.numel() - 1
        lse_shape, ws_batch, cu_ptr = (H, N), 1, cu_seqlens.data_ptr()
        if CHECK_CU_SEQLENS:
            check_cu_seqlens(cu_seqlens, N)
    shape = tuple(q.shape)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, name, torch.bfloat16, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    _check(lse, "lse", torch.float32, dev)
    if tuple(lse.shape) != lse_shape:
        raise ValueError(f"lse must be {lse_shape}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, name, torch.bfloat16, dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    wf = bwd_workspace_floats(ws_batch, H, N)
    if workspace is None:
        workspace = torch.empty(wf, dtype=torch.float32, device=dev)
    _check(workspace, "workspace", torch.float32, dev)
    if workspace.numel() < wf:
        raise ValueError(f"workspace needs {wf} floats")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), int(B), int(H),
                        int(N), int(d), ctypes.c_float(scale), int(bool(causal)), cu_ptr,
                        workspace.data_ptr(), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return dq, dk, dv


def fp8_vt_stride(N: int) -> int:
    return int(load().fa_fp8_vt_stride(int(N)))


def quantize_fp8(x: torch.Tensor, *, transpose: bool = False, out: torch.Tensor | None = None,
                 descale: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Per-(b, h) E4M3 quantisation of bf16 ``x [B, N, H, d]`` (``fa_quantize_fp8``).

    Returns ``(codes, descale)``: uint8 codes ``[B, N, H, d]`` (or ``[B, H, d,
    Np]`` when ``transpose``) and fp32 ``descale [B, H]``.
    """
    lib = load()
    dev = x.device
    _check(x, "x", torch.bfloat16, dev)
    B, N, H, d = _dense_shape(x)
    shape = (B, H, d, fp8_vt_stride(N)) if transpose else (B, N, H, d)
    out = torch.empty(shape, dtype=torch.uint8, device=dev) if out is None else out
    descale = torch.empty((B, H), dtype=torch.float32, device=dev) if descale is None else descale
    _check(out, "out", torch.uint8, dev)
    _check(descale, "descale", torch.float32, dev)
    if tuple(out.shape) != shape or tuple(descale.shape) != (B, H):
        raise ValueError(f"out must be {shape} and descale {(B, H)}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_quantize_fp8(x.data_ptr(), out.data_ptr(), descale.data_ptr(), B, H, N, d,
                                 int(bool(transpose)), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, descale


def fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, vt8: torch.Tensor, descale_q: torch.Tensor,
            descale_k: torch.Tensor, descale_v: torch.Tensor, *, causal: bool = False,
            scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """FP8 forward (``fa_fwd_fp8``): E4M3 ``q8, k8 [B, N, H, d]``, ``vt8
    [B, H, d, Np]``, fp32 descales ``[B, H]``.  Returns bf16 ``o`` and fp32
    ``lse``."""
    lib = load()
    dev = q8.device
    for t, name in ((q8, "q8"), (k8, "k8"), (vt8, "vt8")):
        _check(t, name, torch.uint8, dev)
    B, N, H, d = _dense_shape(q8)
    if tuple(k8.shape) != (B, N, H, d) or tuple(vt8.shape) != (B, H, d, fp8_vt_stride(N)):
        raise ValueError("k8 must be like q8 and vt8 [B, H, d, fp8_vt_stride(N)]")
    for t, name in ((descale_q, "descale_q"), (descale_k, "descale_k"), (descale_v, "descale_v")):
        _check(t, name, torch.float32, dev)
        if tuple(t.shape) != (B, H):
            raise ValueError(f"{name} must be {(B, H)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, dev)
    _check(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (B, N, H, d) or tuple(lse.shape) != (B, H, N):
        raise ValueError(f"out must be {(B, N, H, d)} and lse {(B, H, N)}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), descale_q.data_ptr(),
                            descale_k.data_ptr(), descale_v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, N, d, ctypes.c_float(scale), int(bool(causal)),
                            ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def fp8_vt_stride_packed(T: int, B: int) -> int:
    return int(load().fa_fp8_vt_stride_packed(int(T), int(B)))


def _packed_cu(cu_seqlens, dev, T: int):
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [B+1]")
    if CHECK_CU_SEQLENS:
        check_cu_seqlens(cu_seqlens, T)
    return cu_seqlens.numel() - 1


def quantize_fp8_packed(x: torch.Tensor, cu_seqlens: torch.Tensor, *, transpose: bool = False,
                        out: torch.Tensor | None = None, descale: torch.Tensor | None = None,
                        stream: torch.cuda.Stream | None = None):
    """Per-(sequence, head) E4M3 quantisation of packed bf16 ``x [T, H, d]``
    (``fa_quantize_fp8_packed``).  Returns uint8 codes ``[T, H, d]`` (or the
    packed V^T layout ``[H, d, fp8_vt_stride_packed(T, B)]`` when
    ``transpose``) and fp32 ``descale [B, H]``."""
    lib = load()
    dev = x.device
    _check(x, "x", torch.bfloat16, dev)
    if x.dim() != 3:
        raise ValueError("packed x must be [T, H, d]")
    T, H, d = (int(v) for v in x.shape)
    B = _packed_cu(cu_seqlens, dev, T)
    shape = (H, d, fp8_vt_stride_packed(T, B)) if transpose else (T, H, d)
    # the columns past the last sequence's padding are not written: zero them
    out = (torch.zeros if transpose else torch.empty)(shape, dtype=torch.uint8, device=dev) if out is None else out
    descale = torch.empty((B, H), dtype=torch.float32, device=dev) if descale is None else descale
    _check(out, "out", torch.uint8, dev)
    _check(descale, "descale", torch.float32, dev)
    if tuple(out.shape) != shape or tuple(descale.shape) != (B, H):
        raise ValueError(f"out must be {shape} and descale {(B, H)}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_quantize_fp8_packed(x.data_ptr(), out.data_ptr(), descale.data_ptr(), cu_seqlens.data_ptr(),
                                        B, H, T, d, int(bool(transpose)), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, descale


def fwd_fp8_packed(q8: torch.Tensor, k8: torch.Tensor, vt8: torch.Tensor, descale_q: torch.Tensor,
                   descale_k: torch.Tensor, descale_v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                   causal: bool = False, scale: float | None = None, out: torch.Tensor | None = None,
                   lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """FP8 forward over packed sequences (``fa_fwd_fp8_packed``): E4M3 ``q8,
    k8 [T, H, d]``, ``vt8 [H, d, fp8_vt_stride_packed(T, B)]``, fp32 descales
    ``[B, H]``.  Returns bf16 ``o [T, H, d]`` and fp32 ``lse [H, T]``."""
    lib = load()
    dev = q8.device
    for t, name in ((q8, "q8"), (k8, "k8"), (vt8, "vt8")):
        _check(t, name, torch.uint8, dev)
    if q8.dim() != 3:
        raise ValueError("packed q8 must be [T, H, d]")
    T, H, d = (int(v) for v in q8.shape)
    B = _packed_cu(cu_seqlens, dev, T)
    if tuple(k8.shape) != (T, H, d) or tuple(vt8.shape) != (H, d, fp8_vt_stride_packed(T, B)):
        raise ValueError("k8 must be like q8 and vt8 [H, d, fp8_vt_stride_packed(T, B)]")
    for t, name in ((descale_q, "descale_q"), (descale_k, "descale_k"), (descale_v, "descale_v")):
        _check(t, name, torch.float32, dev)
        if tuple(t.shape) != (B, H):
            raise ValueError(f"{name} must be {(B, H)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty((H, T), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, dev)
    _check(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (T, H, d) or tuple(lse.shape) != (H, T):
        raise ValueError(f"out must be {(T, H, d)} and lse {(H, T)}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_fwd_fp8_packed(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), descale_q.data_ptr(),
                                   descale_k.data_ptr(), descale_v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   cu_seqlens.data_ptr(), B, H, T, d, ctypes.c_float(scale), int(bool(causal)),
                                   ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse


def fwd_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, window_left: int = -1,
               window_right: int = -1, alibi_slopes: torch.Tensor | None = None,
               scale: float | None = None, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """``fa_fwd_masked``: window mask (``i - left <= j <= i + right``, negative =
    unbounded) and optional per-head ALiBi slopes (fp32 ``[H]``), dense
    ``[B, N, H, d]``.  Returns ``(o, lse)``."""
    lib = load()
    dev = q.device
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, name, torch.bfloat16, dev)
    B, N, H, d = _dense_shape(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if alibi_slopes is not None:
        _check(alibi_slopes, "alibi_slopes", torch.float32, dev)
        if tuple(alibi_slopes.shape) != (H,):
            raise ValueError(f"alibi_slopes must be [{H}]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(out, "out", torch.bfloat16, dev)
    _check(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (B, N, H, d) or tuple(lse.shape) != (B, H, N):
        raise ValueError(f"out must be {(B, N, H, d)} and lse {(B, H, N)}")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.fa_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, N, d, ctypes.c_float(scale), int(window_left), int(window_right),
                               alibi_slopes.data_ptr() if alibi_slopes is not None else None,
                               ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise FaError(rc, strerror(rc))
    return out, lse

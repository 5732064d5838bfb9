"""MI355X-native fused exact-attention forward (HIP kernel + C ABI)."""
from .fa import (EXP_HW, EXP_MIXED, EXP_POLY, RESCALE_ALWAYS, RESCALE_STRICT,
                 RESCALE_THRESHOLD, FaError, fwd, load, strerror, tile_keys, tile_rows)

__all__ = ["fwd", "load", "strerror", "tile_rows", "tile_keys", "FaError",
           "EXP_HW", "EXP_POLY", "EXP_MIXED",
           "RESCALE_ALWAYS", "RESCALE_STRICT", "RESCALE_THRESHOLD"]

"""Writes fp8_quant_cases.json: hand-derived E4M3 codes that fix the FP8
quantisation reading.

The FlashAttention-3 notes of "FlashAttention 1-4 explained" run the forward
on FP8 matrix units but give no scaling policy.  The reading taken here
(OCP E4M3, per-(sequence, head) descale = amax / 448) leaves one more choice
that changes codes: the order of the fp32 steps.  The reading fixes it as

    descale = fp32(amax / 448)
    inv     = fp32(1 / descale)
    y       = fp32(x * inv)
    code    = E4M3 round-to-nearest-even(y)

A plausible alternative multiplies by fp32(448 / amax) instead.  The two
differ in the last bit of y for some (amax, x), and sometimes that last bit
decides the E4M3 rounding.  This script finds such pairs among bf16 values
and records, for each, the code of the reading and the code of the
alternative, both derived here from first principles: fp32 rounding with
Python's struct (IEEE binary32, nearest-even), E4M3 rounding with exact
rationals over the format's value grid.  Nothing here runs the oracle or the
GPU path.  Run: ``python tests/golden/make_fp8_quant_cases.py``.
"""
import json
import os
import random
import struct
from fractions import Fraction


def f32(x: float) -> float:
    """Round a Python float (binary64) to the nearest binary32 value."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


# E4M3 (OCP "fn"): bias 7, 3 mantissa bits, subnormals, 0x7f is NaN
GRID = []
for code in range(0x7F):
    e, m = code >> 3, code & 7
    val = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    GRID.append((val, code))


def e4m3_rne(y: float) -> int:
    a = Fraction(abs(y))
    assert a <= 448
    best = None
    for val, code in GRID:
        dist = abs(val - a)
        if best is None or dist < best[0] or (dist == best[0] and code % 2 == 0):
            best = (dist, code)
    code = best[1]
    return code | 0x80 if y < 0 else code


def reading(amax: float, x: float):
    descale = f32(amax / 448.0)
    inv = f32(1.0 / descale)
    y = f32(x * inv)
    return descale, inv, y, e4m3_rne(max(-448.0, min(448.0, y)))


def alternative(amax: float, x: float):
    r = f32(448.0 / amax)
    y = f32(x * r)
    return y, e4m3_rne(max(-448.0, min(448.0, y)))


def main():
    rng = random.Random(20241203)
    cases = []
    tried = 0
    while len(cases) < 12 and tried < 2_000_000:
        tried += 1
        amax_bits = rng.randrange(0x3C00, 0x4400)      # bf16 in [2^-7, 2^9)
        amax = bf16(amax_bits)
        x_bits = rng.randrange(0x0000, 0x8000)
        x = bf16(x_bits)
        if not (0 < x <= amax):
            continue
        descale, inv, y, code = reading(amax, x)
        y_alt, code_alt = alternative(amax, x)
        if code == code_alt:
            continue
        cases.append({
            "amax_bf16": f"0x{amax_bits:04x}", "x_bf16": f"0x{x_bits:04x}",
            "amax": amax, "x": x,
            "descale_fp32": descale, "inv_fp32": inv, "y_fp32": y,
            "code": code, "y_alternative_fp32": y_alt, "code_alternative": code_alt,
        })
    out = {
        "cite": "FP8 forward of the FlashAttention-3 notes in 'FlashAttention 1-4 explained' "
                "(format and scaling not given there; this is the library's reading: "
                "E4M3 RNE of x * fp32(1 / fp32(amax / 448)), every step in fp32).",
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_quant_cases.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"{len(cases)} cases after {tried} draws -> {path}")


if __name__ == "__main__":
    main()

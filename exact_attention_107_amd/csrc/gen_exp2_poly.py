"""Derive the minimax polynomial p(f) ~ 2^f on [0, 1) used by the FMA exp2.

p(f) = 1 + c1 f + c2 f^2 + c3 f^3, with p(0) = 1 held exactly so that the
kernel's exponent-field add gives exactly +0 for x <= -127 and can never wrap
(p(f) >= 1 on [0, 1)).  c1..c3 minimise the relative error
max |p(f) / 2^f - 1| by Remez exchange in float64; they are then rounded to
float32 and the float32 Horner evaluation the kernel performs is measured.
Run: ``python exact_attention_107_amd/csrc/gen_exp2_poly.py [degree]``.
"""
import sys

import numpy as np


def remez_fixed_c0(degree: int, iters: int = 40):
    n = degree                      # unknowns c1..cn and the levelled error E
    x = 0.5 - 0.5 * np.cos(np.pi * (np.arange(n + 1) + 0.5) / (n + 1))
    grid = np.linspace(0.0, 1.0, 400001)
    c = None
    for _ in range(iters):
        # 1 + sum_k c_k x^k - 2^x = (-1)^i E 2^x at the n+1 reference points
        A = np.zeros((n + 1, n + 1))
        rhs = np.exp2(x) - 1.0
        for i in range(n + 1):
            A[i, :n] = x[i] ** np.arange(1, n + 1)
            A[i, n] = -((-1) ** i) * np.exp2(x[i])
        sol = np.linalg.solve(A, rhs)
        c = np.concatenate([[1.0], sol[:n]])
        err = np.polyval(c[::-1], grid) / np.exp2(grid) - 1.0
        # exchange: the extremum of each sign run, excluding the pinned f = 0
        sign = np.sign(err)
        runs, start = [], 1
        for i in range(2, len(grid) + 1):
            if i == len(grid) or sign[i] != sign[start]:
                seg = slice(start, i)
                runs.append(start + int(np.argmax(np.abs(err[seg]))))
                start = i
        if len(runs) < n + 1:
            break
        best = max(range(len(runs) - n), key=lambda s: min(abs(err[j]) for j in runs[s:s + n + 1]))
        x = grid[runs[best:best + n + 1]]
    return c, float(np.max(np.abs(err)))


def f32_horner_error(c32):
    f = np.linspace(0.0, 1.0, 1 << 20, endpoint=False, dtype=np.float32)
    p = np.float32(c32[-1])
    for coef in c32[-2::-1]:
        p = (p * f + np.float32(coef)).astype(np.float32)
    rel = p.astype(np.float64) / np.exp2(f.astype(np.float64)) - 1.0
    return float(np.max(np.abs(rel))), float(p.min())


if __name__ == "__main__":
    deg = int(sys.argv[1]) if len(sys.argv) > 1 else 3
    c, e = remez_fixed_c0(deg)
    c32 = [np.float32(v) for v in c]
    print(f"degree {deg}, p(0) = 1: minimax relative error {e:.3e}")
    for i, v in enumerate(c32):
        print(f"  c{i} = {float(v):.9e}f  /* {np.float32(v).view(np.uint32):#010x} */")
    err32, pmin = f32_horner_error(c32)
    print(f"float32 Horner: max relative error {err32:.3e}, min p on [0,1) = {pmin!r}")

"""Each plausible mistake planted in the oracle fails at least one pin.

The mutants are text substitutions in a temporary copy of oracle.c, built on
the CPU with gcc; the real oracle is untouched.
"""
import functools
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "causal_strict_lower": ("const int nvis = jb->causal ? i + 1 : n;",
                            "const int nvis = jb->causal ? (i > 0 ? i : 1) : n;"),
    "causal_upper": ("const int nvis = jb->causal ? i + 1 : n;",
                     "const int nvis = jb->causal ? n - i : n;"),
    "no_scale": ("s[j] = jb->scale * dot;", "s[j] = dot;"),
    "scale_squared": ("s[j] = jb->scale * dot;", "s[j] = jb->scale * jb->scale * dot;"),
    "no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "lse_without_max": ("jb->lse[r] = m + log(l);", "jb->lse[r] = log(l);"),
    "lse_log2": ("jb->lse[r] = m + log(l);", "jb->lse[r] = m + log2(l);"),
    "unnormalised": ("const double p = s[j] / l;", "const double p = s[j];"),
    "q_as_key": ("const uint16_t *kj = jb->k +", "const uint16_t *kj = jb->q +"),
    "k_as_value": ("const uint16_t *vj = jb->v +", "const uint16_t *vj = jb->k +"),
    "drop_last_key": ("const int nvis = jb->causal ? i + 1 : n;",
                      "const int nvis = jb->causal ? i + 1 : (n > 1 ? n - 1 : n);"),
    "head_of_query_zero": ("const uint16_t *qi = jb->q + ((t0 + i) * H + h) * (int64_t)d;",
                           "const uint16_t *qi = jb->q + ((t0 + i) * H + 0) * (int64_t)d;"),
    "value_row_of_query": ("const uint16_t *vj = jb->v + ((t0 + j) * H + h) * (int64_t)d;",
                           "const uint16_t *vj = jb->v + ((t0 + i) * H + h) * (int64_t)d;"),
    "dot_drops_last_dim": ("for (int x = 0; x < d; ++x)\n            for (int u = 0; u < KB; ++u)",
                           "for (int x = 0; x < d - 1; ++x)\n            for (int u = 0; u < KB; ++u)"),
    "dot_drops_last_dim_tail": ("for (int x = 0; x < d; ++x)\n            dot +=",
                                "for (int x = 0; x < d - 1; ++x)\n            dot +="),
    "key_block_one_row": ("kj[u] = jb->k + ((t0 + j + u) * H + h)", "kj[u] = jb->k + ((t0 + j) * H + h)"),
    "key_block_q_as_key": ("kj[u] = jb->k + ((t0 + j + u)", "kj[u] = jb->q + ((t0 + j + u)"),
    "key_block_scale_dropped": ("for (int u = 0; u < KB; ++u) s[j + u] = jb->scale * dot[u];",
                                "for (int u = 0; u < KB; ++u) s[j + u] = dot[u];"),
    "query_dims_swapped": ("for (int x = 0; x < d; ++x) qd[x] = widen_bf16(qi[x]);",
                                 "for (int x = 0; x < d; ++x) qd[x] = widen_bf16(qi[x ^ 1]);"),
    "packed_ignores_offset": ("*start = jb->cu[b];", "*start = 0;"),
    "range_high_inclusive": ("const int hi = jb->kv_hi < nvis ? jb->kv_hi : nvis;",
                             "const int hi = jb->kv_hi + 1 < nvis ? jb->kv_hi + 1 : nvis;"),
    "range_ignores_low": ("const int lo = jb->kv_lo > 0 ? jb->kv_lo : 0;", "const int lo = 0;"),
    "range_ignores_causal": ("const int hi = jb->kv_hi < nvis ? jb->kv_hi : nvis;",
                             "const int hi = jb->kv_hi < jb->N ? jb->kv_hi : jb->N;"),
}


@pytest.fixture(scope="module")
def builddir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, builddir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = builddir / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = builddir / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", str(path),
                    "-o", str(so), "-lm"], check=True)
    lib = oracle.load_library(str(so))
    attn = functools.partial(oracle.attention, lib=lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(attn)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


MERGE_MUTANTS = {
    # plain mean of the parts: ignores how much mass each part holds
    "merge_unweighted": lambda o, l: (np.mean(o, axis=0), np.log(np.sum(np.exp(l), axis=0))),
    # weights exp(LSE_s) without normalising by their sum
    "merge_unnormalised": lambda o, l: (np.sum(np.exp(l)[..., None] * o, axis=0),
                                        np.log(np.sum(np.exp(l), axis=0))),
    # log of the mean instead of the sum
    "merge_lse_mean": lambda o, l: (oracle.merge(o, l)[0], np.log(np.mean(np.exp(l), axis=0))),
}


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_mutant_is_caught(name, monkeypatch, oracle_lib):
    import oracle_pins
    monkeypatch.setattr(oracle_pins, "oracle_merge", MERGE_MUTANTS[name])
    attn = functools.partial(oracle.attention, lib=oracle_lib)
    with np.errstate(all="ignore"), pytest.raises(AssertionError):
        oracle_pins.pin_key_range_partition_merge(attn)


MATRIX_SRC = os.path.join(os.path.dirname(oracle.__file__), "matrix.py")
MATRIX_MUTANTS = {
    "causal_upper": ("keys[None, :k_end - lo] > ri[:, None]", "keys[None, :k_end - lo] < ri[:, None]"),
    "causal_strict": ("keys[None, :k_end - lo] > ri[:, None]", "keys[None, :k_end - lo] >= ri[:, None]"),
    "no_scale": ("S = (qh[ri] @ kh[lo:k_end].T) * sc", "S = qh[ri] @ kh[lo:k_end].T"),
    "unnormalised": ("ob = (E / torch.where(seen, l, torch.ones_like(l))[:, None]) @ vh[lo:k_end]",
                     "ob = E @ vh[lo:k_end]"),
    "lse_without_max": ("torch.where(seen, m + torch.log(l), m)", "torch.where(seen, torch.log(l), m)"),
    "k_as_value": ("@ vh[lo:k_end]", "@ kh[lo:k_end]"),
    "range_ignores_low": ("lo, hi = (0, n) if key_range is None else (max(0, int(key_range[0])),",
                          "lo, hi = (0, n) if key_range is None else (0,"),
    "causal_keys_stop_early": ("k_end = min(hi, int(ri.max()) + 1) if causal else hi",
                               "k_end = min(hi, int(ri.max())) if causal else hi"),
    "packed_ignores_offset": ("return torch.from_numpy(_widen(flat[t0:t0 + n, h, :]))",
                              "return torch.from_numpy(_widen(flat[0:n, h, :]))"),
    "head_zero": ("return torch.from_numpy(_widen(flat[t0:t0 + n, h, :]))",
                  "return torch.from_numpy(_widen(flat[t0:t0 + n, 0, :]))"),
}


@pytest.mark.parametrize("name", sorted(MATRIX_MUTANTS))
def test_matrix_mutant_is_caught(name):
    """The same pins catch plausible mistakes in the whole-matrix form."""
    import types
    old, new = MATRIX_MUTANTS[name]
    src = open(MATRIX_SRC).read().replace("from . import _widen, all_rows", "from oracle import _widen, all_rows")
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mod = types.ModuleType(f"matrix_{name}")
    exec(compile(src.replace(old, new), f"matrix_{name}.py", "exec"), mod.__dict__)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod.attention)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"

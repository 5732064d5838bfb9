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
    "dot_drops_last_dim": ("for (int x = 0; x < d; ++x)\n            dot +=",
                           "for (int x = 0; x < d - 1; ++x)\n            dot +="),
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

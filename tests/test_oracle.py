"""The fp64 oracle against its pins (CPU only)."""
import functools

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS
from oracle.online import online_attention
from exact_attention_107_amd.workloads import RUNS, make_inputs


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(functools.partial(oracle.attention, lib=oracle_lib))


def test_online_rescale_counts():
    """Conditional rescale skips most corrections on a long N(0,1) row set
    (the pages report about 90% skipped); strict never skips a needed one."""
    inp = make_inputs(RUNS["mid"], B=1, H=1, N=1024)
    q, k, v = (inp[x][0, :, 0] for x in ("q", "k", "v"))
    _, _, n_always = online_attention(q, k, v, scale=inp["scale"], causal=False, Br=64, Bc=64,
                                      rescale="always")
    _, _, n_strict = online_attention(q, k, v, scale=inp["scale"], causal=False, Br=64, Bc=64,
                                      rescale="strict")
    _, _, n_thr = online_attention(q, k, v, scale=inp["scale"], causal=False, Br=64, Bc=64,
                                   rescale="threshold", tau=8 * np.log(2))
    blocks = 1024 * (1024 // 64 - 1)
    assert n_strict < 0.5 * blocks
    assert n_thr <= n_strict


def test_row_validation(oracle_lib):
    q = np.zeros((1, 4, 1, 8), dtype=np.uint16)
    with pytest.raises(RuntimeError):
        oracle.attention(q, q, q, scale=1.0, causal=False, rows=np.array([[0, 0, 4]]), lib=oracle_lib)
    with pytest.raises(RuntimeError):
        oracle.attention(q, q, q, scale=1.0, causal=False, rows=np.array([[0, 1, 0]]), lib=oracle_lib)

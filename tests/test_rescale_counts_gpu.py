"""The counting instance of the forward (fa_fwd_rescale_counts, needs an MI355X).

It must compute exactly what fa_fwd_variant computes, count one wave-step per
64-key tile after each wave's first, and its counts must follow the rescale
rules: no reference moves when every score is equal, every step rescales
when each key tile raises every row's maximum by more than the threshold, and
the threshold rule never moves a row that the strict rule leaves alone.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import Run, bf16_bits, make_inputs
from gpu_helpers import assert_within, full_parity, run_gpu, to_dev

pytestmark = pytest.mark.gpu

ROWS, KEYS, WAVES = 256, 64, 8  # d = 128 geometry: rows per workgroup, keys per tile, waves


def expected_steps(B, H, N, causal):
    """Wave-steps after each wave's first key tile, from the tile geometry."""
    steps = 0
    for q0 in range(0, N, ROWS):
        kv_end = min(N, q0 + ROWS) if causal else N
        kt_end = -(-kv_end // KEYS)
        for w in range(WAVES):
            wrow0 = q0 + 32 * w
            nkv_w = min(kt_end, (wrow0 + 31) // KEYS + 1) if causal else kt_end
            steps += max(nkv_w - 1, 0)
    return B * H * steps


def counted(inp, mode):
    q, k, v = (to_dev(inp[x]) for x in ("q", "k", "v"))
    c = torch.zeros(4, dtype=torch.int64, device="cuda")
    o, lse = fa.fwd(q, k, v, causal=inp["causal"], scale=inp["scale"], rescale_mode=mode, counts=c)
    torch.cuda.synchronize()
    return o, lse, [int(x) for x in c.cpu().tolist()]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mode", [fa.RESCALE_STRICT, fa.RESCALE_THRESHOLD])
def test_same_result_and_step_count(causal, mode):
    inp = make_inputs(Run("cnt", 2, 3, 1000, 128, causal, 31, sigma_qk=3.0, boost_frac=0.01))
    o, lse, c = counted(inp, mode)
    o_ref, lse_ref = run_gpu(inp, rescale_mode=mode, exp_mode=fa.EXP_HW)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, lse_ref)
    steps = expected_steps(2, 3, 1000, causal)
    assert c[0] == steps and c[3] == 32 * steps
    assert 0 <= c[1] <= c[0] and 0 <= c[2] <= c[3]


@pytest.mark.parametrize("mode", [fa.RESCALE_STRICT, fa.RESCALE_THRESHOLD])
def test_equal_scores_never_rescale(mode):
    inp = make_inputs(Run("cnt0", 1, 2, 700, 128, False, 32))
    inp["q"] = np.zeros_like(inp["q"])
    o, lse, c = counted(inp, mode)
    assert c[0] == expected_steps(1, 2, 700, False) and c[1] == 0 and c[2] == 0


@pytest.mark.parametrize("mode", [fa.RESCALE_STRICT, fa.RESCALE_THRESHOLD])
def test_rising_scores_rescale_every_step(mode):
    """Q = 1, K = t + 1 on key tile t: each tile raises every row's scaled log2
    score by 128 / sqrt(128) * log2(e) ~ 16.3 > 8."""
    B, H, N, d = 1, 2, 768, 128  # whole workgroups: no padding rows
    inp = make_inputs(Run("cnt1", B, H, N, d, False, 33))
    inp["q"] = bf16_bits(np.ones((B, N, H, d), np.float32))
    tile = (np.arange(N) // KEYS + 1).astype(np.float32)
    inp["k"] = bf16_bits(np.broadcast_to(tile[None, :, None, None], (B, N, H, d)).copy())
    o, lse, c = counted(inp, mode)
    steps = expected_steps(B, H, N, False)
    assert c[0] == steps and c[1] == steps and c[2] == 32 * steps
    m, _ = full_parity(inp, rescale_mode=mode, exp_mode=fa.EXP_HW)
    assert_within(m, "rising scores")


def test_threshold_moves_a_subset_of_strict():
    inp = make_inputs(Run("cnt2", 2, 4, 2048, 128, True, 34))
    _, _, cs = counted(inp, fa.RESCALE_STRICT)
    _, _, ct = counted(inp, fa.RESCALE_THRESHOLD)
    assert cs[0] == ct[0] and cs[3] == ct[3]
    assert ct[1] <= cs[1] and ct[2] <= cs[2]
    print("strict", cs, "threshold", ct)

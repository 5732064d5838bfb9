"""HIP path at the size limits of the C ABI (needs an MI355X).

- a long sequence (N = 131072 keys, 2048 key tiles per query tile), causal and
  not, on sampled rows;
- the largest token stride the library accepts (H * d = 2^22 elements, 8 MiB
  between consecutive tokens of one head), which drives the per-lane buffer
  offsets of the direct loads and stores to their largest values, on sampled
  rows of every sampled head.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import Run, make_inputs
from gpu_helpers import assert_within, run_gpu, sampled_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence(causal):
    run = Run("long131k", 1, 2, 131072, 128, causal, 2024)
    inp = make_inputs(run)
    o, lse = run_gpu(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    m = sampled_parity(inp, o, lse, count=96, seed=1)
    print("N=131072 causal", causal, m)
    assert_within(m, f"N=131072 causal={causal}")


@pytest.mark.parametrize("d,H,N,causal", [(64, 65536, 24, False), (128, 32768, 70, True)])
def test_largest_token_stride(d, H, N, causal):
    assert H * d == 1 << 22  # the largest H * d the library accepts
    run = Run("stride", 1, H, N, d, causal, 2025)
    inp = make_inputs(run)
    o, lse = run_gpu(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    m = sampled_parity(inp, o, lse, count=256, seed=2)
    print(f"H*d=2^22 d={d}", m)
    assert_within(m, f"token stride 2^22 d={d}")


def test_token_stride_past_limit_rejected():
    """One element more per token than the library accepts: FA_ERR_SHAPE, no launch."""
    d, H = 64, (1 << 16) + 1
    q = torch.zeros((1, 1, H, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fwd(q, q, q)
    assert e.value.code == 2

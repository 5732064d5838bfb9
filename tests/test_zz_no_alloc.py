"""The allocation-free split-KV entry point (fa_fwd_splitkv_static) through
the C ABI, against the workspace entry point fa_fwd_splitkv (needs an
MI355X).  Two calls in a row share the GPU's static scratch, the second on a
smaller input; each must equal fa_fwd_splitkv bit for bit, and the small one
the oracle within the forward's tolerances."""
from __future__ import annotations

import pytest
import torch

from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import Run, make_inputs
from gpu_helpers import assert_within, from_dev, metrics, to_dev

pytestmark = pytest.mark.gpu

# (B, H, N, d, causal, splits): the first fills 63.0 of the 64 MiB scratch
CALLS = [(1, 4, 16000, 128, False, 2), (1, 2, 1000, 64, True, 2)]


def test_static_scratch_matches_workspace_entry_two_calls():
    import oracle
    for i, (B, H, N, d, causal, S) in enumerate(CALLS):
        assert S * B * N * H * (d + 1) * 4 <= fa.STATIC_SCRATCH_BYTES
        inp = make_inputs(Run("static", B, H, N, d, causal, 300 + i))
        q, k, v = (to_dev(inp[x]) for x in ("q", "k", "v"))
        o_ref, l_ref = fa.fwd_splitkv(q, k, v, causal=causal, scale=inp["scale"], splits=S)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
        fa.fwd_splitkv_static(q, k, v, causal=causal, scale=inp["scale"], splits=S, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"call {i}"
        assert torch.equal(lse, l_ref), f"call {i}"
        if i == 1:
            ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=causal)
            assert_within(metrics(from_dev(o), lse.cpu().numpy(), ro, rl), "static split-KV")


def test_static_scratch_rejects_oversized_request():
    B, H, N, d = 1, 4, 16384, 128
    q = torch.zeros(B, N, H, d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fwd_splitkv_static(q, q, q, splits=2)
    assert e.value.code == fa.FA_ERR_SCRATCH

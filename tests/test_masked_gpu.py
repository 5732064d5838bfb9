"""Window mask and linear distance bias (fa_fwd_masked), HIP path vs the
oracle, through the C ABI (needs an MI355X).  Same tolerances as fa_fwd:
the modifications change which scores enter the softmax and add an exact
fp32 term to them, nothing else."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import Run, make_inputs
from gpu_helpers import assert_within, from_dev, metrics, to_dev
from oracle import mods as omods

pytestmark = pytest.mark.gpu


def _alibi(H):
    # the usual geometric slopes 2^(-8 (h + 1) / H)
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], np.float32)


def _run(inp, left, right, slopes):
    q, k, v = (to_dev(inp[x]) for x in ("q", "k", "v"))
    sl = torch.from_numpy(slopes).cuda() if slopes is not None else None
    o, lse = fa.fwd_masked(q, k, v, window_left=left, window_right=right, alibi_slopes=sl, scale=inp["scale"])
    torch.cuda.synchronize()
    return o, lse


WINDOWS = [(-1, 0), (128, 0), (100, 37), (0, 0), (-1, 200), (300, -1), (63, 64), (-1, -1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", WINDOWS, ids=lambda w: f"{w[0]}_{w[1]}")
@pytest.mark.parametrize("bias", [False, True])
def test_masked_small(d, window, bias):
    inp = make_inputs(Run("mk", 1, 3, 700, d, False, 91))
    slopes = _alibi(3) if bias else None
    o, lse = _run(inp, *window, slopes)
    ro, rl = omods.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], left=window[0], right=window[1],
                             slopes=slopes)
    m = metrics(from_dev(o), lse.cpu().numpy(), ro, rl)
    print(f"d={d} window={window} bias={bias} {m}")
    assert_within(m, f"window={window} bias={bias}")


def test_masked_d256_and_ragged_batch():
    inp = make_inputs(Run("mk2", 2, 2, 333, 256, False, 92))
    slopes = _alibi(2)
    o, lse = _run(inp, 50, 10, slopes)
    ro, rl = omods.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], left=50, right=10, slopes=slopes)
    assert_within(metrics(from_dev(o), lse.cpu().numpy(), ro, rl), "d=256")


def test_masked_full_size_sampled():
    """A long sliding-window causal run with ALiBi at benchmark size, on
    sampled rows."""
    inp = make_inputs(Run("mkl", 1, 16, 16384, 128, False, 93))
    slopes = _alibi(16)
    o, lse = _run(inp, 1024, 0, slopes)
    rng = np.random.Generator(np.random.PCG64(3))
    rows = np.array([(0, int(rng.integers(16)), i) for i in
                     [0, 1, 1023, 1024, 1025, 8191, 16383] + list(rng.integers(0, 16384, 1200))], dtype=np.int64)
    ro, rl = omods.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], left=1024, right=0, slopes=slopes,
                             rows=rows)
    rt = torch.from_numpy(rows)
    og = from_dev(o[rt[:, 0].cuda(), rt[:, 2].cuda(), rt[:, 1].cuda()])
    lg = lse[rt[:, 0].cuda(), rt[:, 1].cuda(), rt[:, 2].cuda()].cpu().numpy()
    assert_within(metrics(og, lg, ro, rl), "sliding window 1024")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_masked_rejects_bad_arguments():
    q = torch.zeros(1, 64, 1, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError):
        fa.fwd_masked(q, q.clone(), q.clone(), window_left=4, window_right=0)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_masked_huge_window_edges_mean_unbounded(d):
    """An edge of N - 1 or more hides no key: INT_MAX (and N, N + 5) on either
    side give bitwise the result of an unbounded side."""
    inp = make_inputs(Run("mkw", 2, 2, 300, d, False, 94))
    big = 2 ** 31 - 1
    ref = _run(inp, -1, -1, None)
    ref_c = _run(inp, -1, 0, None)
    for left, right, r in ((big, big, ref), (-1, big, ref), (big, -1, ref), (300, 305, ref), (big, 0, ref_c),
                           (299, 0, ref_c)):
        o, lse = _run(inp, left, right, None)
        assert torch.equal(o.view(torch.int16), r[0].view(torch.int16)), (left, right)
        assert torch.equal(lse, r[1]), (left, right)
    ro, rl = omods.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], left=-1, right=-1, slopes=None)
    assert_within(metrics(from_dev(ref[0]), ref[1].cpu().numpy(), ro, rl), "unbounded window")


# ---------------------------------------------------------------------------
# Packed sequences (cu_seqlens): positions count from each sequence's start.

PACKED_LENGTHS = [1, 0, 5, 130, 257, 64, 300, 33]


def _packed(lengths, d, H=3, seed=94):
    return make_inputs(Run("mkp", len(lengths), H, 0, d, False, seed, varlen=True), lengths=lengths)


def _run_packed(inp, left, right, slopes):
    q, k, v = (to_dev(inp[x]) for x in ("q", "k", "v"))
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], dtype=np.int32)).cuda()
    sl = torch.from_numpy(slopes).cuda() if slopes is not None else None
    o, lse = fa.fwd_masked_packed(q, k, v, cu, window_left=left, window_right=right, alibi_slopes=sl,
                                  scale=inp["scale"])
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [(-1, 0), (100, 37), (0, 0), (-1, -1), (63, 64)], ids=lambda w: f"{w[0]}_{w[1]}")
@pytest.mark.parametrize("bias", [False, True])
def test_masked_packed_small(d, window, bias):
    """Empty, one-token and ragged sequences, every element."""
    inp = _packed(PACKED_LENGTHS, d)
    slopes = _alibi(3) if bias else None
    o, lse = _run_packed(inp, *window, slopes)
    ro, rl = omods.attention_packed(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], scale=inp["scale"],
                                    left=window[0], right=window[1], slopes=slopes)
    m = metrics(from_dev(o), lse.cpu().numpy(), ro, rl)
    print(f"packed d={d} window={window} bias={bias} {m}")
    assert_within(m, f"packed window={window} bias={bias}")


def test_masked_packed_equals_dense_bitwise():
    """Each packed sequence gives bitwise the output of a dense masked run of
    it alone."""
    lengths = [37, 300, 129, 64]
    inp = _packed(lengths, 128, H=2, seed=95)
    slopes = _alibi(2)
    o, lse = _run_packed(inp, 40, 5, slopes)
    cu = inp["cu_seqlens"]
    for b, n in enumerate(lengths):
        t0 = int(cu[b])
        one = {x: inp[x][None, t0:t0 + n] for x in ("q", "k", "v")}
        one["scale"] = inp["scale"]
        od, ld = _run(one, 40, 5, slopes)
        assert torch.equal(o[t0:t0 + n].view(torch.int16), od[0].view(torch.int16)), b
        assert torch.equal(lse[:, t0:t0 + n], ld[0]), b


def test_masked_packed_many_sequences():
    """More than 64 sequences (the decode walks them 64 at a time)."""
    rng = np.random.default_rng(96)
    lengths = [int(x) for x in rng.integers(0, 160, size=150)]
    inp = _packed(lengths, 64, H=2, seed=97)
    slopes = _alibi(2)
    o, lse = _run_packed(inp, 20, 0, slopes)
    ro, rl = omods.attention_packed(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], scale=inp["scale"],
                                    left=20, right=0, slopes=slopes)
    assert_within(metrics(from_dev(o), lse.cpu().numpy(), ro, rl), "150 sequences")

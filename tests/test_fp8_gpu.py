"""FP8 (E4M3) forward and quantisation, HIP path vs the oracle, through the C
ABI (needs an MI355X).

Quantisation is compared bit for bit (codes and descales).  The FP8 forward
is compared with the exact attention of the dequantised inputs under
per-element bounds derived from the two lossy steps:
  * the E4M3 products are accumulated with a relative error of at most
    2^-11 of the sum of the products' magnitudes (measured on the MFMA by
    exact_attention_107_amd/microbench/fp8_acc.hip against exact sums: worst
    2^-12.1 over 65 536 dot products of uniformly drawn codes; small products
    are truncated against the largest), so a score carries
    d_ij = 2^-11 scale sum_k |q_ik k_jk|;
  * the weights are rounded to E4M3 (relative 2^-4 for normal codes; below
    the normal range an absolute 2^-18 of the row max).
With P_ij the exact normalised weights and v_j the dequantised value rows,
    |dO_i| <= sum_j P_ij (2^-4 + e^(2 d_ij) - 1) |v_j| + 2^-18 sum_j |v_j|
              + 2^-8 |O_i| + 1e-5        (bf16 output, fp32 accumulation),
    |dLSE_i| <= max_j d_ij + 1e-5        (the row sum is taken from fp32 P)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from exact_attention_107_amd import fa
from exact_attention_107_amd.workloads import RUNS, Run, make_inputs
from gpu_helpers import from_dev, sample_rows
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu


def _codes_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _quantized(inp):
    q8, dq = ofp8.quantize(inp["q"])
    k8, dk = ofp8.quantize(inp["k"])
    vt8, dv = ofp8.quantize(inp["v"], transpose=True)
    return q8, k8, vt8, dq, dk, dv


ACC_REL = 2.0 ** -11   # E4M3 MFMA accumulation, relative to sum |products|


def _bound_rows(q8, k8, vt8, dq, dk, dv, scale, causal, rows):
    """Per-element O bounds and per-row LSE bounds for the (b, h, i) rows."""
    N = q8.shape[1]
    Q = ofp8.e4m3_decode(q8) * dq[:, None, :, None]
    K = ofp8.e4m3_decode(k8) * dk[:, None, :, None]
    Vt = ofp8.e4m3_decode(vt8[..., :N]) * dv[:, :, None, None]
    sc = float(np.float32(scale))
    out = np.zeros((len(rows), q8.shape[3]))
    lse_b = np.zeros(len(rows))
    for r, (b, h, i) in enumerate(rows):
        nvis = i + 1 if causal else N
        s = (K[b, :nvis, h] @ Q[b, i, h]) * sc
        p = np.exp(s - s.max())
        p /= p.sum()
        delta = ACC_REL * sc * (np.abs(K[b, :nvis, h]) @ np.abs(Q[b, i, h]))
        av = np.abs(Vt[b, h][:, :nvis])
        out[r] = av @ (p * (2.0 ** -4 + np.expm1(2 * delta))) + 2.0 ** -18 * av.sum(axis=1)
        lse_b[r] = delta.max() + 1e-5
    return out, lse_b


def _run_fp8(q8, k8, vt8, dq, dk, dv, scale, causal):
    o, lse = fa.fwd_fp8(_codes_dev(q8), _codes_dev(k8), _codes_dev(vt8), _codes_dev(dq), _codes_dev(dk),
                        _codes_dev(dv), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check_rows(inp, causal, q8, k8, vt8, dq, dk, dv, o, lse, rows, what):
    o_ref, l_ref = ofp8.attention(q8, k8, vt8, dq, dk, dv, scale=inp["scale"], causal=causal, rows=rows)
    rt = torch.from_numpy(rows)
    og = from_dev(o[rt[:, 0].cuda(), rt[:, 2].cuda(), rt[:, 1].cuda()])
    lg = lse[rt[:, 0].cuda(), rt[:, 1].cuda(), rt[:, 2].cuda()].cpu().numpy().astype(np.float64)
    bound, lse_bound = _bound_rows(q8, k8, vt8, dq, dk, dv, inp["scale"], causal, rows)
    bound = bound + 2.0 ** -8 * np.abs(o_ref) + 1e-5
    err = np.abs(og - o_ref)
    lerr = np.abs(lg - l_ref)
    print(f"{what}: max|dO| {err.max():.3e} mean|dO| {err.mean():.3e} max err/bound {np.max(err / bound):.3f} "
          f"max|dLSE| {lerr.max():.2e} max dLSE/bound {np.max(lerr / lse_bound):.3f}")
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    assert np.all(err <= bound), f"{what}: error above the E4M3 bound, worst ratio {np.max(err / bound):.3f}"
    assert np.all(lerr <= lse_bound), f"{what}: LSE above its bound, worst ratio {np.max(lerr / lse_bound):.3f}"


def _all_rows(B, H, N):
    return np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(N)], dtype=np.int64)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("transpose", [False, True])
def test_quantize_bit_exact(d, transpose):
    inp = make_inputs(Run("q", 2, 3, 130, d, False, 81, sigma_qk=2.0))
    x = inp["q"].copy()
    x[1, :, 2, :] = 0  # an all-zero head
    codes, ds = fa.quantize_fp8(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda(),
                                transpose=transpose)
    torch.cuda.synchronize()
    ref_c, ref_d = ofp8.quantize(x, transpose=transpose)
    assert np.array_equal(ds.cpu().numpy(), ref_d)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_small_ragged(d, causal):
    inp = make_inputs(Run("f8", 2, 3, 300, d, causal, 82))
    qz = _quantized(inp)
    o, lse = _run_fp8(*qz, inp["scale"], causal)
    _check_rows(inp, causal, *qz, o, lse, _all_rows(2, 3, 300), f"d={d} causal={causal}")


@pytest.mark.parametrize("N", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_fwd_edge_lengths(N, causal):
    inp = make_inputs(Run("f8e", 1, 2, N, 128, causal, 400 + N))
    qz = _quantized(inp)
    o, lse = _run_fp8(*qz, inp["scale"], causal)
    _check_rows(inp, causal, *qz, o, lse, _all_rows(1, 2, N), f"N={N} causal={causal}")


def test_fp8_fwd_wide_logits():
    inp = make_inputs(Run("f8w", 1, 2, 500, 128, False, 83, sigma_qk=3.0, boost_frac=0.01))
    qz = _quantized(inp)
    o, lse = _run_fp8(*qz, inp["scale"], False)
    _check_rows(inp, False, *qz, o, lse, _all_rows(1, 2, 500), "wide logits")


def test_fp8_fwd_deterministic():
    inp = make_inputs(Run("f8d", 1, 2, 700, 128, True, 84))
    qz = _quantized(inp)
    a = _run_fp8(*qz, inp["scale"], True)
    b = _run_fp8(*qz, inp["scale"], True)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", ["wide", "mid_causal", "wide_d256"])
def test_fp8_fwd_full_size_sampled(name):
    """The benchmark shapes at full size on sampled rows."""
    run = RUNS[name]
    inp = make_inputs(run)
    qz = _quantized(inp)
    o, lse = _run_fp8(*qz, inp["scale"], run.causal)
    rows = sample_rows(inp, 1500, seed=9)
    _check_rows(inp, run.causal, *qz, o, lse, rows, name)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_fp8_end_to_end_against_bf16_oracle():
    """GPU quantisation + FP8 forward against the exact bf16-input attention:
    the inputs' own E4M3 rounding adds error, so only its size is checked
    loosely (informational)."""
    import oracle
    inp = make_inputs(Run("f8x", 1, 2, 256, 128, False, 85))
    x = {n: torch.from_numpy(inp[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    q8, dq = fa.quantize_fp8(x["q"])
    k8, dk = fa.quantize_fp8(x["k"])
    vt8, dv = fa.quantize_fp8(x["v"], transpose=True)
    o, lse = fa.fwd_fp8(q8, k8, vt8, dq, dk, dv, scale=inp["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=False)
    err = np.abs(from_dev(o) - o_ref)
    print(f"end to end: max|dO| {err.max():.3e} mean|dO| {err.mean():.3e} "
          f"max|dLSE| {np.abs(lse.cpu().numpy() - l_ref).max():.3e}")
    assert err.mean() <= 2e-2


# ---------------------------------------------------------------------------
# Packed sequences (cu_seqlens): per-(sequence, head) scales, the packed V^T
# layout, work items decoded from cu_seqlens.

def _packed(lengths, d, seed, H=3, sigma=1.0):
    r = Run("f8p", len(lengths), H, 0, d, True, seed, varlen=True, sigma_qk=sigma)
    inp = make_inputs(r, lengths=lengths)
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int32)
    return inp, cu


def _quantized_packed(inp, cu):
    q8, dq = ofp8.quantize_packed(inp["q"], cu)
    k8, dk = ofp8.quantize_packed(inp["k"], cu)
    vt8, dv = ofp8.quantize_packed(inp["v"], cu, transpose=True)
    return q8, k8, vt8, dq, dk, dv


def _run_fp8_packed(q8, k8, vt8, dq, dk, dv, cu, scale, causal):
    o, lse = fa.fwd_fp8_packed(_codes_dev(q8), _codes_dev(k8), _codes_dev(vt8), _codes_dev(dq), _codes_dev(dk),
                               _codes_dev(dv), _codes_dev(cu), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _check_packed(inp, cu, causal, qz, o, lse, what, seqs=None, rows_per_seq=None, seed=0):
    """Rows of the listed sequences (all rows, or a sample of rows_per_seq)
    against the exact attention of the sequence's dequantised inputs, under
    the dense bounds applied to the sequence alone."""
    q8, k8, vt8, dq, dk, dv = qz
    starts = ofp8.padded_starts(cu)
    lengths = np.diff(cu)
    rng = np.random.default_rng(seed)
    checked = 0
    for b in (range(len(lengths)) if seqs is None else seqs):
        n = int(lengths[b])
        if n == 0:
            continue
        t0, st = int(cu[b]), int(starts[b])
        one = dict(scale=inp["scale"])
        sq = (q8[None, t0:t0 + n], k8[None, t0:t0 + n], vt8[None, :, :, st:st + n],
              dq[b:b + 1], dk[b:b + 1], dv[b:b + 1])
        H = q8.shape[1]
        if rows_per_seq is None or rows_per_seq >= n * H:
            rows = _all_rows(1, H, n)
        else:
            pick = rng.choice(n * H, size=rows_per_seq, replace=False)
            rows = np.stack([np.zeros_like(pick), pick % H, pick // H], axis=1)
        o1 = o[t0:t0 + n][None]
        l1 = lse[:, t0:t0 + n][None]
        _check_rows(one, causal, *sq, o1, l1, rows, f"{what} seq {b} (n={n})")
        checked += len(rows)
    assert checked > 0


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("transpose", [False, True])
def test_quantize_packed_bit_exact(d, transpose):
    inp, cu = _packed([1, 0, 5, 130, 257, 64, 300, 33], d, 91, sigma=2.0)
    x = inp["q"].copy()
    x[cu[3]:cu[4], 1, :] = 0  # an all-zero (sequence, head)
    codes, ds = fa.quantize_fp8_packed(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda(),
                                       _codes_dev(cu), transpose=transpose)
    torch.cuda.synchronize()
    ref_c, ref_d = ofp8.quantize_packed(x, cu, transpose=transpose)
    assert np.array_equal(ds.cpu().numpy(), ref_d)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_packed_small(d, causal):
    """Empty, one-token and ragged sequences, every row."""
    inp, cu = _packed([1, 0, 5, 130, 257, 64, 300, 33], d, 92)
    qz = _quantized_packed(inp, cu)
    o, lse = _run_fp8_packed(*qz, cu, inp["scale"], causal)
    _check_packed(inp, cu, causal, qz, o, lse, f"packed d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_packed_equals_dense_bitwise(causal):
    """Each packed sequence gives bitwise the O and LSE of a dense FP8 run of
    it alone with the same codes and scales."""
    lengths = [37, 300, 129, 64]
    inp, cu = _packed(lengths, 128, 93)
    q8, k8, vt8, dq, dk, dv = _quantized_packed(inp, cu)
    o, lse = _run_fp8_packed(q8, k8, vt8, dq, dk, dv, cu, inp["scale"], causal)
    starts = ofp8.padded_starts(cu)
    for b, n in enumerate(lengths):
        t0, st, pad = int(cu[b]), int(starts[b]), (n + 63) // 64 * 64
        od, ld = _run_fp8(q8[None, t0:t0 + n], k8[None, t0:t0 + n], vt8[None, :, :, st:st + pad],
                          dq[b:b + 1], dk[b:b + 1], dv[b:b + 1], inp["scale"], causal)
        assert torch.equal(o[t0:t0 + n].view(torch.int16), od[0].view(torch.int16)), b
        assert torch.equal(lse[:, t0:t0 + n], ld[0]), b


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_packed_many_sequences(causal):
    """More than 64 sequences (the decode walks them 64 at a time)."""
    rng = np.random.default_rng(94)
    lengths = [int(x) for x in rng.integers(0, 160, size=150)]
    inp, cu = _packed(lengths, 64, 95, H=2)
    qz = _quantized_packed(inp, cu)
    o, lse = _run_fp8_packed(*qz, cu, inp["scale"], causal)
    _check_packed(inp, cu, causal, qz, o, lse, f"150 sequences causal={causal}")


def test_fp8_packed_workload_sampled():
    """The packed causal benchmark batch (32 sequences of 128..8192 tokens, 16
    heads) at full size.  The oracle quantises the shortest, a middle and the
    longest sequence; the others hold zero codes with unit scales (they are
    launched but not checked), and sampled rows of the three are checked."""
    run = RUNS["varlen_causal"]
    inp = make_inputs(run)
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int32)
    lengths = np.diff(cu)
    order = np.argsort(lengths, kind="stable")
    seqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    T, H, d = inp["q"].shape
    B = len(lengths)
    Tp = ofp8.vt_stride_packed(T, B)
    q8 = np.zeros((T, H, d), np.uint8)
    k8 = np.zeros((T, H, d), np.uint8)
    vt8 = np.zeros((H, d, Tp), np.uint8)
    dq, dk, dv = (np.ones((B, H), np.float32) for _ in range(3))
    starts = ofp8.padded_starts(cu)
    for b in seqs:
        t0, n, st = int(cu[b]), int(lengths[b]), int(starts[b])
        one = np.array([0, n], np.int32)
        c, s_ = ofp8.quantize_packed(inp["q"][t0:t0 + n], one)
        q8[t0:t0 + n], dq[b] = c, s_[0]
        c, s_ = ofp8.quantize_packed(inp["k"][t0:t0 + n], one)
        k8[t0:t0 + n], dk[b] = c, s_[0]
        c, s_ = ofp8.quantize_packed(inp["v"][t0:t0 + n], one, transpose=True)
        vt8[:, :, st:st + n], dv[b] = c[:, :, :n], s_[0]
    qz = (q8, k8, vt8, dq, dk, dv)
    o, lse = _run_fp8_packed(*qz, cu, inp["scale"], True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    _check_packed(inp, cu, True, qz, o, lse, "varlen_causal", seqs=seqs, rows_per_seq=600, seed=96)

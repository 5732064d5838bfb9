"""bench.py on the CPU: the parts of its contract that need no GPU.

- more than one GPU is refused with a message and exit code 2 (the forward is a
  single-GPU kernel with no collectives);
- the stored HBM-traffic record is used only while the forward kernel's sources
  are unchanged (its fingerprint must match), and then it is close to the
  algorithmic bytes;
- the sampled-parity helper flags an output outside the forward's tolerances.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_traffic_record_only_for_its_kernel():
    fp = bench.kernel_fingerprint()
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert bench.traffic_for("0" * 16) is None
    if rec["kernel_fingerprint"] != fp:
        # sources changed since the counters were taken: the bench reports null
        assert bench.traffic_for(fp) is None
        return
    assert bench.traffic_for(fp) == rec["bytes_per_launch"]
    # the measured bytes are the algorithmic ones within a few per cent
    alg = rec["algorithmic_read_bytes"] + rec["algorithmic_write_bytes"]
    assert abs(rec["bytes_per_launch"] / alg - 1.0) < 0.05


def test_sampled_parity_flags_errors(monkeypatch):
    # CPU tensors stand in for device ones: sampled_parity moves its indices with .cuda()
    monkeypatch.setattr(torch.Tensor, "cuda", lambda self, *a, **k: self)
    B, N, H, d = 1, 4, 2, 8
    rng = np.random.Generator(np.random.PCG64(0))
    o_ref = rng.standard_normal((3, d))
    lse_ref = rng.standard_normal(3)
    rows = np.array([[0, 0, 1], [0, 1, 3], [0, 1, 0]], dtype=np.int64)
    o = torch.zeros((B, N, H, d), dtype=torch.bfloat16)
    lse = torch.zeros((B, H, N), dtype=torch.float32)
    for r, (b, h, i) in enumerate(rows):
        o[b, i, h] = torch.from_numpy(o_ref[r]).to(torch.bfloat16)
        lse[b, h, i] = float(lse_ref[r])
    inp = {"cu_seqlens": None}
    good = bench.sampled_parity(inp, rows, o_ref, lse_ref, o, lse, torch)
    assert good["pass"] and good["rows"] == 3
    o[0, 3, 1, 5] += 0.25
    bad = bench.sampled_parity(inp, rows, o_ref, lse_ref, o, lse, torch)
    assert not bad["pass"] and bad["max_abs_o"] > 0.2

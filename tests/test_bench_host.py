"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the
algorithmic FLOP counts behind the roofline figures (checked against brute
force over blocks and token pairs), and the profile record that is reported
only while the profiled kernel source is unchanged."""
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from block_sparse_causal_amd import stem
from block_sparse_causal_amd import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_attention_flops_count_executed_blocks():
    # 4 B^2 d per executed (head, query block, key block); the diagonal
    # block's causal half counted once when diag_half is set
    w = syn.custom([1000, 77, 2050], 4, 2, 64, "bf16", 64, sink_blocks=1, k_min=3, rho0=0.5,
                   tau=6.0)
    p = stem.plan_for(w)
    i = p.info
    tile = 4.0 * w.block * w.block * w.head_dim
    executed = int(np.asarray(p.budget).sum())
    assert bench.attn_flops(p, diag_half=False) == tile * executed * w.num_q_heads
    assert bench.attn_flops(p, diag_half=True) == \
        tile * (executed - 0.5 * i.total_blocks) * w.num_q_heads


@pytest.mark.parametrize("stride", [1, 2, 8, 64])
def test_antidiag_flops_count_sampled_pairs(stride):
    # 2 d per (query token, key token) pair on a sampled anti-diagonal with
    # the key not after the query, counted by brute force
    w = syn.custom([130, 64, 9], 2, 1, 64, "bf16", 64)
    pairs = 0
    for n in w.seqlens:
        for qp in range(n):
            for kp in range(qp + 1):
                if qp // stride >= kp // stride and \
                        (qp % stride) + (kp % stride) == stride - 1:
                    pairs += 1
    assert bench.antidiag_flops(w, stride) == 2.0 * w.head_dim * pairs * w.num_q_heads


def test_traffic_record_only_for_the_profiled_source(tmp_path, monkeypatch):
    src_dir = tmp_path / "block_sparse_causal_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "attn.hip"
    src.write_bytes(b"kernel v1")
    sha = hashlib.sha256(b"kernel v1").hexdigest()
    rec = {"kernel": "k", "source_sha256": sha, "fetch_bytes": 10, "write_bytes": 5}
    (tmp_path / "profiles" / "attn_w.md").write_text(
        "# profile\n\ntraffic_record: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_record("w") == rec
    src.write_bytes(b"kernel v2")
    assert bench.traffic_record("w") is None
    assert bench.traffic_record("missing") is None

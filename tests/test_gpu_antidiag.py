"""GPU parity of the anti-diagonal sampled metric (stem_score_antidiag,
through the C ABI) against the oracle, and of the path that selects and
attends with it.

Small workloads are checked on every metric row and every selection row,
over strides from 1 (every causal token pair) to the block size (one group
per block), ragged and empty sequences, sequences too short to hold a
sample, B = 64 / 128, d = 64 / 128, bf16 and f32 inputs and the three metric
forms.  The 128K
layer runs in the benchmark's configuration (stride 16) and is checked on
sampled metric rows, every selection row and sampled attention rows.
"""
import numpy as np
import pytest

from block_sparse_causal_amd import stem
from block_sparse_causal_amd import synthetic as syn
from oracle import stem_oracle as O
from tests import _harness as H
from tests._golden import pages_parameters

pytestmark = pytest.mark.gpu


def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


W = {
    "b64-d128-varlen": syn.custom([1000, 77, 0, 2050], 8, 2, 128, "bf16", 64,
                                  sink_blocks=2, k_min=3, rho0=0.5, tau=8.0, seed=31),
    "b128-d128-gqa4": syn.custom([4100, 300], 4, 1, 128, "bf16", 128,
                                 sink_blocks=1, k_min=4, rho0=0.4, tau=6.0, seed=32),
    "b64-d64-gqa7": syn.custom([1500], 7, 1, 64, "bf16", 64,
                               sink_blocks=3, k_min=2, rho0=1.0, tau=4.0, seed=33),
    "b128-d64-short": syn.custom([1337, 1, 3], 2, 2, 64, "bf16", 128,
                                 sink_blocks=0, k_min=1, rho0=0.2, tau=3.0, seed=34),
    "b64-d128-tiny": syn.custom([1, 3, 5, 9, 67, 0, 130], 2, 1, 128, "bf16", 64,
                                sink_blocks=1, k_min=2, rho0=0.5, tau=2.0, seed=35),
    "f32-b64-d64": syn.custom([1024, 100], 2, 1, 64, "f32", 64, rope_theta=None,
                              sink_blocks=1, k_min=2, rho0=1.0, tau=4.0, seed=37),
    "f32-b128-d128": syn.custom([700, 129, 3], 2, 2, 128, "f32", 128,
                                sink_blocks=2, k_min=1, rho0=0.0, tau=1.0, seed=38),
    "single-head-1k-fp32": syn.WORKLOADS["single-head-1k-fp32"],
}

CASES = [("b64-d128-varlen", 1), ("b64-d128-varlen", 4), ("b64-d128-varlen", 64),
         ("b128-d128-gqa4", 2), ("b128-d128-gqa4", 16), ("b128-d128-gqa4", 128),
         ("b64-d64-gqa7", 8), ("b64-d64-gqa7", 32),
         ("b128-d64-short", 4), ("b128-d64-short", 64),
         ("b64-d128-tiny", 8), ("b64-d128-tiny", 16),
         ("f32-b64-d64", 4), ("f32-b64-d64", 16), ("f32-b128-d128", 1), ("f32-b128-d128", 32),
         ("single-head-1k-fp32", 16)]


def _check(w, stride, n_attn_rows=24):
    H.log(f"case antidiag {w.name} stride {stride} metric {w.metric}")
    r = H.DeviceRun(w, score_stride=stride)
    wv = O.pool_vnorm(r.x.v, w.cu_seqlens, w.block)
    ref = O.score_antidiag(r.x.q, r.x.k, wv, w.cu_seqlens, w.block, stride, w.metric, w.beta)
    fin = np.isfinite(ref)
    # -inf (additive form, rows without samples) must match exactly
    assert np.array_equal(np.isfinite(r.scores), fin), "non-finite pattern differs"
    assert np.all(r.scores[~fin] == ref[~fin])
    err, rel = H.check_scores(r.scores[fin], ref[fin], w.dtype, f"antidiag {w.name}/{stride}",
                              w.metric)
    H.select_rows_crossfed(r, H.all_rows(r))
    worst, lw = H.attn_rows_crossfed(r, H.sample_rows(r, n_attn_rows, seed=stride))
    H.log(f"  scores max err {err:.3g} (rel {rel:.3g}); attention {worst:.3g}, lse {lw:.3g}")
    return r


@pytest.mark.parametrize("name,stride", CASES)
def test_antidiag_every_row(name, stride):
    _cuda()
    _check(W[name], stride)


@pytest.mark.parametrize("metric", ["additive", "routing"])
def test_antidiag_metric_forms(metric):
    _cuda()
    _check(W["b64-d128-varlen"].replace(metric=metric, beta=pages_parameters()["beta"]), 8)


def test_antidiag_rows_without_samples():
    # sequences of 1 and 3 tokens at stride 16 hold no causal anti-diagonal
    # pair: their metric rows are 0 and selection still keeps the diagonal
    _cuda()
    w = syn.custom([1, 3, 200], 2, 1, 128, "bf16", 64, sink_blocks=1, k_min=1, rho0=0.5,
                   tau=2.0, seed=36)
    r = _check(w, 16)
    assert np.all(r.scores[:, :2] == 0.0)
    assert np.all(r.idx[:, 0, 0] == 0) and np.all(r.idx[:, 1, 0] == 0)


def test_antidiag_many_sequences():
    # 150 short sequences of mixed lengths (empty, shorter than a group,
    # ragged) in one launch: every kernel walks the sequence table
    _cuda()
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(0, 300, size=150)]
    lens[:4] = [0, 1, 7, 64]
    w = syn.custom(lens, 4, 2, 64, "bf16", 64, sink_blocks=1, k_min=2, rho0=0.5, tau=3.0,
                   seed=42).replace(name="many-sequences")
    for stride in (4, 32):
        _check(w, stride, n_attn_rows=32)


def test_antidiag_rejects_bad_arguments():
    import torch
    _cuda()
    w = W["b64-d64-gqa7"]
    plan = stem.plan_for(w).to("cuda")
    i = plan.info
    q = torch.zeros((i.total_tokens, i.num_q_heads, i.head_dim), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((i.total_tokens, i.num_kv_heads, i.head_dim), dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros((i.num_kv_heads, i.total_blocks), dtype=torch.float32, device="cuda")
    sc = torch.zeros((i.num_q_heads, i.score_elems_per_head), dtype=torch.float32, device="cuda")
    for bad in (0, 3, 12, 128, -4):
        with pytest.raises(stem.StemError) as e:
            stem.stem_score_antidiag(plan, q, k, vn, bad, sc)
        assert e.value.status == stem.STEM_EINVAL


def _full_size_rows(w, stride, n_rows, seed):
    H.log(f"case antidiag full-size {w.name} stride {stride}: generating inputs")
    r = H.DeviceRun(w, out_dtype="bf16", score_stride=stride)
    H.log("  GPU done; metric rows (sampled)")
    wv = O.pool_vnorm(r.x.v, w.cu_seqlens, w.block)
    offs, _ = O.score_offsets(r.cu_blocks)
    seq_of = np.repeat(np.arange(len(r.cu_blocks) - 1), np.diff(r.cu_blocks))
    G = w.num_q_heads // w.num_kv_heads
    for (h, b) in H.sample_rows(r, n_rows, seed=seed):
        s = int(seq_of[b]); i = b - int(r.cu_blocks[s])
        b0 = int(r.cu_blocks[s])
        t = O.antidiag_row_logits(r.x.q, r.x.k, w.cu_seqlens, w.block, stride, h, s, i)
        ref = O.metric_from_logits(t, wv[h // G, b0:b0 + i + 1], w.metric, w.beta)
        got = r.scores[h, int(offs[s]) + O.tri(i):][:i + 1]
        H.check_scores(got, ref, w.dtype, f"antidiag scores {(h, b)}", w.metric)
    H.log("  selection rows (all)")
    H.select_rows_crossfed(r, H.all_rows(r))
    H.log("  attention rows (sampled)")
    worst, lw = H.attn_rows_crossfed(r, H.sample_rows(r, 32, seed=seed + 1))
    H.log(f"  attention max err {worst:.3g}, lse {lw:.3g}")


@pytest.mark.timeout(900)
def test_antidiag_full_size_varlen():
    """The packed batch of four sequences (8K, 16K, 32K, 64K tokens, B = 64) at
    stride 8: many sequences in one launch, each with its own tiles."""
    _cuda()
    _full_size_rows(syn.WORKLOADS["llama3-8b-varlen-120k-b64"], 8, 24, seed=7)


@pytest.mark.timeout(900)
def test_antidiag_full_size_128k():
    """The 128K Llama-3-8B-shaped layer (32/8 heads, d = 128, B = 128) at
    stride 16: sampled metric rows against the oracle, every selection row on
    the GPU's metric, sampled attention rows on the GPU's lists."""
    _cuda()
    w = syn.WORKLOADS["llama3-8b-128k-b128"]
    stride = 16
    H.log(f"case antidiag full-size {w.name} stride {stride}: generating inputs")
    r = H.DeviceRun(w, out_dtype="bf16", score_stride=stride)
    H.log("  GPU done; metric rows (sampled)")
    wv = O.pool_vnorm(r.x.v, w.cu_seqlens, w.block)
    offs, _ = O.score_offsets(r.cu_blocks)
    G = w.num_q_heads // w.num_kv_heads
    for (h, b) in H.sample_rows(r, 20, seed=5):
        t = O.antidiag_row_logits(r.x.q, r.x.k, w.cu_seqlens, w.block, stride, h, 0, b)
        ref = O.metric_from_logits(t, wv[h // G, :b + 1], w.metric, w.beta)
        got = r.scores[h, int(offs[0]) + O.tri(b):][:b + 1]
        H.check_scores(got, ref, w.dtype, f"antidiag scores {(h, b)}", w.metric)
    H.log("  selection rows (all)")
    H.select_rows_crossfed(r, H.all_rows(r))
    H.log("  attention rows (sampled)")
    worst, lw = H.attn_rows_crossfed(r, H.sample_rows(r, 48, seed=6))
    H.log(f"  attention max err {worst:.3g}, lse {lw:.3g}")

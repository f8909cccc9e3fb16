"""GPU parity of the HIP path (called through the C ABI) against the oracle.

Small workloads are checked element by element over every row; they still
span several 32-row score tiles, several key blocks per row, ragged final
blocks, empty sequences and every kernel variant (bf16 / f32 inputs,
B = 64 / 128, d = 64 / 128, f32 / bf16 outputs).  The full-size workloads
run in the benchmark's launch configuration and are checked on every pooled
value and every selection row, and on sampled attention rows.
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


SMALL = {
    "bf16-b64-d128-varlen-ragged": syn.custom([1000, 77, 0, 2050], 8, 2, 128, "bf16", 64,
                                              sink_blocks=2, k_min=3, rho0=0.5, tau=8.0, seed=11),
    "bf16-b128-d128-gqa4": syn.custom([4100, 300], 4, 1, 128, "bf16", 128,
                                      sink_blocks=1, k_min=4, rho0=0.4, tau=6.0, seed=12),
    "bf16-b64-d64-gqa7": syn.custom([1500], 7, 1, 64, "bf16", 64,
                                    sink_blocks=3, k_min=2, rho0=1.0, tau=4.0, seed=13),
    "bf16-b128-d64": syn.custom([1337, 1], 2, 2, 64, "bf16", 128,
                                sink_blocks=0, k_min=1, rho0=0.2, tau=3.0, seed=14),
    "f32-b64-d64": syn.custom([1024, 100], 2, 1, 64, "f32", 64, rope_theta=None,
                              sink_blocks=1, k_min=2, rho0=1.0, tau=4.0, seed=15),
    "f32-b128-d128": syn.custom([700, 129], 2, 2, 128, "f32", 128,
                                sink_blocks=2, k_min=1, rho0=0.0, tau=1.0, seed=16),
    "f32-b64-d128": syn.custom([555], 4, 2, 128, "f32", 64,
                               sink_blocks=1, k_min=3, rho0=0.7, tau=5.0, seed=17),
    "f32-b128-d64": syn.custom([640], 2, 1, 64, "f32", 128,
                               sink_blocks=1, k_min=1, rho0=0.5, tau=2.0, seed=18),
}


def _full_check(r: H.DeviceRun):
    w = r.w
    ref = O.prefill(r.x.q, r.x.k, r.x.v, w.cu_seqlens, w.block, w.sink_blocks, w.k_min,
                    w.rho0, w.tau, metric=w.metric, beta=w.beta, budget_mode=w.budget_mode,
                    k_start=w.k_start, mu=w.mu)
    np.testing.assert_array_equal(r.budget, ref["budget"])
    t = H.TOL[w.dtype]
    # stage 1: pooled values
    np.testing.assert_allclose(r.qbar, ref["qbar"], rtol=t["pool"], atol=t["pool"])
    np.testing.assert_allclose(r.kbar, ref["kbar"], rtol=t["pool"], atol=t["pool"])
    np.testing.assert_allclose(r.vnorm, ref["w"], rtol=t["pool"], atol=t["pool"])
    # metric
    H.check_scores(r.scores, ref["m"], w.dtype, "scores", w.metric)
    # selection, on the GPU's own scores: bit-exact
    H.select_rows_crossfed(r, H.all_rows(r))
    # attention with the GPU's lists: every row
    o, lse = O.sparse_attn(r.x.q, r.x.k, r.x.v, r.idx, r.count, w.cu_seqlens, w.block)
    err = H.check_out(r.out, o, w.dtype, r.out_dtype, "attention")
    assert np.abs(r.lse - lse).max() <= t["lse"]
    # end to end: where the oracle's own selection differs, the swapped
    # blocks must be near-ties of the oracle metric
    differ = np.argwhere(np.any(ref["idx"] != r.idx, axis=2))
    offs, _ = O.score_offsets(r.cu_blocks)
    seq_of = np.repeat(np.arange(len(r.cu_blocks) - 1), np.diff(r.cu_blocks))
    for h, b in differ:
        s = int(seq_of[b]); i = b - int(r.cu_blocks[s])
        m = ref["m"][h, int(offs[s]) + O.tri(i):][:i + 1]
        a = set(r.idx[h, b]) - set(ref["idx"][h, b])
        c = set(ref["idx"][h, b]) - set(r.idx[h, b])
        for x in a:
            for y in c:
                assert abs(m[x] - m[y]) <= 2 * t["score"], (h, b, x, y)
    H.log(f"{w.name}: attention max err {err:.3g}, rows with a near-tie swap {len(differ)}")


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workload_every_stage(name):
    _cuda()
    H.log(f"case {name}")
    _full_check(H.DeviceRun(SMALL[name]))


@pytest.mark.parametrize("name", ["bf16-b64-d128-varlen-ragged", "bf16-b128-d128-gqa4"])
def test_bf16_output_mode(name):
    _cuda()
    H.log(f"case {name} bf16 out")
    r = H.DeviceRun(SMALL[name], out_dtype="bf16")
    rows = H.all_rows(r)
    H.attn_rows_crossfed(r, rows, "bf16-out")


# The pages' other forms of the two rules: the additive metric
# s + beta*max(0, log w^2), routing alone (w ignored), and the linear budget
# from k_start to mu*k_start.
MODES = {
    "bf16-b64-d128-additive": syn.custom([1000, 77, 0, 2050], 8, 2, 128, "bf16", 64,
                                         sink_blocks=2, k_min=3, rho0=0.5, tau=8.0, seed=41,
                                         metric="additive", beta=0.5),
    "bf16-b128-d64-routing": syn.custom([1337, 1], 4, 2, 64, "bf16", 128, sink_blocks=1,
                                        k_min=1, rho0=0.4, tau=3.0, seed=42, metric="routing"),
    "bf16-b128-d128-linear": syn.custom([4100, 300], 4, 1, 128, "bf16", 128, sink_blocks=1,
                                        k_min=2, seed=43, budget_mode="linear", k_start=12.0,
                                        mu=0.25),
    "f32-b64-d128-additive-linear": syn.custom([555, 900], 4, 2, 128, "f32", 64,
                                               sink_blocks=1, k_min=1, seed=44,
                                               budget_mode="linear", k_start=6.5, mu=0.5,
                                               metric="additive", beta=1.5),
    "f32-b128-d64-routing": syn.custom([640], 2, 1, 64, "f32", 128, rope_theta=None,
                                       sink_blocks=0, k_min=1, rho0=0.5, tau=2.0, seed=45,
                                       metric="routing"),
}


@pytest.mark.parametrize("name", list(MODES))
def test_metric_and_budget_modes_every_stage(name):
    _cuda()
    H.log(f"case mode {name}")
    _full_check(H.DeviceRun(MODES[name]))


def test_single_head_1k_fp32_workload():
    _cuda()
    w = syn.WORKLOADS["single-head-1k-fp32"]
    H.log("case single-head-1k-fp32")
    _full_check(H.DeviceRun(w))


def test_vnorm_max_mode():
    _cuda()
    w = SMALL["bf16-b64-d128-varlen-ragged"]
    r = H.DeviceRun(w, vnorm_mode=stem.STEM_VNORM_MAX)
    np.testing.assert_allclose(r.vnorm, O.pool_vnorm(r.x.v, w.cu_seqlens, w.block, "max"),
                               rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype,B,d", [("bf16", 64, 128), ("bf16", 128, 128), ("f32", 64, 64)])
def test_full_budget_equals_dense_causal(dtype, B, d):
    """With every causal block kept, the path is dense causal attention."""
    _cuda()
    w = syn.custom([700, 1200], 4, 2, d, dtype, B, sink_blocks=1, k_min=10 ** 6, rho0=0.0,
                   tau=1.0, seed=21)
    r = H.DeviceRun(w)
    assert np.all(r.count == np.concatenate([np.arange(1, n + 1) for n in np.diff(r.cu_blocks)]))
    o, lse = O.dense_causal_attn(r.x.q, r.x.k, r.x.v, w.cu_seqlens)
    H.check_out(r.out, o, dtype, "f32", "dense")
    assert np.abs(r.lse - lse).max() <= H.TOL[dtype]["lse"]


def test_many_short_sequences():
    """150 sequences of 0 to 299 tokens packed in one launch (every stage
    walks the sequence table), checked on every row."""
    _cuda()
    rng = np.random.default_rng(43)
    lens = [int(x) for x in rng.integers(0, 300, size=150)]
    lens[:4] = [0, 1, 65, 128]
    w = syn.custom(lens, 4, 2, 128, "bf16", 64, sink_blocks=2, k_min=1, rho0=0.7, tau=2.0,
                   seed=44).replace(name="many-sequences")
    H.log("case many short sequences")
    _full_check(H.DeviceRun(w))


def test_edge_shapes():
    """Tiny and degenerate sequences: length 1, shorter than a block, exactly
    one block, empty; no sinks; zero k_min; zero decay."""
    _cuda()
    for seqlens, S, kmin, rho0 in [([1], 0, 0, 0.0), ([63, 64, 65, 0, 1], 1, 0, 0.0),
                                   ([5000], 0, 0, 0.0), ([129, 2, 300], 4, 1, 3.0)]:
        w = syn.custom(seqlens, 4, 2, 128, "bf16", 64, sink_blocks=S, k_min=kmin, rho0=rho0,
                       tau=2.0, seed=31)
        H.log(f"case edge {seqlens} S={S} k_min={kmin}")
        _full_check(H.DeviceRun(w))


def test_equal_scores_pick_smallest_blocks():
    """Constant K and V make every metric in a row equal: the kept blocks
    must be the smallest block numbers (ties go to the earlier block)."""
    _cuda()
    w = syn.custom([64 * 40], 2, 1, 128, "bf16", 64, sink_blocks=2, k_min=5, rho0=0.0, tau=1.0)
    x = syn.generate(w)
    one = syn.bf16_bits(np.ones(1, np.float32))[0]
    x.k_bits[:] = one; x.v_bits[:] = one
    x.k[:] = 1.0; x.v[:] = 1.0
    r = H.DeviceRun(w, x=x)
    for h in range(2):
        for i in range(40):
            # k_i = min(i + 1, 2 + 1 + 5): the 5 free slots go to blocks 2..6
            want = list(range(i + 1)) if i < 8 else list(range(7)) + [i]
            assert list(r.idx[h, i, :r.count[h, i]]) == want, (h, i)
    H.select_rows_crossfed(r, H.all_rows(r))


def test_select_long_budget_and_wide_ties():
    """Both selection strategies: budgets of more than 64 free slots (every
    key takes part in the threshold search), and rows whose metrics are all
    equal with more than 64 candidates tied at the threshold."""
    _cuda()
    w = syn.custom([64 * 300], 2, 1, 128, "bf16", 64, sink_blocks=2, k_min=100, rho0=0.0,
                   tau=1.0, seed=51)
    H.log("case select k_min=100")
    _full_check(H.DeviceRun(w))
    w = syn.custom([64 * 200], 2, 1, 128, "bf16", 64, sink_blocks=2, k_min=5, rho0=0.0, tau=1.0)
    x = syn.generate(w)
    one = syn.bf16_bits(np.ones(1, np.float32))[0]
    x.k_bits[:] = one; x.v_bits[:] = one
    x.k[:] = 1.0; x.v[:] = 1.0
    H.log("case select 200 tied blocks")
    r = H.DeviceRun(w, x=x)
    for h in range(2):
        for i in range(200):
            want = list(range(i + 1)) if i < 8 else list(range(7)) + [i]
            assert list(r.idx[h, i, :r.count[h, i]]) == want, (h, i)
    H.select_rows_crossfed(r, H.all_rows(r))


# ----------------------------------------------------------------- full size


def _full_size(name, n_attn_rows: int, **params):
    w = (syn.WORKLOADS[name] if isinstance(name, str) else name).replace(**params)
    name = w.name
    H.log(f"case full-size {name}: generating inputs")
    r = H.DeviceRun(w, out_dtype="bf16")
    H.log(f"case full-size {name}: GPU done, checking pooled values")
    t = H.TOL[w.dtype]
    np.testing.assert_allclose(r.qbar, O.pool_mean(r.x.q, w.cu_seqlens, w.block),
                               rtol=t["pool"], atol=t["pool"])
    np.testing.assert_allclose(r.kbar, O.pool_mean(r.x.k, w.cu_seqlens, w.block),
                               rtol=t["pool"], atol=t["pool"])
    wref = O.pool_vnorm(r.x.v, w.cu_seqlens, w.block)
    np.testing.assert_allclose(r.vnorm, wref, rtol=t["pool"], atol=t["pool"])
    H.log(f"case full-size {name}: selection rows (all)")
    H.select_rows_crossfed(r, H.all_rows(r))
    assert np.array_equal(r.count.sum(axis=1), np.full(w.num_q_heads, r.budget.sum()))
    np.testing.assert_array_equal(
        r.budget, O.budgets_for(r.cu_blocks, w.sink_blocks, w.k_min, w.rho0, w.tau,
                                w.budget_mode, w.k_start, w.mu))
    H.log(f"case full-size {name}: metric rows (sampled)")
    qbar = O.pool_mean(r.x.q, w.cu_seqlens, w.block)
    kbar = O.pool_mean(r.x.k, w.cu_seqlens, w.block)
    offs, _ = O.score_offsets(r.cu_blocks)
    seq_of = np.repeat(np.arange(len(r.cu_blocks) - 1), np.diff(r.cu_blocks))
    for (h, b) in H.sample_rows(r, 256, seed=1):
        s = int(seq_of[b]); i = b - int(r.cu_blocks[s])
        ref = O.score_row_values(qbar, kbar, wref, r.cu_blocks, w.head_dim, h, s, i,
                                 w.metric, w.beta)
        got = r.scores[h, int(offs[s]) + O.tri(i):][:i + 1]
        H.check_scores(got, ref, w.dtype, f"scores {(h, b)}", w.metric)
    H.log(f"case full-size {name}: attention rows (sampled)")
    worst, lw = H.attn_rows_crossfed(r, H.sample_rows(r, n_attn_rows, seed=2))
    H.log(f"case full-size {name}: attention max err {worst:.3g}, lse {lw:.3g}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama3-8b-32k-b64", "llama3-8b-128k-b128",
                                  "qwen2.5-7b-64k-b64", "llama3-8b-varlen-120k-b64"])
def test_full_size_workload(name):
    _cuda()
    _full_size(name, 96)


@pytest.mark.timeout(900)
def test_full_size_additive_metric_linear_budget():
    """The 32K layer with the pages' additive metric and linear budget, at the
    ablation's best values beta = 0.2 and mu = 0.7."""
    _cuda()
    pp = pages_parameters()
    _full_size("llama3-8b-32k-b64", 64, metric="additive", beta=pp["beta"], budget_mode="linear",
               k_start=24.0, mu=pp["mu"])


@pytest.mark.timeout(900)
def test_maximum_sequence_length():
    """The longest sequence the library accepts (4096 blocks of 64 tokens):
    the selection then holds 4094 candidates per row (64 per lane), and the
    metric has 128 key tiles per row tile."""
    _cuda()
    w = syn.custom([64 * 4096], 2, 1, 64, "bf16", 64, sink_blocks=2, k_min=8, rho0=0.5,
                   tau=64.0, seed=61).replace(name="max-seq-4096-blocks")
    _full_size(w, 48)

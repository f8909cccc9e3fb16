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
    # KV-head counts for each way the attention grid places work on the 8
    # XCDs: 4 KV heads (each shared by two XCDs, 3 query heads per group),
    # 3 (contiguous ranges) and 16 (two KV heads per XCD)
    "bf16-b64-d128-hkv4-g3": syn.custom([900, 2000, 333], 12, 4, 128, "bf16", 64,
                                        sink_blocks=2, k_min=3, rho0=0.5, tau=8.0, seed=19),
    "bf16-b128-d64-hkv3-g2": syn.custom([1500, 700], 6, 3, 64, "bf16", 128,
                                        sink_blocks=1, k_min=2, rho0=0.5, tau=4.0, seed=20),
    "bf16-b64-d64-hkv16": syn.custom([700, 64], 16, 16, 64, "bf16", 64,
                                     sink_blocks=1, k_min=2, rho0=0.6, tau=4.0, seed=21),
    # B = 64, d = 64 with two query heads per KV head: the head-pair kernel
    "bf16-b64-d64-pairs": syn.custom([1500, 333, 64], 4, 2, 64, "bf16", 64,
                                     sink_blocks=2, k_min=3, rho0=0.5, tau=6.0, seed=22),
    # uniform budgets of 2 sinks + 1 diagonal + k_min: lists of 32 blocks (the
    # longest the head-pair kernel takes) and of 33 (single-head workgroups)
    "bf16-b64-d128-lists32": syn.custom([64 * 45, 500], 4, 2, 128, "bf16", 64,
                                        sink_blocks=2, k_min=29, rho0=0.0, tau=1.0, seed=23),
    "bf16-b64-d128-lists33": syn.custom([64 * 45, 500], 4, 2, 128, "bf16", 64,
                                        sink_blocks=2, k_min=30, rho0=0.0, tau=1.0, seed=24),
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
    ndiff = H.selection_agreement(r, ref["idx"], ref["m"], range(w.num_q_heads), w.name)
    H.log(f"{w.name}: attention max err {err:.3g}, rows with a near-tie swap {ndiff}")


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
    # k_start as a fraction of each row's causal blocks, the pages' mu
    "bf16-b64-d128-linear-fraction": syn.custom([1000, 77, 0, 2050], 8, 2, 128, "bf16", 64,
                                                sink_blocks=2, k_min=1, seed=46,
                                                budget_mode="linear_fraction", k_start=0.4,
                                                mu=pages_parameters()["mu"]),
    "bf16-b128-d128-additive-pages-beta": syn.custom([4100, 300], 4, 1, 128, "bf16", 128,
                                                     sink_blocks=1, k_min=3, rho0=0.4, tau=6.0,
                                                     seed=47, metric="additive"),
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


def _special_scores(n: int, rng: np.random.Generator) -> np.ndarray:
    """Metric values with every class the selection orders specially: NaN
    (ranks last), -0 and +0 (equal), +-inf, negatives, denormals and runs of
    equal values, mixed with ordinary values."""
    pool = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, -2.5, -1e-30, 1e-42, 0.25, 0.25, 3.0,
                     1.0, 1.0, 7.5, 1e30], dtype=np.float32)
    m = rng.standard_normal(n).astype(np.float32)
    pick = rng.random(n) < 0.6
    m[pick] = pool[rng.integers(0, pool.size, int(pick.sum()))]
    return m


@pytest.mark.parametrize("k_min,block", [(5, 64), (40, 64), (100, 64), (3, 128)])
def test_select_special_metric_values(k_min, block):
    """stem_select on metric rows holding NaN, signed zeros, infinities,
    negatives and wide ties (written straight into the metric buffer): the
    kept lists must equal the oracle's selection on the same values, every
    row, both selection strategies (budgets up to and above 64 free slots)."""
    _cuda()
    import torch
    cu = [0, block * 300, block * 300 + 17, block * 300 + 17 + block * 70 + 5]
    Hq = 2
    H.log(f"case select special values k_min={k_min} B={block}")
    plan = stem.stem_plan(cu, Hq, 1, 128, block, "bf16", 2, k_min, 0.5, 8.0).to("cuda")
    i = plan.info
    rng = np.random.default_rng(1000 + k_min + block)
    m = np.stack([_special_scores(int(i.score_elems_per_head), rng) for _ in range(Hq)])
    scores = torch.from_numpy(m).to("cuda")
    idx = torch.full((Hq, i.total_blocks, i.kmax), -7, dtype=torch.int32, device="cuda")
    count = torch.full((Hq, i.total_blocks), -7, dtype=torch.int32, device="cuda")
    stem.stem_select(plan, scores, idx, count)
    torch.cuda.synchronize()
    idx, count = idx.cpu().numpy(), count.cpu().numpy()
    cub = O.block_layout(cu, block)
    bud = O.budgets_for(cub, 2, k_min, 0.5, 8.0)
    offs, _ = O.score_offsets(cub)
    for h in range(Hq):
        for s in range(len(cub) - 1):
            for r in range(int(cub[s + 1] - cub[s])):
                b = int(cub[s]) + r
                row0 = int(offs[s]) + O.tri(r)
                want = O.select_row(m[h, row0:row0 + r + 1].astype(np.float64), r, int(bud[b]), 2)
                n = int(count[h, b])
                assert n == want.size, (h, b, n, want.size)
                assert np.array_equal(idx[h, b, :n], want), (h, b, idx[h, b, :n], want)
                assert np.all(idx[h, b, n:] == -1), (h, b)


def _moving_max_inputs(w, slope: float, gain: float, seed: int):
    """Q and K sharing one direction (dimension 0) along which a key's logit
    (after the 1/sqrt(d) scale) grows by ``slope`` per token position in its
    sequence (falls, for a negative slope), over noise scaled by ``gain``:
    the running maximum of a row moves at every stage (slope > 0), sits on
    the first keys while later weights underflow (slope < 0), or jumps about
    (slope 0, large gain).  V is scaled by 1/8 (exactly): with a few keys
    carrying each row, the output is close to single rows of V, and the bf16
    rounding of the weights (relative 2^-9) then costs a part of |v| that the
    absolute bar should not see."""
    x = syn.generate(w, seed=seed)
    q, k = x.q * gain, x.k * gain
    if w.dtype == "bf16":
        x.v_bits = syn.bf16_bits(x.v * np.float32(0.125))
        x.v = syn.bf16_bits_to_f32(x.v_bits)
    else:
        x.v = x.v * np.float32(0.125)
    cu = w.cu_seqlens
    beta = 4.0
    alpha = slope * np.sqrt(w.head_dim) / beta
    for si in range(len(cu) - 1):
        t = np.arange(cu[si + 1] - cu[si], dtype=np.float32)
        k[cu[si]:cu[si + 1], :, 0] = alpha * t[:, None]
        q[cu[si]:cu[si + 1], :, 0] = beta
    if w.dtype == "bf16":
        x.q_bits, x.k_bits = syn.bf16_bits(q), syn.bf16_bits(k)
        x.q, x.k = syn.bf16_bits_to_f32(x.q_bits), syn.bf16_bits_to_f32(x.k_bits)
    else:
        x.q, x.k = q, k
    return x


MOVING_MAX = {
    # head pairs (lists of at most 32 blocks), single-head B = 64 (longer
    # lists) and B = 128; bf16 inputs (with f32 inputs logits this large
    # leave the 1e-5 bars below f32's own resolution)
    "bf16-b64-pairs": syn.custom([64 * 20 + 13, 64 * 3], 4, 2, 128, "bf16", 64, sink_blocks=2,
                                 k_min=6, rho0=0.5, tau=8.0, seed=61),
    "bf16-b64-long": syn.custom([64 * 50 + 7], 2, 1, 128, "bf16", 64, sink_blocks=2,
                                k_min=40, rho0=0.5, tau=8.0, seed=62),
    "bf16-b128": syn.custom([128 * 12 + 77, 300], 4, 1, 128, "bf16", 128, sink_blocks=1,
                            k_min=4, rho0=0.5, tau=8.0, seed=63),
}


@pytest.mark.parametrize("slope,gain", [(0.5, 1.0), (-0.5, 1.0), (0.0, 6.0)])
@pytest.mark.parametrize("name", list(MOVING_MAX))
def test_attention_moving_maximum(name, slope, gain):
    """The attention kernel's online softmax where a row's maximum logit
    moves at every stage (reference raised each time), stays on the first
    keys (later weights underflow), or jumps by tens of units, with logits
    far beyond the f32 range of exp (up to ~650): every row against the
    oracle, on block lists drawn by the oracle's selection from a random
    metric (the attention sees only the lists)."""
    _cuda()
    import torch
    w = MOVING_MAX[name]
    H.log(f"case moving maximum {name} slope={slope} gain={gain}")
    x = _moving_max_inputs(w, slope, gain, seed=w.seed + 7)
    plan = stem.plan_for(w).to("cuda")
    i = plan.info
    cub = O.block_layout(w.cu_seqlens, w.block)
    bud = O.budgets_for(cub, w.sink_blocks, w.k_min, w.rho0, w.tau)
    rng = np.random.default_rng(w.seed)
    m = rng.random((w.num_q_heads, int(i.score_elems_per_head)))
    idx, cnt = O.select(m, cub, bud, w.sink_blocks, kmax=int(i.kmax))
    q, k, v = H.upload(x)
    out = torch.empty((i.total_tokens, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.num_q_heads, i.total_tokens), dtype=torch.float32, device="cuda")
    stem.stem_sparse_attn(plan, q, k, v, torch.from_numpy(idx).to("cuda"),
                          torch.from_numpy(cnt).to("cuda"), out, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.sparse_attn(x.q, x.k, x.v, idx, cnt, w.cu_seqlens, w.block)
    err = H.check_out(out.cpu().numpy(), o_ref, w.dtype, "f32", f"moving maximum {name}")
    got_lse = lse.cpu().numpy()
    H.log(f"  output max err {err:.3g}, LSE max err {np.abs(got_lse - lse_ref).max():.3g} "
          f"(LSE up to {np.abs(lse_ref).max():.0f})")
    assert np.isfinite(got_lse).all()
    # The row sum is taken over the bf16-rounded weights (the ones that
    # multiply V), each within 2^-8 of its f32 value; when one key carries a
    # row and its weight against the lazily moved reference is not a power of
    # two, the sum, and so the LSE, keeps up to ln(1 + 2^-8) of that rounding
    # (on ordinary rows many weights share it and the error is ~1e-6).  f32
    # logits of magnitude up to ~2e3 add well under 1e-4.
    lse_bar = float(np.log1p(2.0 ** -8)) + 1e-4
    assert np.abs(got_lse - lse_ref).max() <= lse_bar


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
    _whole_group(r)


def _whole_group(r: H.DeviceRun):
    """Every row of KV head 0 and its G query heads: the oracle's own path
    (its fp64 metric, its own selection) against the GPU's metric, and its
    attention on the GPU's block lists against the GPU's output; rows where
    the two selections differ may only swap near-tied blocks."""
    w = r.w
    G = w.num_q_heads // w.num_kv_heads
    q, k, v = r.x.q[:, :G], r.x.k[:, :1], r.x.v[:, :1]
    H.log(f"case full-size {w.name}: oracle path over KV group 0 ({G} query heads)")
    ref = O.prefill(q, k, v, w.cu_seqlens, w.block, w.sink_blocks, w.k_min, w.rho0, w.tau,
                    metric=w.metric, beta=w.beta, budget_mode=w.budget_mode,
                    k_start=w.k_start, mu=w.mu)
    np.testing.assert_array_equal(ref["budget"], r.budget)
    H.check_scores(r.scores[:G], ref["m"], w.dtype, "group-0 scores", w.metric)
    o, lse = O.sparse_attn(q, k, v, r.idx[:G], r.count[:G], w.cu_seqlens, w.block)
    err = H.check_out(r.out[:, :G], o, w.dtype, r.out_dtype, "group-0 attention")
    assert np.abs(r.lse[:G] - lse).max() <= H.TOL[w.dtype]["lse"]
    ndiff = H.selection_agreement(r, ref["idx"], ref["m"], range(G), w.name)
    rows = G * int(r.cu_blocks[-1])
    H.log(f"case full-size {w.name}: group 0, {rows} rows: attention max err {err:.3g}; "
          f"oracle's own selection differs in {ndiff} rows, each by near-tied blocks only")


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


def _random_case(seed: int):
    """A seeded random small bf16 workload: head shape, block size, sequence
    lengths (with partial and very short sequences), budget and metric."""
    rng = np.random.default_rng(1000 + seed)
    hkv = int(rng.choice([1, 2, 3, 4]))
    g = int(rng.integers(1, 6))
    B = int(rng.choice([64, 128]))
    d = int(rng.choice([64, 128]))
    nseq = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.integers(1, 40 * B, size=nseq)]
    metric = str(rng.choice(["output_aware", "additive", "routing"]))
    kw = dict(sink_blocks=int(rng.integers(0, 4)), k_min=int(rng.integers(1, 40)),
              rho0=float(rng.uniform(0.0, 1.0)), tau=float(rng.uniform(1.0, 16.0)),
              seed=200 + seed, metric=metric)
    return syn.custom(lens, g * hkv, hkv, d, "bf16", B, **kw)


@pytest.mark.parametrize("seed", range(20))
def test_random_small_workloads_every_stage(seed):
    _cuda()
    w = _random_case(seed)
    H.log(f"case random {seed}: lens {w.seqlens} heads {w.num_q_heads}/{w.num_kv_heads} "
          f"d {w.head_dim} B {w.block} metric {w.metric}")
    _full_check(H.DeviceRun(w))

"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the oracle.  Tolerances (absolute, max over elements):

  * bf16 inputs: 2e-2 on scores and on the f32 attention output; the bf16
    output is allowed 2e-2 plus half a bf16 ulp of the reference value
    (rounding the output to bf16 alone costs up to half an ulp, which
    exceeds 2e-2 once |o| >= 8).  Scores must also match to 1e-4 relative:
    both paths read identical bf16 values and differ only in summation order
    and f32 vs f64 arithmetic.
  * f32 inputs: 1e-5 on scores and outputs.
  * block selection: bit-exact when both sides rank the same score array.
"""
from __future__ import annotations

import math

import numpy as np

from block_sparse_causal_amd import stem
from block_sparse_causal_amd import synthetic as syn
from oracle import stem_oracle as O

TOL = {"bf16": dict(score=2e-2, score_rel=1e-4, out=2e-2, lse=2e-3, pool=2e-5),
       "f32": dict(score=1e-5, score_rel=1e-5, out=1e-5, lse=1e-5, pool=1e-5)}


def log(msg: str) -> None:
    print(msg, flush=True)


def upload(x: syn.Inputs, device="cuda"):
    import torch
    if x.workload.dtype == "bf16":
        conv = lambda b: torch.from_numpy(b.view(np.int16)).to(device).view(torch.bfloat16)
        return conv(x.q_bits), conv(x.k_bits), conv(x.v_bits)
    return tuple(torch.from_numpy(a).to(device) for a in (x.q, x.k, x.v))


class DeviceRun:
    """Plan, upload and run the whole path once; keep host copies."""

    def __init__(self, w: syn.Workload, x: syn.Inputs = None, out_dtype="f32", vnorm_mode=0,
                 plan_override=None, score_stride=None):
        import torch
        self.w = w
        self.x = x if x is not None else syn.generate(w)
        self.plan = stem.plan_for(w, **(plan_override or {})).to("cuda")
        q, k, v = upload(self.x)
        odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        b = stem.prefill(self.plan, q, k, v, out_dtype=odt, vnorm_mode=vnorm_mode,
                         score_stride=score_stride)
        self.score_stride = score_stride
        torch.cuda.synchronize()
        self.qbar = b.qbar.cpu().numpy()
        self.kbar = b.kbar.cpu().numpy()
        self.vnorm = b.vnorm.cpu().numpy()
        self.scores = b.scores.cpu().numpy()
        self.idx = b.idx.cpu().numpy()
        self.count = b.count.cpu().numpy()
        self.out = b.out.float().cpu().numpy()
        self.lse = b.lse.cpu().numpy()
        self.out_dtype = out_dtype
        self.cu_blocks = np.asarray(self.plan.cu_blocks, dtype=np.int64)
        self.budget = np.asarray(self.plan.budget, dtype=np.int64)
        del b, q, k, v


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return np.exp2(e - 8)  # a bf16 ulp at |x| is 2^(e-7); half of it is 2^(e-8)


def check_out(got: np.ndarray, ref: np.ndarray, dtype: str, out_dtype: str, what: str):
    tol = TOL[dtype]["out"]
    err = np.abs(got - ref)
    if out_dtype == "bf16":
        bound = tol + bf16_half_ulp(ref)
    else:
        bound = np.full_like(ref, tol)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, max err "
                           f"{err.max():.3g} (bound {tol})")
    return float(err.max())


def check_scores(got: np.ndarray, ref: np.ndarray, dtype: str, what: str,
                 metric: str = "output_aware"):
    """Softmax metrics are positive and checked relative to each value; the
    additive metric is a logit that crosses zero, so its relative check uses
    max(|ref|, 1) (an absolute bound below 1)."""
    t = TOL[dtype]
    err = np.abs(got - ref)
    assert err.max() <= t["score"], f"{what}: max abs err {err.max():.3g}"
    floor = 1.0 if metric == "additive" else 1e-30
    rel = err / np.maximum(np.abs(ref), floor)
    assert rel.max() <= t["score_rel"], f"{what}: max rel err {rel.max():.3g}"
    return float(err.max()), float(rel.max())


def near_tie(mx: float, my: float, dtype: str, metric: str = "output_aware") -> bool:
    """Whether two oracle metric values are close enough for the GPU's f32
    scores (each within score_rel of its reference, relative to max(|m|, 1)
    for the additive metric, relative to |m| otherwise) to rank them the
    other way round: |mx - my| <= score_rel * (|mx| + |my|)."""
    rel = TOL[dtype]["score_rel"]
    floor = 1.0 if metric == "additive" else 1e-30
    return abs(mx - my) <= rel * (max(abs(mx), floor) + max(abs(my), floor))


def selection_agreement(r: DeviceRun, ref_idx: np.ndarray, ref_m: np.ndarray, heads,
                        what: str) -> int:
    """End to end: rows where the oracle's own selection (from its fp64
    metric) differs from the GPU's.  In such a row every block the GPU kept
    and the oracle did not, and every block the oracle kept and the GPU did
    not, must be a near-tie of the oracle metric.  Returns the number of
    differing rows."""
    offs, _ = O.score_offsets(r.cu_blocks)
    seq_of = np.repeat(np.arange(len(r.cu_blocks) - 1), np.diff(r.cu_blocks))
    gpu = r.idx[list(heads)]
    differ = np.argwhere(np.any(ref_idx != gpu, axis=2))
    for hh, b in differ:
        s = int(seq_of[b]); i = b - int(r.cu_blocks[s])
        m = ref_m[hh, int(offs[s]) + O.tri(i):][:i + 1]
        a = set(gpu[hh, b]) - set(ref_idx[hh, b])
        c = set(ref_idx[hh, b]) - set(gpu[hh, b])
        assert len(a) == len(c), (what, hh, b)
        for x in a:
            for y in c:
                assert near_tie(m[x], m[y], r.w.dtype, r.w.metric), \
                    (what, int(hh), int(b), int(x), int(y), m[x], m[y])
    return len(differ)


def select_rows_crossfed(r: DeviceRun, rows):
    """Oracle selection on the GPU's own scores must equal the GPU's lists."""
    offs, _ = O.score_offsets(r.cu_blocks)
    seq_of = np.repeat(np.arange(len(r.cu_blocks) - 1), np.diff(r.cu_blocks))
    S = r.w.sink_blocks
    for (h, b) in rows:
        s = int(seq_of[b]); i = b - int(r.cu_blocks[s])
        row0 = int(offs[s]) + O.tri(i)
        m = r.scores[h, row0:row0 + i + 1].astype(np.float64)
        want = O.select_row(m, i, int(r.budget[b]), S)
        n = int(r.count[h, b])
        assert n == want.size, (h, b, n, want.size)
        got = r.idx[h, b, :n]
        assert np.array_equal(got, want), (h, b, got, want)
        assert np.all(r.idx[h, b, n:] == -1), (h, b)


def attn_rows_crossfed(r: DeviceRun, rows, what="attn"):
    """Oracle attention with the GPU's block lists, on sampled rows."""
    res = O.sparse_attn(r.x.q, r.x.k, r.x.v, r.idx, r.count, r.w.cu_seqlens, r.w.block,
                        rows=rows)
    cu = r.w.cu_seqlens
    seq_of = np.repeat(np.arange(len(r.cu_blocks) - 1), np.diff(r.cu_blocks))
    worst = 0.0
    lse_worst = 0.0
    for (h, b), (o, l) in res.items():
        s = int(seq_of[b]); i = b - int(r.cu_blocks[s])
        t0 = int(cu[s]) + i * r.w.block
        t1 = t0 + o.shape[0]
        worst = max(worst, check_out(r.out[t0:t1, h], o, r.w.dtype, r.out_dtype, f"{what} {(h, b)}"))
        le = np.abs(r.lse[h, t0:t1] - l).max()
        assert le <= TOL[r.w.dtype]["lse"], f"{what} lse {(h, b)}: {le}"
        lse_worst = max(lse_worst, float(le))
    return worst, lse_worst


def all_rows(r: DeviceRun):
    return [(h, b) for h in range(r.w.num_q_heads) for b in range(int(r.cu_blocks[-1]))]


def sample_rows(r: DeviceRun, n: int, seed: int = 0):
    """First, last and diagonal-interesting rows plus a random sample."""
    rng = np.random.default_rng(seed)
    nbT = int(r.cu_blocks[-1])
    Hq = r.w.num_q_heads
    rows = set()
    for s in range(len(r.cu_blocks) - 1):
        b0, b1 = int(r.cu_blocks[s]), int(r.cu_blocks[s + 1])
        for b in {b0, b0 + 1, b0 + 2, b1 - 1}:
            if b0 <= b < b1:
                rows.add((int(rng.integers(Hq)), b))
                rows.add((Hq - 1, b))
    while len(rows) < n and len(rows) < Hq * nbT:
        rows.add((int(rng.integers(Hq)), int(rng.integers(nbT))))
    return sorted(rows)

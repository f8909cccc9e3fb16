"""CPU oracle for the Stem block-sparse causal prefill path.  TEST INFRASTRUCTURE.

This module is the plain, slow, obviously-correct definition that the HIP path
is checked against.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import it; the library never calls it and never falls
back to it.  It shares no code with the GPU path.  Everything is NumPy in
float64 (inputs are upcast exactly from the bf16 / fp32 values the GPU reads),
and the loops follow the method's stages in the order the pages give them.

Sources.  All five pages carry the title "Stem: Rethinking Causal Information
Flow in Sparse Attention" (arXiv 2603.06274); they are told apart here by host
and language:
  [es] gist.science, Spanish  - "Resumen tecnico" sections 1, 2.A, 2.B, "Implementacion"
  [it] gist.science, Italian  - "Sommario tecnico" sections 2.A, 2.B, 2.C
  [nl] gist.science, Dutch    - "Technische samenvatting": Methodologie, Implementatie
  [fr] gist.science, French   - "Resume technique" sections 1, 2.A, 2.B, 2.C
  [shd] shd-paper.top, Chinese - method detail section and the English abstract

The pages describe a three-stage pipeline ([es] "Implementacion", [nl]
"Implementatie", [fr] 2.C): (1) downsample Q, K and a V magnitude to block
level, (2) fix a per-query-block budget by the Token Position-Decay rule,
(3) keep the top blocks under the Output-Aware Metric and run exact softmax
attention over those blocks only.  Where the pages leave a step open, the
reading taken is stated in the function that implements it:

  * pooling: arithmetic mean of Q and of K over a block's tokens; the block's
    V magnitude is the mean of the per-token L2 norms (the pages only say
    "block-level Q, K and V magnitude"; [nl] mentions a max-pooled V
    magnitude, kept as a variant);
  * metric: m_ij = softmax_j(qbar_i . kbar_j / sqrt(d)) * w_j over the causal
    key blocks j <= i.  Inside one row log m_ij = s_ij + log w_j - log Z_i,
    so it orders blocks exactly like the pages' additive form
    s_ij + beta*max(0, log ||V_j||^2) with beta = 1/2 whenever log w_j^2 > 0
    ([es] 2.B equation, [fr] 2.B equation);
  * budget: k_dyn(i) = max(k_min, ceil(rho0 * exp(-i/tau) * (i+1))) plus the
    S sink blocks plus the diagonal block, capped at the i+1 causal blocks
    (the pages give a decay from a high to a low budget: linear in [es] 2.A,
    [fr] 2.A, exponential in [shd]);
  * ties in the metric go to the smaller block index, NaN ranks last;
  * every token of query block i attends to the union of i's selected key
    blocks, with the token-level causal mask applied inside the diagonal
    block only;
  * a final partial block (sequence length not a multiple of the block size)
    pools over its valid tokens only;
  * anti-diagonal sampling ([fr] 2.C step 1), the alternative block logit:
    the log-mean-exp of anti-diagonal samples of the token logits, in place
    of the pooled logit (reading stated above antidiag_row_logits).
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# block layout


def block_layout(cu_seqlens: Sequence[int], block: int) -> np.ndarray:
    """cu_blocks[s] = first global block of sequence s (ceil(len/block) each)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nb = [(int(cu[s + 1] - cu[s]) + block - 1) // block for s in range(len(cu) - 1)]
    return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64) if nb else np.zeros(1, np.int64)


def tri(n: int) -> int:
    return n * (n + 1) // 2


def score_offsets(cu_blocks: np.ndarray) -> Tuple[np.ndarray, int]:
    """Start of each sequence's packed lower triangle inside one head, and
    the per-head total.  Row i of a sequence starts tri(i) further on."""
    nbs = np.diff(cu_blocks)
    offs = np.zeros(len(nbs) + 1, dtype=np.int64)
    for s, n in enumerate(nbs):
        offs[s + 1] = offs[s] + tri(int(n))
    return offs, int(offs[-1])


# ----------------------------------------------------------------------------
# stage 1: downsampling ([es] "Implementacion" step 1, [nl] "Implementatie"
# step 1, [it] 2.C, [fr] 2.C step 1)


def pool_mean(x: np.ndarray, cu_seqlens: Sequence[int], block: int,
              dtype=np.float64) -> np.ndarray:
    """Block mean of x [T, H, d] -> [H, nbT, d] (float64; ``dtype`` only
    selects the precision of a timing run of the baseline)

    Block j of sequence s covers its tokens [j*B, min((j+1)*B, len_s)); the
    mean is over the tokens actually present."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cub = block_layout(cu, block)
    T, H, d = x.shape
    out = np.zeros((H, int(cub[-1]), d), dtype=dtype)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        for jl in range(int(cub[s + 1] - cub[s])):
            t0 = a + jl * block
            t1 = min(t0 + block, e)
            seg = x[t0:t1].astype(dtype)               # [n, H, d]
            out[:, int(cub[s]) + jl, :] = seg.sum(axis=0) / (t1 - t0)
    return out


def pool_vnorm(v: np.ndarray, cu_seqlens: Sequence[int], block: int,
               mode: str = "mean", dtype=np.float64) -> np.ndarray:
    """Block V magnitude w [Hkv, nbT]: mean (default) or max over the block's
    tokens of the token's L2 norm ||v_t||_2."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cub = block_layout(cu, block)
    T, H, d = v.shape
    out = np.zeros((H, int(cub[-1])), dtype=dtype)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        for jl in range(int(cub[s + 1] - cub[s])):
            t0 = a + jl * block
            t1 = min(t0 + block, e)
            seg = v[t0:t1].astype(dtype)
            norms = np.sqrt((seg * seg).sum(axis=2))   # [n, H]
            if mode == "mean":
                out[:, int(cub[s]) + jl] = norms.sum(axis=0) / (t1 - t0)
            elif mode == "max":
                out[:, int(cub[s]) + jl] = norms.max(axis=0)
            else:
                raise ValueError(mode)
    return out


# ----------------------------------------------------------------------------
# Output-Aware Metric ([es] 2.B equation and text, [it] 2.B, [nl] OAM,
# [fr] 2.B): routing relevance of the block times the magnitude of its values


METRICS = ("output_aware", "additive", "routing")


def score(qbar: np.ndarray, kbar: np.ndarray, w: np.ndarray,
          cu_blocks: np.ndarray, head_dim: int, metric: str = "output_aware",
          beta: float = 0.2, dtype=np.float64) -> np.ndarray:
    """Packed lower-triangular metric m [Hq, tri_total] (float64; ``dtype``
    as for pool_mean).

    For query head h (KV head g = h // (Hq/Hkv)), sequence s and local query
    block i, the row holds, for j = 0..i (local key blocks):
        s_ij = qbar_i . kbar_j / sqrt(head_dim)
        p_ij = exp(s_ij - max_j s) / sum_j exp(s_ij - max_j s)
        m_ij = p_ij * w_j                         metric "output_aware"
             = s_ij + beta * max(0, log(w_j^2))   metric "additive" (the
               displayed formula of [es] 2.B and [fr] 2.B; beta defaults to
               0.2, the value [nl] gives in its Output-Aware Metric paragraph
               and [es] 3 reports as the ablation's best)
             = p_ij                               metric "routing" (attention
               score alone, the criterion [es] 1 argues against)
    """
    Hq = qbar.shape[0]
    offs, total = score_offsets(cu_blocks)
    out = np.zeros((Hq, total), dtype=dtype)
    for h in range(Hq):
        for s in range(len(cu_blocks) - 1):
            nb = int(cu_blocks[s + 1]) - int(cu_blocks[s])
            for i in range(nb):
                row0 = int(offs[s]) + tri(i)
                out[h, row0:row0 + i + 1] = score_row_values(qbar, kbar, w, cu_blocks,
                                                             head_dim, h, s, i,
                                                             metric, beta, dtype)
    return out


def score_row_values(qbar: np.ndarray, kbar: np.ndarray, w: np.ndarray,
                     cu_blocks: np.ndarray, head_dim: int, h: int, s: int, i: int,
                     metric: str = "output_aware", beta: float = 0.2,
                     dtype=np.float64) -> np.ndarray:
    """One row of the metric: m_i0 .. m_ii for query head h, sequence s,
    local query block i (see score)."""
    if metric not in METRICS:
        raise ValueError(metric)
    g = h // (qbar.shape[0] // kbar.shape[0])
    b0 = int(cu_blocks[s])
    logits = kbar[g, b0:b0 + i + 1, :] @ qbar[h, b0 + i, :] * dtype(1.0 / math.sqrt(head_dim))
    return metric_from_logits(logits, w[g, b0:b0 + i + 1], metric, beta, dtype)


def metric_from_logits(logits: np.ndarray, wj: np.ndarray, metric: str = "output_aware",
                       beta: float = 0.2, dtype=np.float64) -> np.ndarray:
    """The metric of one row from its block logits s_i0 .. s_ii and the key
    blocks' V magnitudes (the three forms listed in score).  A row whose
    logits are all -inf (no sampled evidence, see antidiag_row_logits) gets
    routing weight 0 everywhere."""
    if metric not in METRICS:
        raise ValueError(metric)
    logits = np.asarray(logits, dtype=dtype)
    wj = np.asarray(wj, dtype=dtype)
    if metric == "additive":
        # log(0) = -inf, so a block of zero values gets no bonus
        with np.errstate(divide="ignore"):
            lw2 = np.log(wj * wj)
        return logits + beta * np.maximum(0.0, lw2)
    top = logits.max()
    if not np.isfinite(top):
        p = np.zeros_like(logits)
    else:
        p = np.exp(logits - top)
        p /= p.sum()
    return p if metric == "routing" else p * wj


def score_row(m: np.ndarray, cu_blocks: np.ndarray, h: int, s: int, i: int) -> np.ndarray:
    offs, _ = score_offsets(cu_blocks)
    row0 = int(offs[s]) + tri(i)
    return m[h, row0:row0 + i + 1]


# ----------------------------------------------------------------------------
# Anti-diagonal sampled block logits ([fr] 2.C, step 1: the block metric is
# computed with anti-diagonal sampling, for efficiency; the page gives no
# stride and no formula).  Reading taken here:
#   * a sequence's tokens are cut into groups of `stride` consecutive
#     positions (the last group may be short); stride divides the block size,
#     so block i holds groups i*B/stride .. (i+1)*B/stride - 1;
#   * the sample of query group r and key group c is the anti-diagonal of
#     their stride x stride tile of token logits: query position
#     r*stride + stride-1-u with key position c*stride + u, u = 0..stride-1,
#     keeping only pairs whose two tokens exist and whose key does not come
#     after the query; the sample value is the mean of q.k/sqrt(d) over
#     those pairs (a group pair with no such pair gives no sample);
#   * the block logit t_ij is the log of the mean of exp(sample) over the
#     samples of query block i and key block j (-inf if there are none),
#     so softmax_j(t_ij) is the share of query block i's sampled attention
#     mass that lands on key block j;
#   * t_ij then takes the place of the pooled logit s_ij in the metric,
#     unchanged otherwise (metric_from_logits).
# With stride 1 every causal token pair is sampled and t_ij is the exact
# log-mean-exp of the block pair's token logits.


def antidiag_row_logits(q: np.ndarray, k: np.ndarray, cu_seqlens: Sequence[int],
                        block: int, stride: int, h: int, s: int, i: int) -> np.ndarray:
    """t_i0 .. t_ii (float64) for query head h, sequence s, local query
    block i; q [T, Hq, d], k [T, Hkv, d]."""
    if stride < 1 or block % stride:
        raise ValueError("stride must divide the block size")
    T, Hq, d = q.shape
    g = h // (Hq // k.shape[1])
    t0 = int(cu_seqlens[s])
    n = int(cu_seqlens[s + 1]) - t0
    gpb = block // stride
    ng = -(-n // stride)
    rows = np.arange(i * gpb, min((i + 1) * gpb, ng))
    cols = np.arange(0, min((i + 1) * gpb, ng))
    u = np.arange(stride)
    qpos = rows[:, None] * stride + (stride - 1) - u[None, :]      # [R, stride]
    kpos = cols[:, None] * stride + u[None, :]                     # [C, stride]
    ok = ((qpos[:, None, :] < n) & (kpos[None, :, :] < n) &
          (kpos[None, :, :] <= qpos[:, None, :]))                  # [R, C, stride]
    qi = np.minimum(qpos, n - 1)
    kj = np.minimum(kpos, n - 1)
    # token logits of the rows' query tokens against the keys up to block i
    qt = q[t0:t0 + n, h, :].astype(np.float64)
    kt = k[t0:t0 + n, g, :].astype(np.float64)
    lq0, lq1 = int(qi.min()), int(qi.max()) + 1
    lk1 = int(kj.max()) + 1
    L = (qt[lq0:lq1] @ kt[:lk1].T) / math.sqrt(d)
    vals = L[(qi - lq0)[:, None, :], kj[None, :, :]]
    cnt = ok.sum(axis=2)
    tot = np.where(ok, vals, 0.0).sum(axis=2)
    out = np.full(i + 1, -np.inf)
    for j in range(i + 1):
        sel = (cols >= j * gpb) & (cols < (j + 1) * gpb)
        c = cnt[:, sel]
        x = tot[:, sel][c > 0] / c[c > 0]
        if x.size:
            top = x.max()
            out[j] = top + math.log(np.exp(x - top).mean())
    return out


def antidiag_block_logits(q: np.ndarray, k: np.ndarray, cu_seqlens: Sequence[int],
                          block: int, stride: int) -> np.ndarray:
    """Packed lower-triangular anti-diagonal block logits t [Hq, tri_total]."""
    cu_blocks = block_layout(cu_seqlens, block)
    offs, total = score_offsets(cu_blocks)
    Hq = q.shape[1]
    out = np.full((Hq, total), -np.inf)
    for h in range(Hq):
        for s in range(len(cu_blocks) - 1):
            for i in range(int(cu_blocks[s + 1]) - int(cu_blocks[s])):
                row0 = int(offs[s]) + tri(i)
                out[h, row0:row0 + i + 1] = antidiag_row_logits(q, k, cu_seqlens, block,
                                                                stride, h, s, i)
    return out


def score_antidiag(q: np.ndarray, k: np.ndarray, w: np.ndarray, cu_seqlens: Sequence[int],
                   block: int, stride: int, metric: str = "output_aware",
                   beta: float = 0.2) -> np.ndarray:
    """The metric with anti-diagonal sampled block logits in place of the
    pooled ones: packed m [Hq, tri_total] (float64)."""
    cu_blocks = block_layout(cu_seqlens, block)
    offs, total = score_offsets(cu_blocks)
    t = antidiag_block_logits(q, k, cu_seqlens, block, stride)
    Hq = q.shape[1]
    G = Hq // k.shape[1]
    out = np.zeros((Hq, total))
    for h in range(Hq):
        for s in range(len(cu_blocks) - 1):
            b0 = int(cu_blocks[s])
            for i in range(int(cu_blocks[s + 1]) - b0):
                row0 = int(offs[s]) + tri(i)
                out[h, row0:row0 + i + 1] = metric_from_logits(
                    t[h, row0:row0 + i + 1], w[h // G, b0:b0 + i + 1], metric, beta)
    return out


# ----------------------------------------------------------------------------
# Token Position-Decay budget ([es] 2.A, [it] 2.A, [nl] TPD, [fr] 2.A; the
# exponential decay of [shd] method detail); one budget per query block
# ([es] "Implementacion" step 2, [nl] "Implementatie" step 2)


def budget(nb: int, sink_blocks: int, k_min: int, rho0: float, tau: float) -> np.ndarray:
    """k_i for the nb query blocks of one sequence (int64).

    k_dyn(i) = max(k_min, ceil(rho0 * exp(-i/tau) * (i+1)))   (float64 math)
    k_i      = i+1                          if i < S
             = min(i+1, S + 1 + k_dyn(i))   otherwise
    i is the 0-based block index within the sequence, tau is in blocks and
    (i+1) counts the causal key blocks of row i."""
    out = np.zeros(nb, dtype=np.int64)
    for i in range(nb):
        if i < sink_blocks:
            out[i] = i + 1
            continue
        x = rho0 * math.exp(-i / tau) * (i + 1)
        kd = max(k_min, int(math.ceil(x)))
        out[i] = min(i + 1, sink_blocks + 1 + kd)
    return out


def budget_linear(nb: int, sink_blocks: int, k_min: int, k_start: float,
                  mu: float) -> np.ndarray:
    """The pages' linear form ([es] 2.A, [fr] 2.A): the number of dynamically
    chosen blocks goes linearly from k_start at the first query block of the
    sequence to k_end = mu*k_start at its last, rounded up and floored at
    k_min; sinks and diagonal are added on top and the causal count caps it:
        f        = i / (nb - 1)            (0 when nb = 1)
        k_dyn(i) = max(k_min, ceil(k_start*(1-f) + mu*k_start*f))
        k_i      = i+1 if i < S, else min(i+1, S + 1 + k_dyn(i))"""
    out = np.zeros(nb, dtype=np.int64)
    for i in range(nb):
        if i < sink_blocks:
            out[i] = i + 1
            continue
        frac = 0.0 if nb <= 1 else i / (nb - 1)
        kd = max(k_min, int(math.ceil(k_start * (1.0 - frac) + mu * k_start * frac)))
        out[i] = min(i + 1, sink_blocks + 1 + kd)
    return out


def budget_linear_fraction(nb: int, sink_blocks: int, k_min: int, k_start: float,
                           mu: float) -> np.ndarray:
    """The linear ramp of [es] 2.A / [fr] 2.A read as a share of each row's
    causal blocks (the pages give no unit for k_start): query block i keeps
    the fraction r(i) = k_start at the sequence's first block decaying
    linearly to mu*k_start at its last, of its i+1 key blocks, rounded up and
    floored at k_min; sinks and diagonal on top, the causal count caps it:
        f        = i / (nb - 1)            (0 when nb = 1)
        r(i)     = k_start*(1-f) + mu*k_start*f
        k_dyn(i) = max(k_min, ceil(r(i) * (i+1)))
        k_i      = i+1 if i < S, else min(i+1, S + 1 + k_dyn(i))"""
    out = np.zeros(nb, dtype=np.int64)
    for i in range(nb):
        if i < sink_blocks:
            out[i] = i + 1
            continue
        frac = 0.0 if nb <= 1 else i / (nb - 1)
        share = k_start * (1.0 - frac) + mu * k_start * frac
        kd = max(k_min, int(math.ceil(share * (i + 1))))
        out[i] = min(i + 1, sink_blocks + 1 + kd)
    return out


# ----------------------------------------------------------------------------
# selection: forced sink blocks (initial tokens are recursive anchors, [es] 1,
# [fr] 1 and 2.A) plus the diagonal, then the top blocks of the metric
# ([es] "Implementacion" step 3, [nl] "Implementatie" step 3)


def _rank_key(values: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Order for 'best first': larger metric first, ties to smaller index,
    NaN last.  Returns a permutation of positions."""
    v = values.astype(np.float64)
    nan = np.isnan(v)
    neg = np.where(nan, 0.0, -v)
    neg = neg + 0.0          # -0.0 -> +0.0 so that -0 and +0 tie
    return np.lexsort((idx, neg, nan))


def select_row(m_row: np.ndarray, i: int, k_i: int, sink_blocks: int) -> np.ndarray:
    """Selected key blocks of query block i, ascending (int64).

    forced F = {0..min(S, i+1)-1} U {i}; candidates C = {S..i-1}; the best
    (k_i - |F|) candidates by m are added (all of them if fewer remain)."""
    forced = set(range(min(sink_blocks, i + 1)))
    forced.add(i)
    cand = np.arange(sink_blocks, i, dtype=np.int64)
    take = max(0, k_i - len(forced))
    chosen: List[int] = []
    if take > 0 and cand.size:
        order = _rank_key(m_row[cand], cand)
        chosen = [int(c) for c in cand[order[:take]]]
    return np.array(sorted(forced | set(chosen)), dtype=np.int64)


def select(m: np.ndarray, cu_blocks: np.ndarray, budgets: np.ndarray,
           sink_blocks: int, kmax: Optional[int] = None):
    """idx [Hq, nbT, kmax] int32 (-1 padded, ascending, sequence-local block
    numbers) and count [Hq, nbT] int32.  ``budgets`` is per global block."""
    Hq = m.shape[0]
    nbT = int(cu_blocks[-1])
    if kmax is None:
        kmax = int(budgets.max()) if nbT else 0
    idx = np.full((Hq, nbT, kmax), -1, dtype=np.int32)
    cnt = np.zeros((Hq, nbT), dtype=np.int32)
    for h in range(Hq):
        for s in range(len(cu_blocks) - 1):
            b0 = int(cu_blocks[s])
            for i in range(int(cu_blocks[s + 1]) - b0):
                sel = select_row(score_row(m, cu_blocks, h, s, i), i,
                                 int(budgets[b0 + i]), sink_blocks)
                idx[h, b0 + i, :sel.size] = sel
                cnt[h, b0 + i] = sel.size
    return idx, cnt


# ----------------------------------------------------------------------------
# exact softmax aggregation over the selected blocks only ([es]
# "Implementacion" step 3, [it] 2.C, [nl] "Implementatie" step 3, [fr] 2.C
# step 3)


def attn_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens, block: int,
             s: int, i: int, h: int, G: int, blocks: Iterable[int], dtype=np.float64):
    """Output rows and natural-log LSE for the tokens of query block i of
    sequence s, query head h, attending to the given local key blocks.

    Token-level causality: key token position p may be seen by query token
    position t iff p <= t (positions are local to the sequence)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    a, e = int(cu[s]), int(cu[s + 1])
    g = h // G
    t0 = a + i * block
    t1 = min(t0 + block, e)
    keys = []
    for j in blocks:
        j0 = a + int(j) * block
        keys.extend(range(j0, min(j0 + block, e)))
    keys = np.asarray(keys, dtype=np.int64)
    qi = q[t0:t1, h, :].astype(dtype)
    kj = k[keys, g, :].astype(dtype)
    vj = v[keys, g, :].astype(dtype)
    d = q.shape[2]
    logits = (qi @ kj.T) / math.sqrt(d)
    allowed = keys[None, :] <= np.arange(t0, t1)[:, None]
    logits = np.where(allowed, logits, -np.inf)
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vj) / l
    lse = (mx + np.log(l))[:, 0]
    return o, lse


def sparse_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                count: np.ndarray, cu_seqlens, block: int,
                rows: Optional[Iterable[Tuple[int, int]]] = None, dtype=np.float64):
    """Block-sparse causal attention.

    Returns (o [T, Hq, d], lse [Hq, T]) in float64 for every row when
    ``rows`` is None; otherwise a dict {(h, global_block): (o_rows, lse_rows)}
    for just the requested (query head, global query block) pairs."""
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cub = block_layout(cu, block)
    seq_of_block = np.repeat(np.arange(len(cu) - 1), np.diff(cub))

    def one(h, b):
        s = int(seq_of_block[b])
        i = b - int(cub[s])
        blocks = idx[h, b, :int(count[h, b])]
        return attn_row(q, k, v, cu, block, s, i, h, G, blocks, dtype)

    if rows is not None:
        return {(h, b): one(h, b) for (h, b) in rows}
    o = np.zeros((T, Hq, d), dtype=dtype)
    lse = np.zeros((Hq, T), dtype=dtype)
    for h in range(Hq):
        for b in range(int(cub[-1])):
            s = int(seq_of_block[b])
            t0 = int(cu[s]) + (b - int(cub[s])) * block
            t1 = min(t0 + block, int(cu[s + 1]))
            ob, lb = one(h, b)
            o[t0:t1, h, :] = ob
            lse[h, t0:t1] = lb
    return o, lse


def dense_causal_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens):
    """Ordinary causal softmax attention per sequence, written independently
    of the block machinery (for the full-budget check).  float64."""
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    o = np.zeros((T, Hq, d), dtype=np.float64)
    lse = np.zeros((Hq, T), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        n = e - a
        if n == 0:
            continue
        mask = np.tril(np.ones((n, n), dtype=bool))
        for h in range(Hq):
            qq = q[a:e, h, :].astype(np.float64)
            kk = k[a:e, h // G, :].astype(np.float64)
            vv = v[a:e, h // G, :].astype(np.float64)
            lg = np.where(mask, qq @ kk.T / math.sqrt(d), -np.inf)
            mx = lg.max(axis=1, keepdims=True)
            p = np.exp(lg - mx)
            l = p.sum(axis=1, keepdims=True)
            o[a:e, h, :] = (p @ vv) / l
            lse[h, a:e] = (mx + np.log(l))[:, 0]
    return o, lse


# ----------------------------------------------------------------------------
# the whole path


def budgets_for(cu_blocks: np.ndarray, sink_blocks: int, k_min: int,
                rho0: float, tau: float, mode: str = "exp", k_start: float = 0.0,
                mu: float = 0.0) -> np.ndarray:
    """Per-global-block budget table, each sequence restarting at i = 0;
    mode "exp" uses budget, mode "linear" budget_linear and mode
    "linear_fraction" budget_linear_fraction."""
    if mode == "exp":
        parts = [budget(int(cu_blocks[s + 1] - cu_blocks[s]), sink_blocks, k_min, rho0, tau)
                 for s in range(len(cu_blocks) - 1)]
    elif mode == "linear":
        parts = [budget_linear(int(cu_blocks[s + 1] - cu_blocks[s]), sink_blocks, k_min,
                               k_start, mu)
                 for s in range(len(cu_blocks) - 1)]
    elif mode == "linear_fraction":
        parts = [budget_linear_fraction(int(cu_blocks[s + 1] - cu_blocks[s]), sink_blocks,
                                        k_min, k_start, mu)
                 for s in range(len(cu_blocks) - 1)]
    else:
        raise ValueError(mode)
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def prefill(q, k, v, cu_seqlens, block, sink_blocks, k_min, rho0, tau,
            vnorm_mode: str = "mean", metric: str = "output_aware", beta: float = 0.2,
            budget_mode: str = "exp", k_start: float = 0.0, mu: float = 0.0,
            score_stride: Optional[int] = None):
    """pool -> score -> budget -> select -> attention.  Returns a dict of
    every intermediate (float64 / int).  With score_stride set, the metric
    takes the anti-diagonal sampled block logits (score_antidiag)."""
    d = q.shape[2]
    cub = block_layout(cu_seqlens, block)
    qbar = pool_mean(q, cu_seqlens, block)
    kbar = pool_mean(k, cu_seqlens, block)
    w = pool_vnorm(v, cu_seqlens, block, vnorm_mode)
    if score_stride is None:
        m = score(qbar, kbar, w, cub, d, metric, beta)
    else:
        m = score_antidiag(q, k, w, cu_seqlens, block, score_stride, metric, beta)
    bud = budgets_for(cub, sink_blocks, k_min, rho0, tau, budget_mode, k_start, mu)
    idx, cnt = select(m, cub, bud, sink_blocks)
    o, lse = sparse_attn(q, k, v, idx, cnt, cu_seqlens, block)
    return dict(qbar=qbar, kbar=kbar, w=w, m=m, budget=bud, idx=idx,
                count=cnt, o=o, lse=lse, cu_blocks=cub)

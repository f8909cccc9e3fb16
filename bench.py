"""Benchmark of the Stem sparse-prefill path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --sweep        latency against context length, Stem vs dense

A step is one pass of the whole path over one batch of synthetic input with
the inputs already resident in HBM: stem_pool -> stem_score -> stem_select
-> stem_sparse_attn, all through the C ABI on one stream.  Each call is
bracketed by HIP events on that stream, so per-stage times (and the
attention kernel's own duration, used for the roofline) are measured live.

Reported (one JSON line on stdout, progress on stderr):
  value       prefill latency per step in ms (the metric is a latency)
  roofline    the attention kernel against the bf16 matrix-core peak, with
              algorithmic FLOPs = 4 B^2 d per executed (head, query block,
              key block), the diagonal block counted as half a tile
  stages      per-stage ms; effective TFLOP/s of attention and of the step
  dense       the same attention kernel with every causal block kept (the
              dense causal comparator) and the speed-up over it
  ceilings    the chip's matrix-core rate on random and on constant bf16
              operands and its streaming HBM read rate, re-measured by the
              library's probe kernels (the published peaks assume neither
              the power limit nor the memory system's efficiency), and the
              attention kernel's time on its own block lists with V, Q, or
              Q, K and V set to zero (same work, operands that do not toggle)
  cpu_baseline  the CPU oracle timed stage by stage on a bounded sample and
              scaled up (fp64, the oracle's precision, plus an fp32 line)
  step_ms_spread / attn_ms_spread  mean, median, min and max of the timed
              steps (value is the mean)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("Stem prefill latency (ms) + effective TFLOP/s & % MFMA peak at 128K, "
          "Llama-8B head shape")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3       # MI355X dense f32 matrix-core peak
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_flops(plan, diag_half: bool) -> float:
    i = plan.info
    per_tile = 4.0 * i.block * i.block * i.head_dim
    full = per_tile * i.executed_blocks_per_head * i.num_q_heads
    if not diag_half:
        return full
    return full - 0.5 * per_tile * i.total_blocks * i.num_q_heads


def traffic_record(workload: str, profile: str = None, source: str = "attn.hip"):
    """HBM bytes per launch of a kernel measured by rocprofv3 (FETCH_SIZE and
    WRITE_SIZE, copy-calibrated) and recorded under profiles/ (by default the
    attention kernel's); returned only if the kernel's source is unchanged
    since that measurement."""
    path = os.path.join(ROOT, "profiles", profile or f"attn_{workload}.md")
    src = os.path.join(ROOT, "block_sparse_causal_amd", "csrc", source)
    try:
        rec = None
        for line in open(path):
            if line.startswith("traffic_record:"):
                rec = json.loads(line.split(":", 1)[1])
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != sha:
        return None
    return rec


def upload(x, device="cuda"):
    import torch
    if x.workload.dtype == "bf16":
        conv = lambda b: torch.from_numpy(b.view(np.int16)).to(device).view(torch.bfloat16)
        return conv(x.q_bits), conv(x.k_bits), conv(x.v_bits)
    return tuple(torch.from_numpy(a).to(device) for a in (x.q, x.k, x.v))


def time_path(plan, q, k, v, bufs, steps: int, warmup: int, vnorm_mode=0, score_stride=None):
    """Run warmup + timed steps; return (ms_per_step wall, per-stage ms lists).
    With score_stride set the metric stage is stem_score_antidiag."""
    import torch
    from block_sparse_causal_amd import stem
    st = torch.cuda.current_stream()
    if score_stride is None:
        score = lambda: stem.stem_score(plan, bufs.qbar, bufs.kbar, bufs.vnorm, bufs.scores, st)
    else:
        score = lambda: stem.stem_score_antidiag(plan, q, k, bufs.vnorm, score_stride, bufs.scores,
                                                 st)
    calls = [
        lambda: stem.stem_pool(plan, q, k, v, bufs.qbar, bufs.kbar, bufs.vnorm, vnorm_mode, st),
        score,
        lambda: stem.stem_select(plan, bufs.scores, bufs.idx, bufs.count, st),
        lambda: stem.stem_sparse_attn(plan, q, k, v, bufs.idx, bufs.count, bufs.out, bufs.lse, st),
    ]
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(st)
        for n, c in enumerate(calls):
            c()
            ev[s][n + 1].record(st)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / max(steps, 1)
    stage = [[ev[s][n].elapsed_time(ev[s][n + 1]) for s in range(steps)] for n in range(len(calls))]
    total = [ev[s][0].elapsed_time(ev[s][len(calls)]) for s in range(steps)]
    return wall, stage, total


def antidiag_flops(w, stride: int) -> float:
    """Algorithmic FLOPs of the anti-diagonal samples: 2 d per sampled token
    pair (key not after query, both tokens present), every query head."""
    pairs = 0
    for n in w.seqlens:
        ng = -(-n // stride)
        half = (stride + 1) // 2
        for r in range(ng):
            m = min(stride, n - r * stride)
            pairs += r * m + max(0, min(m - 1, half - 1) - (stride - m) + 1)
    return 2.0 * w.head_dim * pairs * w.num_q_heads


def dense_attention_ms(w, q, k, v, reps: int):
    """The same attention kernel with every causal block kept."""
    import torch
    from block_sparse_causal_amd import stem
    plan = stem.plan_for(w, k_min=1 << 30, rho0=0.0).to(q.device)
    bufs = stem.Buffers(plan, q.device, out_dtype=torch.bfloat16)
    stem.stem_pool(plan, q, k, v, bufs.qbar, bufs.kbar, bufs.vnorm)
    stem.stem_score(plan, bufs.qbar, bufs.kbar, bufs.vnorm, bufs.scores)
    stem.stem_select(plan, bufs.scores, bufs.idx, bufs.count)
    st = torch.cuda.current_stream()
    stem.stem_sparse_attn(plan, q, k, v, bufs.idx, bufs.count, bufs.out, bufs.lse, st)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        stem.stem_sparse_attn(plan, q, k, v, bufs.idx, bufs.count, bufs.out, bufs.lse, st)
        b.record(st)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    flops = attn_flops(plan, diag_half=True)
    del bufs
    return float(np.median(times)), flops


def cpu_baseline(w, x):
    """Time the oracle, as it stands, on one KV-head group (KV head 0 and its
    G query heads: pooling, every metric, selection and attention row of
    those heads), stage by stage, and scale to all KV heads.  The oracle
    computes in fp64; a second line runs the same code in fp32."""
    from oracle import stem_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    G = w.num_q_heads // w.num_kv_heads
    q, k, v = x.q[:, :G], x.k[:, :1], x.v[:, :1]
    cu, B = w.cu_seqlens, w.block

    def run(dt):
        st = {}
        t = time.perf_counter()
        cub = O.block_layout(cu, B)
        qbar = O.pool_mean(q, cu, B, dt)
        kbar = O.pool_mean(k, cu, B, dt)
        wv = O.pool_vnorm(v, cu, B, "mean", dt)
        st["pool"] = time.perf_counter() - t
        t = time.perf_counter()
        m = O.score(qbar, kbar, wv, cub, w.head_dim, w.metric, w.beta, dt)
        st["score"] = time.perf_counter() - t
        t = time.perf_counter()
        bud = O.budgets_for(cub, w.sink_blocks, w.k_min, w.rho0, w.tau, w.budget_mode,
                            w.k_start, w.mu)
        idx, cnt = O.select(m, cub, bud, w.sink_blocks)
        st["budget_select"] = time.perf_counter() - t
        t = time.perf_counter()
        O.sparse_attn(q, k, v, idx, cnt, cu, B, dtype=dt)
        st["attn"] = time.perf_counter() - t
        return st

    f64 = run(np.float64)
    f32 = run(np.float32)
    scale = w.num_kv_heads * 1e3
    nbT = int(O.block_layout(cu, B)[-1])
    sample = (f"oracle prefill of KV head 0 and its {G} query heads of {w.name} "
              f"(pool, metric, budget, selection and attention of all {nbT} query blocks), "
              f"scaled by {w.num_kv_heads} KV heads")
    return dict(value=round(sum(f64.values()) * scale, 1), unit="ms", cores=int(blas_threads),
                kind="oracle", sample=sample, sample_seconds=round(sum(f64.values()), 2),
                host_cpus=len(os.sched_getaffinity(0)), precision="fp64",
                stages_ms={k_: round(v_ * scale, 1) for k_, v_ in f64.items()},
                fp32={"value": round(sum(f32.values()) * scale, 1), "unit": "ms",
                      "stages_ms": {k_: round(v_ * scale, 1) for k_, v_ in f32.items()},
                      "sample_seconds": round(sum(f32.values()), 2)})


def measure_ceilings(reps: int = 5):
    """Best-of-reps rates of the probe kernels, timed with HIP events."""
    import torch
    from block_sparse_causal_amd import stem
    st = torch.cuda.current_stream()
    sink = torch.empty(4096, dtype=torch.float32, device="cuda")

    def best(launch):
        launch()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            work = launch()
            b.record(st)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        return work, min(ms)

    out = {}
    for key, rnd in (("mfma_bf16_random_tflops", True), ("mfma_bf16_constant_tflops", False)):
        flops, ms = best(lambda: stem.stem_probe_mfma(rnd, sink, st))
        out[key] = round(flops / (ms * 1e-3) / 1e12, 1)
    buf = torch.empty(1 << 29, dtype=torch.int64, device="cuda").fill_(0x0123456789)  # 4 GiB
    wsink = torch.zeros(buf.numel() * 8 // 65536, dtype=torch.int32, device="cuda")
    nbytes, ms = best(lambda: stem.stem_probe_hbm_read(buf, wsink, st))
    out["hbm_read_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    return out


def operand_sensitivity(plan, q, k, v, bufs, reps: int = 5):
    """The attention kernel on the step's own block lists, with the real
    operands and with V, with Q, and with Q, K and V replaced by zeros: the
    same instructions, LDS and memory traffic on operands whose bits do not
    toggle.  Median ms of reps alternating rounds (one launch per operand set
    and round)."""
    import torch
    from block_sparse_causal_amd import stem
    st = torch.cuda.current_stream()
    zq, zk, zv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    sets = {"real": (q, k, v), "zero_v": (q, k, zv), "zero_q": (zq, k, v), "zero_qkv": (zq, zk, zv)}
    out, lse = torch.empty_like(bufs.out), torch.empty_like(bufs.lse)
    ms = {n: [] for n in sets}
    for _ in range(reps):
        for n, (qq, kk, vv) in sets.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            stem.stem_sparse_attn(plan, qq, kk, vv, bufs.idx, bufs.count, out, lse, st)
            b.record(st)
            b.synchronize()
            ms[n].append(a.elapsed_time(b))
    del zq, zk, zv, out, lse
    torch.cuda.empty_cache()
    return {n: round(float(np.median(t)), 4) for n, t in ms.items()}


def copy_calibration(nbytes: int = 1 << 30):
    """One device-to-device copy of a known size, for scaling the hardware
    byte counters of a profiling run (its kernel reads and writes nbytes)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {nbytes} bytes read and written")


SWEEP_TOKENS = (8192, 16384, 32768, 65536, 131072)


def sweep(base_name: str, steps: int, warmup: int, dense_reps: int, score_stride=None):
    """Latency of the whole path and of the dense comparator (the same
    attention kernel with every causal block kept) at growing context length,
    with the head shape and Stem parameters of ``base_name`` (and the sampled
    metric at ``score_stride`` if given).  One JSON line per length, then a
    summary line."""
    import torch
    from block_sparse_causal_amd import stem
    from block_sparse_causal_amd import synthetic as syn
    base = syn.WORKLOADS[base_name]
    rows = []
    for n, tokens in enumerate(SWEEP_TOKENS):
        w = base.replace(name=f"{base_name}@{tokens // 1024}k", seqlens=(tokens,),
                         seed=base.seed + 100 + n)
        log(f"sweep {w.name}: generating inputs")
        x = syn.generate(w)
        q, k, v = upload(x)
        del x
        plan = stem.plan_for(w).to("cuda")
        bufs = stem.Buffers(plan, "cuda", out_dtype=torch.bfloat16)
        _, stage, total = time_path(plan, q, k, v, bufs, steps, warmup, score_stride=score_stride)
        del bufs
        step_ms = float(np.mean(total))
        attn_ms = float(np.mean(stage[3]))
        flops = attn_flops(plan, diag_half=True)
        dms, dflops = dense_attention_ms(w, q, k, v, dense_reps)
        row = {"tokens": tokens, "nb": int(plan.info.total_blocks),
               "executed_blocks_per_head": int(plan.info.executed_blocks_per_head),
               "stem_step_ms": round(step_ms, 4),
               "stages_ms": {nm: round(float(np.mean(st_)), 4)
                             for nm, st_ in zip(["pool", "score", "select", "attn"], stage)},
               "stem_attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 1),
               "dense_attn_ms": round(dms, 3),
               "dense_attn_tflops": round(dflops / (dms * 1e-3) / 1e12, 1),
               "speedup": round(dms / step_ms, 2)}
        if score_stride is not None:
            af = antidiag_flops(w, score_stride)
            row["score_stride"] = score_stride
            row["antidiag_tflops"] = round(af / (float(np.mean(stage[1])) * 1e-3) / 1e12, 1)
        log(f"sweep {tokens:>6} tokens: stem {step_ms:.3f} ms, dense {dms:.3f} ms, "
            f"speed-up {dms / step_ms:.2f}x")
        print(json.dumps({"sweep": base_name, **row}), flush=True)
        rows.append(row)
        del q, k, v, plan
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": base_name, "summary": [
        (r["tokens"], r["stem_step_ms"], r["dense_attn_ms"], r["speedup"]) for r in rows]}),
        flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--score-stride", type=int, default=None,
                    help="metric from anti-diagonal samples of the token logits at this stride "
                         "(stem_score_antidiag) instead of the pooled blocks")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the matrix-core and HBM probe kernels")
    ap.add_argument("--tokens", type=int, default=None,
                    help="one sequence of this many tokens with the workload's head shape and "
                         "parameters (a point of the context-length sweep)")
    ap.add_argument("--sweep", action="store_true",
                    help="latency against context length (8K..128K), Stem vs dense")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_causal_amd import stem
    from block_sparse_causal_amd import synthetic as syn

    name = args.workload or syn.HEADLINE
    if args.sweep:
        sweep(name, args.steps, args.warmup, args.dense_reps, args.score_stride)
        return
    w = syn.WORKLOADS[name]
    if args.tokens:
        w = w.replace(name=f"{name}@{args.tokens // 1024}k", seqlens=(args.tokens,),
                      seed=w.seed + 100 + SWEEP_TOKENS.index(args.tokens)
                      if args.tokens in SWEEP_TOKENS else w.seed + 200)
        name = w.name
    log(f"workload {name}: generating seeded inputs")
    t = time.perf_counter()
    x = syn.generate(w)
    log(f"inputs ready in {time.perf_counter() - t:.1f}s; uploading")
    q, k, v = upload(x)
    plan = stem.plan_for(w).to("cuda")
    out_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    bufs = stem.Buffers(plan, "cuda", out_dtype=out_dtype)
    torch.cuda.synchronize()

    log(f"timing {args.warmup} warmup + {args.steps} steps")
    wall_ms, stage, total = time_path(plan, q, k, v, bufs, args.steps, args.warmup,
                                      score_stride=args.score_stride)
    names = ["pool", "score", "select", "attn"]
    stage_ms = {n: float(np.mean(s)) for n, s in zip(names, stage)}
    step_ms = float(np.mean(total))
    spread = lambda v: {"mean": round(float(np.mean(v)), 4), "median": round(float(np.median(v)), 4),
                        "min": round(float(np.min(v)), 4), "max": round(float(np.max(v)), 4)}
    log(f"step {step_ms:.3f} ms (median {np.median(total):.3f}, min {np.min(total):.3f}; "
        f"wall {wall_ms:.3f} ms): " + ", ".join(f"{n} {stage_ms[n]:.3f}" for n in names))

    flops_alg = attn_flops(plan, diag_half=True)
    flops_full = attn_flops(plan, diag_half=False)
    attn_ms = stage_ms["attn"]
    achieved = flops_alg / (attn_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    i = plan.info
    esz = 2 if w.dtype == "bf16" else 4
    pool_bytes = i.total_tokens * (i.num_q_heads + 2 * i.num_kv_heads) * i.head_dim * esz + \
        4 * i.total_blocks * ((i.num_q_heads + i.num_kv_heads) * i.head_dim + i.num_kv_heads)
    select_bytes = 4 * i.num_q_heads * i.score_elems_per_head + \
        4 * i.num_q_heads * i.total_blocks * (i.kmax + 1)

    trec = traffic_record(name)
    # Q, K, V read once, O and LSE written once
    attn_bytes_min = i.total_tokens * (i.num_q_heads + 2 * i.num_kv_heads) * i.head_dim * esz + \
        i.total_tokens * i.num_q_heads * i.head_dim * out_dtype.itemsize + 4 * i.total_tokens * i.num_q_heads
    result = {
        "metric": METRIC,
        "value": round(step_ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; Q,K ~ N(0,1) with RoPE, sink K x3, V ~ N(0,1) x LogNormal(0,0.5))",
        "config": {"workload": name, "seq_lens": list(w.seqlens), "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block": w.block,
                   "sink_blocks": w.sink_blocks, "k_min": w.k_min, "rho0": w.rho0,
                   "tau_blocks": w.tau, "out_dtype": str(out_dtype).replace("torch.", ""),
                   "executed_blocks_per_head": i.executed_blocks_per_head},
        "roofline": {"bound": "mfma", "kernel": "attn", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": (None if trec is None
                                 else trec["fetch_bytes"] + trec["write_bytes"]),
                     "traffic_detail": trec,
                     "algorithmic_bytes_min": attn_bytes_min,
                     "flop_per_launch": flops_alg,
                     "avg_launch_ms": round(attn_ms, 4)},
        "stages_ms": {n: round(stage_ms[n], 4) for n in names},
        "step_ms_spread": spread(total),
        "attn_ms_spread": spread(stage[3]),
        "effective_tflops": {"attn_diag_half": round(achieved, 2),
                             "attn_full_tiles": round(flops_full / (attn_ms * 1e-3) / 1e12, 2),
                             "step_diag_half": round(flops_alg / (step_ms * 1e-3) / 1e12, 2)},
        "hbm_gbs": {"pool": round(pool_bytes / (stage_ms["pool"] * 1e-3) / 1e9, 1),
                    "select": round(select_bytes / (stage_ms["select"] * 1e-3) / 1e9, 1),
                    "peak": PEAK_HBM_GBS},
        "wall_ms_per_step": round(wall_ms, 4),
    }
    if args.score_stride is not None:
        af = antidiag_flops(w, args.score_stride)
        ach = af / (stage_ms["score"] * 1e-3) / 1e12
        result["config"]["score"] = f"antidiag stride {args.score_stride}"
        # the score stage is stem_score_antidiag: the sample products plus
        # the row-softmax kernel
        arec = traffic_record(name, f"antidiag_{name}_stride{args.score_stride}.md", "antidiag.hip")
        result["antidiag"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                              "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                              "traffic": (None if arec is None
                                          else arec["fetch_bytes"] + arec["write_bytes"]),
                              "flop_per_launch": af, "avg_launch_ms": round(stage_ms["score"], 4)}
        log(f"antidiag stride {args.score_stride}: {stage_ms['score']:.3f} ms, {ach:.1f} TFLOP/s")
    operands = None
    if not args.no_ceilings:
        log("attention on zeroed operands (same block lists)")
        operands = operand_sensitivity(plan, q, k, v, bufs)
        log(f"attention ms by operands: {operands}")
    del bufs

    if not args.no_dense:
        log("dense comparator: same kernel, every causal block kept")
        dms, dflops = dense_attention_ms(w, q, k, v, args.dense_reps)
        result["dense"] = {"attn_ms": round(dms, 3),
                           "tflops": round(dflops / (dms * 1e-3) / 1e12, 2),
                           "speedup_vs_stem_step": round(dms / step_ms, 2)}
        log(f"dense attention {dms:.2f} ms -> speed-up {dms / step_ms:.2f}x")

    if not args.no_ceilings:
        log("probe kernels: matrix-core and HBM ceilings")
        c = measure_ceilings()
        c["attn_frac_of_random_mfma"] = round(achieved / c["mfma_bf16_random_tflops"], 4)
        c["pool_frac_of_hbm_read"] = round(result["hbm_gbs"]["pool"] / c["hbm_read_gbs"], 4)
        c["attn_ms_by_operands"] = operands
        result["ceilings"] = c
        log(f"ceilings: {c}")

    if args.copy_calibration:
        copy_calibration()

    if not args.no_cpu:
        log("CPU oracle baseline on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, x)
        log(f"cpu baseline {result['cpu_baseline']['value']} ms (scaled)")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

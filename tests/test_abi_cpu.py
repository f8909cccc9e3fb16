"""Host-side checks of libstem that need no GPU: the library loads and exports
every entry point the header declares, stem_plan agrees with the oracle's
layout and budget tables exactly, and bad arguments are rejected before any
HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_sparse_causal_amd import stem
from block_sparse_causal_amd import synthetic as syn
from oracle import stem_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "stem.h")).read()
    names = set(re.findall(r"^\s*(?:int|const char \*)\s*(stem_\w+)\s*\(", hdr, re.M))
    assert names >= {"stem_plan", "stem_pool", "stem_score", "stem_select",
                     "stem_sparse_attn", "stem_status_str"}
    L = stem.lib()
    for n in sorted(names):
        assert hasattr(L, n), n
    # the binding uses the same names
    for n in names - {"stem_status_str"}:
        assert hasattr(stem, n), n


def test_binding_shares_torchs_hip_runtime():
    # Loading the library first in a fresh process (no torch imported yet)
    # must still leave one HIP runtime mapped: the one torch loads.  Two
    # copies make torch's streams invalid for the library's launches.
    import subprocess
    import sys
    code = ("import re\n"
            "from block_sparse_causal_amd import stem\n"
            "stem.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(sorted(set(re.findall(r'\\S*libamdhip64\\S*', maps))))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    paths = eval(r.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths


def test_struct_layouts_match_header():
    # offsets follow C layout rules; a mismatch would corrupt every call
    assert ctypes.sizeof(stem.stem_params) == 56
    assert stem.stem_params.budget_mode.offset == 24
    assert stem.stem_params.beta.offset == 48
    assert stem.stem_plan_info.metric_mode.offset == 40
    assert stem.stem_plan_info.beta.offset == 48
    assert stem.stem_plan_info.total_tokens.offset == 56
    assert ctypes.sizeof(stem.stem_plan_info) == 56 + 11 * 8
    assert stem.stem_problem.cu_seqlens.offset == 8


@pytest.mark.parametrize("name", list(syn.WORKLOADS))
def test_plan_matches_oracle_tables(name):
    w = syn.WORKLOADS[name]
    p = stem.plan_for(w)
    cub = O.block_layout(w.cu_seqlens, w.block)
    bud = O.budgets_for(cub, w.sink_blocks, w.k_min, w.rho0, w.tau)
    offs, total = O.score_offsets(cub)
    np.testing.assert_array_equal(p.cu_blocks, cub)
    np.testing.assert_array_equal(p.budget, bud)
    np.testing.assert_array_equal(p.tri, offs)
    assert p.info.score_elems_per_head == total
    assert p.info.total_blocks == cub[-1]
    assert p.info.kmax == bud.max()
    assert p.info.executed_blocks_per_head == bud.sum()
    np.testing.assert_array_equal(p.blk_seq, np.repeat(np.arange(len(w.seqlens)), np.diff(cub)))
    assert sorted(p.order.tolist()) == list(range(int(cub[-1])))


@pytest.mark.parametrize("seed", range(20))
def test_plan_budget_random_parameters(seed):
    r = np.random.default_rng(seed)
    seqlens = list(r.integers(0, 3000, size=r.integers(1, 5)))
    block = int(r.choice([64, 128]))
    S = int(r.integers(0, 5))
    k_min = int(r.integers(0, 12))
    rho0 = float(r.choice([0.0, r.uniform(0, 2), 1.0, 0.5]))
    tau = float(r.choice([r.uniform(0.5, 300), 64.0, 1e9]))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    p = stem.stem_plan(cu, 4, 2, 64, block, "bf16", S, k_min, rho0, tau)
    cub = O.block_layout(cu, block)
    np.testing.assert_array_equal(p.budget, O.budgets_for(cub, S, k_min, rho0, tau))


@pytest.mark.parametrize("seed", range(20))
def test_plan_linear_budget_random_parameters(seed):
    r = np.random.default_rng(100 + seed)
    seqlens = list(r.integers(0, 4000, size=r.integers(1, 5)))
    block = int(r.choice([64, 128]))
    S = int(r.integers(0, 5))
    k_min = int(r.integers(0, 6))
    k_start = float(r.choice([r.uniform(0, 40), 16.0, 0.0, 7.5]))
    mu = float(r.choice([r.uniform(0, 1), 0.0, 1.0, 0.3]))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    p = stem.stem_plan(cu, 4, 2, 64, block, "bf16", S, k_min, 0.0, 1.0,
                       budget_mode="linear", k_start=k_start, mu=mu)
    cub = O.block_layout(cu, block)
    np.testing.assert_array_equal(
        p.budget, O.budgets_for(cub, S, k_min, 0.0, 1.0, "linear", k_start, mu))


@pytest.mark.parametrize("seed", range(20))
def test_plan_linear_fraction_budget_random_parameters(seed):
    r = np.random.default_rng(300 + seed)
    seqlens = list(r.integers(0, 4000, size=r.integers(1, 5)))
    block = int(r.choice([64, 128]))
    S = int(r.integers(0, 5))
    k_min = int(r.integers(0, 6))
    k_start = float(r.choice([r.uniform(0, 1), 0.25, 0.0, 1.0]))
    mu = float(r.choice([r.uniform(0, 1), 0.0, 1.0, 0.7]))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    p = stem.stem_plan(cu, 4, 2, 64, block, "bf16", S, k_min, 0.0, 1.0,
                       budget_mode="linear_fraction", k_start=k_start, mu=mu)
    cub = O.block_layout(cu, block)
    np.testing.assert_array_equal(
        p.budget, O.budgets_for(cub, S, k_min, 0.0, 1.0, "linear_fraction", k_start, mu))


def test_plan_carries_metric_mode_and_beta():
    for name, code in stem.METRICS.items():
        p = stem.stem_plan([0, 512], 2, 1, 64, 64, "f32", 1, 1, 0.5, 4.0, metric=name,
                           beta=0.25)
        assert p.info.metric_mode == code and p.info.beta == 0.25


def test_plan_ragged_and_empty_sequences():
    cu = [0, 0, 1, 1, 130, 130]
    p = stem.stem_plan(cu, 2, 1, 64, 64, "f32", 1, 1, 0.5, 4.0)
    assert list(p.cu_blocks) == [0, 0, 1, 1, 4, 4]
    assert p.info.total_tokens == 130
    assert list(p.blk_seq) == [1, 3, 3, 3]


def _status(fn, *args):
    with pytest.raises(stem.StemError) as e:
        fn(*args)
    return e.value.status


def test_plan_rejects_bad_arguments():
    ok = dict(cu_seqlens=[0, 128], num_q_heads=4, num_kv_heads=2, head_dim=64, block=64,
              dtype="bf16", sink_blocks=1, k_min=1, rho0=0.5, tau=4.0)

    def bad(**kw):
        a = dict(ok); a.update(kw)
        return _status(lambda: stem.stem_plan(**a))

    assert bad(num_kv_heads=3) == stem.STEM_EINVAL
    assert bad(num_q_heads=0) == stem.STEM_EINVAL
    assert bad(head_dim=96) == stem.STEM_EUNSUPPORTED
    assert bad(block=32) == stem.STEM_EUNSUPPORTED
    assert bad(dtype="f16") == stem.STEM_EUNSUPPORTED
    assert bad(cu_seqlens=[1, 128]) == stem.STEM_EINVAL
    assert bad(cu_seqlens=[0, 128, 64]) == stem.STEM_EINVAL
    assert bad(sink_blocks=-1) == stem.STEM_EINVAL
    assert bad(k_min=-1) == stem.STEM_EINVAL
    assert bad(rho0=-0.1) == stem.STEM_EINVAL
    assert bad(rho0=float("nan")) == stem.STEM_EINVAL
    assert bad(tau=0.0) == stem.STEM_EINVAL
    assert bad(tau=float("inf")) == stem.STEM_EINVAL
    assert bad(cu_seqlens=[0, 64 * 4097]) == stem.STEM_EUNSUPPORTED
    # the largest sequence is accepted; work items (Hq * blocks) must fit int32
    assert stem.stem_plan(**dict(ok, cu_seqlens=[0, 64 * 4096])).info.max_seq_blocks == 4096
    assert bad(cu_seqlens=[0, 64 * 4096], num_q_heads=2 ** 20, num_kv_heads=1) == stem.STEM_EUNSUPPORTED
    assert bad(budget_mode="cosine") == stem.STEM_EINVAL
    assert bad(metric="oam") == stem.STEM_EINVAL
    assert bad(metric="additive", beta=-1.0) == stem.STEM_EINVAL
    assert bad(beta=float("nan")) == stem.STEM_EINVAL
    assert bad(budget_mode="linear", k_start=-1.0) == stem.STEM_EINVAL
    assert bad(budget_mode="linear", k_start=float("inf")) == stem.STEM_EINVAL
    assert bad(budget_mode="linear", k_start=4.0, mu=1.5) == stem.STEM_EINVAL
    assert bad(budget_mode="linear", k_start=4.0, mu=float("nan")) == stem.STEM_EINVAL
    # a fraction of the causal blocks lies in [0, 1]
    assert bad(budget_mode="linear_fraction", k_start=1.5, mu=0.5) == stem.STEM_EINVAL
    assert bad(budget_mode="linear_fraction", k_start=-0.1, mu=0.5) == stem.STEM_EINVAL
    assert bad(budget_mode="linear_fraction", k_start=float("nan"), mu=0.5) == stem.STEM_EINVAL
    assert bad(budget_mode="linear_fraction", k_start=0.5, mu=2.0) == stem.STEM_EINVAL
    # the exponential parameters are not checked in linear mode, and vice versa
    assert stem.stem_plan(*dict(ok, tau=0.0).values(), budget_mode="linear", k_start=2.0,
                          mu=0.5).info.kmax >= 1


def test_plan_reports_small_buffer():
    L = stem.lib()
    cu = np.array([0, 1000], dtype=np.int32)
    pr = stem.stem_problem(1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, 1, 64, 64, 1)
    pa = stem.stem_params(1, 2, 0.5, 4.0)
    info = stem.stem_plan_info()
    assert L.stem_plan(ctypes.byref(pr), ctypes.byref(pa), ctypes.byref(info), None, 0) == 0
    buf = np.zeros(int(info.plan_bytes) - 1, dtype=np.uint8)
    assert L.stem_plan(ctypes.byref(pr), ctypes.byref(pa), ctypes.byref(info),
                       buf.ctypes.data, buf.nbytes) == stem.STEM_ESPACE


def test_device_calls_reject_bad_arguments_before_any_launch():
    # these return before touching the HIP runtime, so they run without a GPU
    L = stem.lib()
    p = stem.plan_for(syn.custom([256], 4, 2, 64, "bf16", 64))
    info = p.info
    P = 1 << 20  # a fake, 16-byte aligned address: never dereferenced
    assert L.stem_pool(None, P, P, P, P, P, P, P, 0, None) == stem.STEM_EINVAL
    assert L.stem_pool(ctypes.byref(info), None, P, P, P, P, P, P, 0, None) == stem.STEM_EINVAL
    assert L.stem_pool(ctypes.byref(info), P, None, P, P, P, P, P, 0, None) == stem.STEM_EINVAL
    assert L.stem_pool(ctypes.byref(info), P, P + 2, P, P, P, P, P, 0, None) == stem.STEM_EINVAL
    assert L.stem_pool(ctypes.byref(info), P, P, P, P, P, P, P, 7, None) == stem.STEM_EINVAL
    assert L.stem_score(ctypes.byref(info), P, P, P, P, None, None) == stem.STEM_EINVAL
    assert L.stem_select(ctypes.byref(info), P, P, P, None, None) == stem.STEM_EINVAL
    assert L.stem_sparse_attn(ctypes.byref(info), P, P, P, P, P, P, P, 5, None, None) == \
        stem.STEM_EUNSUPPORTED
    assert L.stem_sparse_attn(ctypes.byref(info), P, P, P, P, P, P, P + 4, 0, None, None) == \
        stem.STEM_EINVAL
    bad = stem.stem_plan_info.from_buffer_copy(info)
    bad.magic = 0
    assert L.stem_score(ctypes.byref(bad), P, P, P, P, P, None) == stem.STEM_EINVAL
    # a plan edited past the size limits is refused by every device call
    for field, value in [("max_seq_blocks", 5000), ("total_blocks", 1 << 30),
                         ("num_q_heads", 1 << 30)]:
        big = stem.stem_plan_info.from_buffer_copy(info)
        setattr(big, field, value)
        if field == "num_q_heads":
            big.num_kv_heads = 1
        assert L.stem_select(ctypes.byref(big), P, P, P, P, None) == stem.STEM_EUNSUPPORTED, field
        assert L.stem_sparse_attn(ctypes.byref(big), P, P, P, P, P, P, P, 0, None, None) == \
            stem.STEM_EUNSUPPORTED, field
    assert stem.status_str(stem.STEM_EUNSUPPORTED) == "unsupported configuration"


def test_antidiag_score_rejects_bad_arguments_before_any_launch():
    L = stem.lib()
    P = 1 << 20
    info = stem.plan_for(syn.custom([256], 4, 2, 64, "bf16", 64)).info
    A = L.stem_score_antidiag
    for stride in (0, -1, 3, 6, 128, 1 << 20):
        assert A(ctypes.byref(info), P, P, P, P, stride, P, None) == stem.STEM_EINVAL, stride
    assert A(ctypes.byref(info), P, None, P, P, 4, P, None) == stem.STEM_EINVAL
    assert A(ctypes.byref(info), P, P + 8, P, P, 4, P, None) == stem.STEM_EINVAL
    assert A(ctypes.byref(info), P, P, P, P + 2, 4, P, None) == stem.STEM_EINVAL
    f32 = stem.plan_for(syn.custom([256], 4, 2, 64, "f32", 64)).info
    assert A(ctypes.byref(f32), P, P, P, P, 3, P, None) == stem.STEM_EINVAL
    # stride 1 on the longest sequence with many heads exceeds the work bound
    big = stem.plan_for(syn.custom([64 * 4096], 1024, 1, 64, "bf16", 64)).info
    assert A(ctypes.byref(big), P, P, P, P, 1, P, None) == stem.STEM_EUNSUPPORTED
    # an empty problem is accepted without a launch
    empty = stem.plan_for(syn.custom([0], 4, 2, 64, "bf16", 64)).info
    assert A(ctypes.byref(empty), None, None, None, None, 4, None, None) == stem.STEM_OK

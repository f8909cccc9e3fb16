"""Host-code exercise of a sanitizer build of libstem (run by
test_host_sanitizer.py in a child process with the ASan runtime preloaded;
no GPU, no torch).  Every entry point is called through ctypes: the planner
on random and degenerate problems (its tables checked against the oracle),
and every device call with arguments that its host checks must reject
before any launch.  Exits non-zero on the first mismatch; the sanitizers
abort the process on any memory or undefined-behaviour error."""
import ctypes
import sys

import numpy as np

sys.path.insert(0, sys.argv[2])
from block_sparse_causal_amd import stem  # noqa: E402  (ctypes structures; no torch)
from oracle import stem_oracle as O  # noqa: E402

L = ctypes.CDLL(sys.argv[1])
for name, (res, args) in stem._SIGS.items():
    fn = getattr(L, name)
    fn.restype = res
    fn.argtypes = args


def plan(cu, Hq, Hkv, d, B, dtype, S, kmin, rho0, tau, mode=0, kstart=0.0, mu=0.0,
         metric=0, beta=0.2, capacity=None):
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    pr = stem.stem_problem(len(cu) - 1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                           Hq, Hkv, d, B, dtype)
    pa = stem.stem_params(S, kmin, rho0, tau, mode, metric, kstart, mu, beta)
    info = stem.stem_plan_info()
    rc = L.stem_plan(ctypes.byref(pr), ctypes.byref(pa), ctypes.byref(info), None, 0)
    if rc != 0:
        return rc, None, None
    cap = int(info.plan_bytes) if capacity is None else capacity
    blob = np.zeros(max(cap, 1), dtype=np.uint8)
    rc = L.stem_plan(ctypes.byref(pr), ctypes.byref(pa), ctypes.byref(info), blob.ctypes.data, cap)
    return rc, info, blob


def budget_of(info, blob):
    return np.frombuffer(blob, dtype=np.int32, count=int(info.total_blocks),
                         offset=int(info.off_budget))


rng = np.random.default_rng(7)
modes = {0: "exp", 1: "linear", 2: "linear_fraction"}
checked = 0
for t in range(60):
    seqlens = list(rng.integers(0, 3000, size=rng.integers(1, 6)))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    B = int(rng.choice([64, 128]))
    S, kmin = int(rng.integers(0, 5)), int(rng.integers(0, 6))
    mode = t % 3
    kstart = float(rng.uniform(0, 1)) if mode == 2 else float(rng.uniform(0, 30))
    mu = float(rng.uniform(0, 1))
    rho0, tau = float(rng.uniform(0, 2)), float(rng.uniform(0.5, 100))
    rc, info, blob = plan(cu, 4, 2, 128, B, 1, S, kmin, rho0, tau, mode, kstart, mu)
    assert rc == 0, (t, rc)
    want = O.budgets_for(O.block_layout(cu, B), S, kmin, rho0, tau, modes[mode], kstart, mu)
    assert np.array_equal(budget_of(info, blob), want), t
    checked += 1
    # a blob one byte too small is refused
    assert plan(cu, 4, 2, 128, B, 1, S, kmin, rho0, tau, mode, kstart, mu,
                capacity=int(info.plan_bytes) - 1)[0] == stem.STEM_ESPACE

# degenerate and invalid problems
assert plan([0], 1, 1, 64, 64, 0, 0, 0, 0.0, 1.0)[0] == stem.STEM_EINVAL       # no sequence
assert plan([0, 0, 0], 1, 1, 64, 64, 0, 0, 0, 0.0, 1.0)[0] == 0                # empty sequences
assert plan([0, 10], 3, 2, 64, 64, 0, 0, 0, 0.0, 1.0)[0] == stem.STEM_EINVAL   # GQA ratio
assert plan([0, 10], 2, 1, 96, 64, 0, 0, 0, 0.0, 1.0)[0] == stem.STEM_EUNSUPPORTED
assert plan([0, 64 * 4097], 1, 1, 64, 64, 1, 0, 0, 0.0, 1.0)[0] == stem.STEM_EUNSUPPORTED
assert plan([0, 100, 50], 1, 1, 64, 64, 0, 0, 0, 0.0, 1.0)[0] == stem.STEM_EINVAL
assert plan([0, 100], 1, 1, 64, 64, 0, 0, 0, float("nan"), 1.0)[0] == stem.STEM_EINVAL
assert plan([0, 100], 1, 1, 64, 64, 0, 0, 0, 1.0, 0.0)[0] == stem.STEM_EINVAL
assert plan([0, 100], 1, 1, 64, 64, 0, 0, 0, 1.0, 1.0, mode=2, kstart=1.5)[0] == stem.STEM_EINVAL
assert plan([0, 100], 1, 1, 64, 64, 0, 0, 0, 1.0, 1.0, metric=7)[0] == stem.STEM_EINVAL
assert plan([0, 100], 1, 1, 64, 64, 0, 0, 0, 1.0e300, 1.0e-300)[0] == 0        # huge decay terms
assert L.stem_plan(None, None, None, None, 0) == stem.STEM_EINVAL

# device calls: host checks only (nothing may be launched)
rc, info, blob = plan([0, 1000, 1077], 4, 2, 128, 64, 1, 2, 3, 0.5, 8.0)
assert rc == 0
dev = ctypes.c_void_p(4096)   # a 16-byte aligned address that is never dereferenced
odd = ctypes.c_void_p(4097)
I = ctypes.byref(info)
assert L.stem_pool(I, dev, None, dev, dev, dev, dev, dev, 0, None) == stem.STEM_EINVAL
assert L.stem_pool(I, dev, odd, dev, dev, dev, dev, dev, 0, None) == stem.STEM_EINVAL
assert L.stem_pool(I, dev, dev, dev, dev, dev, dev, dev, 5, None) == stem.STEM_EINVAL
assert L.stem_score(I, dev, None, dev, dev, dev, None) == stem.STEM_EINVAL
assert L.stem_score_antidiag(I, dev, dev, dev, dev, 3, dev, None) == stem.STEM_EINVAL
assert L.stem_score_antidiag(I, dev, dev, dev, dev, 0, dev, None) == stem.STEM_EINVAL
assert L.stem_select(I, dev, dev, None, dev, None) == stem.STEM_EINVAL
assert L.stem_sparse_attn(I, dev, dev, dev, dev, dev, dev, dev, 9, None, None) == \
    stem.STEM_EUNSUPPORTED
assert L.stem_sparse_attn(I, dev, dev, dev, dev, dev, dev, odd, 1, None, None) == stem.STEM_EINVAL
assert L.stem_sparse_attn(I, None, dev, dev, dev, dev, dev, dev, 1, None, None) == stem.STEM_EINVAL
bad = stem.stem_plan_info.from_buffer_copy(info)
bad.magic = 0
assert L.stem_pool(ctypes.byref(bad), dev, dev, dev, dev, dev, dev, dev, 0, None) == stem.STEM_EINVAL
bad = stem.stem_plan_info.from_buffer_copy(info)
bad.max_seq_blocks = 1 << 20
assert L.stem_select(ctypes.byref(bad), dev, dev, dev, dev, None) == stem.STEM_EUNSUPPORTED
# an empty problem launches nothing and succeeds
rc, einfo, _ = plan([0, 0], 2, 1, 64, 64, 1, 1, 1, 0.5, 8.0)
E = ctypes.byref(einfo)
assert L.stem_pool(E, None, None, None, None, None, None, None, 0, None) == 0
assert L.stem_sparse_attn(E, None, None, None, None, None, None, None, 1, None, None) == 0
sink = ctypes.c_double()
assert L.stem_probe_mfma(1, None, 0, ctypes.byref(sink), None) == stem.STEM_EINVAL
assert L.stem_probe_hbm_read(dev, 17, dev, 1, None) == stem.STEM_EINVAL
for code in range(-6, 2):
    assert L.stem_status_str(code)
print(f"sanitized ABI exercise ok ({checked} planner tables)", flush=True)

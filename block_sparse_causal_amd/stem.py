"""Python binding of libstem (the C ABI in include/stem.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (torch is used for device
memory and streams); functions carry the same names as the C entry points.
There is no fallback: if libstem.so is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstem.so")
_lib = None

STEM_OK, STEM_EINVAL, STEM_EUNSUPPORTED, STEM_EHIP, STEM_ESPACE = 0, -1, -2, -3, -4
STEM_F32, STEM_BF16 = 0, 1
STEM_VNORM_MEAN, STEM_VNORM_MAX = 0, 1
STEM_BUDGET_EXP, STEM_BUDGET_LINEAR, STEM_BUDGET_LINEAR_FRACTION = 0, 1, 2
STEM_METRIC_OUTPUT_AWARE, STEM_METRIC_ADDITIVE, STEM_METRIC_ROUTING = 0, 1, 2
BUDGET_MODES = {"exp": STEM_BUDGET_EXP, "linear": STEM_BUDGET_LINEAR,
                "linear_fraction": STEM_BUDGET_LINEAR_FRACTION}
METRICS = {"output_aware": STEM_METRIC_OUTPUT_AWARE, "additive": STEM_METRIC_ADDITIVE,
           "routing": STEM_METRIC_ROUTING}
STEM_PLAN_MAGIC = 0x5354454D

DTYPES = {"f32": STEM_F32, "bf16": STEM_BF16}


class StemError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_str(status)})")
        self.status = status


class stem_problem(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32),
                ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
                ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class stem_params(ctypes.Structure):
    _fields_ = [("sink_blocks", ctypes.c_int32),
                ("k_min", ctypes.c_int32),
                ("rho0", ctypes.c_double),
                ("tau", ctypes.c_double),
                ("budget_mode", ctypes.c_int32),
                ("metric_mode", ctypes.c_int32),
                ("k_start", ctypes.c_double),
                ("mu", ctypes.c_double),
                ("beta", ctypes.c_double)]


class stem_plan_info(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("sink_blocks", ctypes.c_int32),
                ("kmax", ctypes.c_int32),
                ("max_seq_blocks", ctypes.c_int32),
                ("metric_mode", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("beta", ctypes.c_double),
                ("total_tokens", ctypes.c_int64),
                ("total_blocks", ctypes.c_int64),
                ("score_elems_per_head", ctypes.c_int64),
                ("executed_blocks_per_head", ctypes.c_int64),
                ("plan_bytes", ctypes.c_int64),
                ("off_cu_seqlens", ctypes.c_int64),
                ("off_cu_blocks", ctypes.c_int64),
                ("off_tri", ctypes.c_int64),
                ("off_blk_seq", ctypes.c_int64),
                ("off_budget", ctypes.c_int64),
                ("off_order", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIGS = {
    "stem_plan": (ctypes.c_int, [ctypes.POINTER(stem_problem), ctypes.POINTER(stem_params),
                                 ctypes.POINTER(stem_plan_info), _P, ctypes.c_int64]),
    "stem_pool": (ctypes.c_int, [ctypes.POINTER(stem_plan_info), _P, _P, _P, _P, _P, _P, _P,
                                 ctypes.c_int32, _P]),
    "stem_score": (ctypes.c_int, [ctypes.POINTER(stem_plan_info), _P, _P, _P, _P, _P, _P]),
    "stem_select": (ctypes.c_int, [ctypes.POINTER(stem_plan_info), _P, _P, _P, _P, _P]),
    "stem_score_antidiag": (ctypes.c_int, [ctypes.POINTER(stem_plan_info), _P, _P, _P, _P,
                                           ctypes.c_int32, _P, _P]),
    "stem_sparse_attn": (ctypes.c_int, [ctypes.POINTER(stem_plan_info), _P, _P, _P, _P, _P, _P,
                                        _P, ctypes.c_int32, _P, _P]),
    "stem_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "stem_probe_mfma": (ctypes.c_int, [ctypes.c_int32, _P, ctypes.c_int64,
                                       ctypes.POINTER(ctypes.c_double), _P]),
    "stem_probe_hbm_read": (ctypes.c_int, [_P, ctypes.c_int64, _P, ctypes.c_int64, _P]),
}


def lib() -> ctypes.CDLL:
    """Load libstem.so (built in-tree by block_sparse_causal_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_causal_amd.build`")
        # torch first: its HIP libraries load their own copy of the HIP runtime
        # by the unversioned name, which libstem.so's versioned dependency then
        # resolves to.  Loaded the other way round, the process would hold two
        # runtimes, and torch's streams and allocations would be foreign to the
        # one the kernels are launched on.
        import torch  # noqa: F401
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().stem_status_str(int(status)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != STEM_OK:
        raise StemError(fn, rc)


# ---------------------------------------------------------------- planning


class Plan:
    """Result of stem_plan: the info struct, the host plan blob and (after
    ``to(device)``) its device copy."""

    def __init__(self, info: stem_plan_info, blob: np.ndarray):
        self.info = info
        self.blob = blob
        self.dev = None

    def to(self, device="cuda"):
        import torch
        if self.info.plan_bytes:
            self.dev = torch.from_numpy(self.blob).to(device)
        else:
            self.dev = torch.zeros(16, dtype=torch.uint8, device=device)
        return self

    def _array(self, off: int, n: int, dtype) -> np.ndarray:
        return np.frombuffer(self.blob, dtype=dtype, count=n, offset=off)

    @property
    def cu_blocks(self) -> np.ndarray:
        return self._array(self.info.off_cu_blocks, self.info.num_seqs + 1, np.int32)

    @property
    def tri(self) -> np.ndarray:
        return self._array(self.info.off_tri, self.info.num_seqs + 1, np.int64)

    @property
    def blk_seq(self) -> np.ndarray:
        return self._array(self.info.off_blk_seq, self.info.total_blocks, np.int32)

    @property
    def budget(self) -> np.ndarray:
        return self._array(self.info.off_budget, self.info.total_blocks, np.int32)

    @property
    def order(self) -> np.ndarray:
        return self._array(self.info.off_order, self.info.total_blocks, np.int32)

    @property
    def dev_ptr(self) -> int:
        if self.dev is None:
            raise RuntimeError("plan not uploaded: call plan.to(device) first")
        return self.dev.data_ptr()


def stem_plan(cu_seqlens: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
              block: int, dtype: str, sink_blocks: int, k_min: int, rho0: float,
              tau: float, budget_mode: str = "exp", k_start: float = 0.0, mu: float = 0.0,
              metric: str = "output_aware", beta: float = 0.2) -> Plan:
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    pr = stem_problem(len(cu) - 1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                      num_q_heads, num_kv_heads, head_dim, block, DTYPES.get(dtype, 99))
    pa = stem_params(sink_blocks, k_min, float(rho0), float(tau),
                     BUDGET_MODES.get(budget_mode, 99), METRICS.get(metric, 99),
                     float(k_start), float(mu), float(beta))
    info = stem_plan_info()
    L = lib()
    _check("stem_plan", L.stem_plan(ctypes.byref(pr), ctypes.byref(pa), ctypes.byref(info),
                                    None, 0))
    blob = np.zeros(max(int(info.plan_bytes), 16), dtype=np.uint8)
    _check("stem_plan", L.stem_plan(ctypes.byref(pr), ctypes.byref(pa), ctypes.byref(info),
                                    blob.ctypes.data, blob.nbytes))
    return Plan(info, blob)


def plan_for(workload, **override) -> Plan:
    """stem_plan for a synthetic.Workload (parameters may be overridden)."""
    w = workload.replace(**override) if override else workload
    return stem_plan(w.cu_seqlens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block,
                     w.dtype, w.sink_blocks, w.k_min, w.rho0, w.tau, w.budget_mode,
                     w.k_start, w.mu, w.metric, w.beta)


# ---------------------------------------------------------------- device calls


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, name, dtype, shape):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _io_dtype(plan: Plan):
    import torch
    return torch.bfloat16 if plan.info.dtype == STEM_BF16 else torch.float32


def stem_pool(plan: Plan, q, k, v, qbar, kbar, vnorm, vnorm_mode: int = STEM_VNORM_MEAN,
              stream=None) -> None:
    import torch
    i = plan.info
    T, Hq, Hkv, d, nbT = i.total_tokens, i.num_q_heads, i.num_kv_heads, i.head_dim, i.total_blocks
    dt = _io_dtype(plan)
    _need(q, "q", dt, (T, Hq, d)); _need(k, "k", dt, (T, Hkv, d)); _need(v, "v", dt, (T, Hkv, d))
    _need(qbar, "qbar", torch.float32, (Hq, nbT, d))
    _need(kbar, "kbar", torch.float32, (Hkv, nbT, d))
    _need(vnorm, "vnorm", torch.float32, (Hkv, nbT))
    _check("stem_pool", lib().stem_pool(ctypes.byref(i), plan.dev_ptr, q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), qbar.data_ptr(), kbar.data_ptr(),
                                        vnorm.data_ptr(), int(vnorm_mode), _stream(stream)))


def stem_score(plan: Plan, qbar, kbar, vnorm, scores, stream=None) -> None:
    import torch
    i = plan.info
    _need(qbar, "qbar", torch.float32, (i.num_q_heads, i.total_blocks, i.head_dim))
    _need(kbar, "kbar", torch.float32, (i.num_kv_heads, i.total_blocks, i.head_dim))
    _need(vnorm, "vnorm", torch.float32, (i.num_kv_heads, i.total_blocks))
    _need(scores, "scores", torch.float32, (i.num_q_heads, i.score_elems_per_head))
    _check("stem_score", lib().stem_score(ctypes.byref(i), plan.dev_ptr, qbar.data_ptr(),
                                          kbar.data_ptr(), vnorm.data_ptr(), scores.data_ptr(),
                                          _stream(stream)))


def stem_score_antidiag(plan: Plan, q, k, vnorm, stride: int, scores, stream=None) -> None:
    import torch
    i = plan.info
    dt = _io_dtype(plan)
    _need(q, "q", dt, (i.total_tokens, i.num_q_heads, i.head_dim))
    _need(k, "k", dt, (i.total_tokens, i.num_kv_heads, i.head_dim))
    _need(vnorm, "vnorm", torch.float32, (i.num_kv_heads, i.total_blocks))
    _need(scores, "scores", torch.float32, (i.num_q_heads, i.score_elems_per_head))
    _check("stem_score_antidiag",
           lib().stem_score_antidiag(ctypes.byref(i), plan.dev_ptr, q.data_ptr(), k.data_ptr(),
                                     vnorm.data_ptr(), int(stride), scores.data_ptr(),
                                     _stream(stream)))


def stem_select(plan: Plan, scores, idx, count, stream=None) -> None:
    import torch
    i = plan.info
    _need(scores, "scores", torch.float32, (i.num_q_heads, i.score_elems_per_head))
    _need(idx, "idx", torch.int32, (i.num_q_heads, i.total_blocks, i.kmax))
    _need(count, "count", torch.int32, (i.num_q_heads, i.total_blocks))
    _check("stem_select", lib().stem_select(ctypes.byref(i), plan.dev_ptr, scores.data_ptr(),
                                            idx.data_ptr(), count.data_ptr(), _stream(stream)))


def stem_sparse_attn(plan: Plan, q, k, v, idx, count, out, lse=None, stream=None) -> None:
    import torch
    i = plan.info
    T, Hq, Hkv, d = i.total_tokens, i.num_q_heads, i.num_kv_heads, i.head_dim
    dt = _io_dtype(plan)
    _need(q, "q", dt, (T, Hq, d)); _need(k, "k", dt, (T, Hkv, d)); _need(v, "v", dt, (T, Hkv, d))
    _need(idx, "idx", torch.int32, (Hq, i.total_blocks, idx.shape[2] if idx is not None else 0))
    if idx.shape[2] != i.kmax:
        raise ValueError(f"idx must have kmax={i.kmax} columns")
    _need(count, "count", torch.int32, (Hq, i.total_blocks))
    _need(out, "out", None, (T, Hq, d))
    if out.dtype == torch.float32:
        odt = STEM_F32
    elif out.dtype == torch.bfloat16:
        odt = STEM_BF16
    else:
        raise ValueError("out must be float32 or bfloat16")
    if lse is not None:
        _need(lse, "lse", torch.float32, (Hq, T))
    _check("stem_sparse_attn",
           lib().stem_sparse_attn(ctypes.byref(i), plan.dev_ptr, q.data_ptr(), k.data_ptr(),
                                  v.data_ptr(), idx.data_ptr(), count.data_ptr(), out.data_ptr(),
                                  odt, _ptr(lse), _stream(stream)))


def stem_probe_mfma(random_operands: bool, sink, stream=None) -> float:
    """Launch the matrix-core probe; returns the launch's flop count.  sink:
    float32 device tensor (4096 elements suffice)."""
    import torch
    _need(sink, "sink", torch.float32, (sink.numel(),))
    flops = ctypes.c_double()
    _check("stem_probe_mfma",
           lib().stem_probe_mfma(int(bool(random_operands)), sink.data_ptr(), sink.numel(),
                                 ctypes.byref(flops), _stream(stream)))
    return flops.value


def stem_probe_hbm_read(buf, sink, stream=None) -> int:
    """Launch the streaming-read probe over the bytes of the contiguous
    device tensor buf; returns the bytes read.  sink: int32 device tensor
    of at least ceil(bytes / 65536) elements (one per 64 KiB chunk)."""
    import torch
    _need(sink, "sink", torch.int32, (sink.numel(),))
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    _check("stem_probe_hbm_read",
           lib().stem_probe_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), sink.numel(),
                                     _stream(stream)))
    return nbytes


# ---------------------------------------------------------------- conveniences


class Buffers:
    """Every intermediate and output of one prefill, allocated once."""

    def __init__(self, plan: Plan, device="cuda", out_dtype=None):
        import torch
        i = plan.info
        f = dict(device=device, dtype=torch.float32)
        self.qbar = torch.empty((i.num_q_heads, i.total_blocks, i.head_dim), **f)
        self.kbar = torch.empty((i.num_kv_heads, i.total_blocks, i.head_dim), **f)
        self.vnorm = torch.empty((i.num_kv_heads, i.total_blocks), **f)
        self.scores = torch.empty((i.num_q_heads, i.score_elems_per_head), **f)
        self.idx = torch.empty((i.num_q_heads, i.total_blocks, max(i.kmax, 1)),
                               device=device, dtype=torch.int32)
        self.count = torch.empty((i.num_q_heads, i.total_blocks), device=device, dtype=torch.int32)
        odt = out_dtype if out_dtype is not None else _io_dtype(plan)
        self.out = torch.empty((i.total_tokens, i.num_q_heads, i.head_dim), device=device, dtype=odt)
        self.lse = torch.empty((i.num_q_heads, i.total_tokens), **f)


def prefill(plan: Plan, q, k, v, bufs: Optional[Buffers] = None, out_dtype=None,
            vnorm_mode: int = STEM_VNORM_MEAN, stream=None,
            score_stride: Optional[int] = None) -> Buffers:
    """pool -> score -> select -> sparse attention, all on the GPU.  With
    score_stride set, the metric comes from anti-diagonal samples of the
    token logits (stem_score_antidiag) instead of the pooled blocks."""
    if bufs is None:
        bufs = Buffers(plan, q.device, out_dtype)
    stem_pool(plan, q, k, v, bufs.qbar, bufs.kbar, bufs.vnorm, vnorm_mode, stream)
    if score_stride is None:
        stem_score(plan, bufs.qbar, bufs.kbar, bufs.vnorm, bufs.scores, stream)
    else:
        stem_score_antidiag(plan, q, k, bufs.vnorm, score_stride, bufs.scores, stream)
    stem_select(plan, bufs.scores, bufs.idx, bufs.count, stream)
    stem_sparse_attn(plan, q, k, v, bufs.idx, bufs.count, bufs.out, bufs.lse, stream)
    return bufs

"""Seeded synthetic prefill inputs (Q, K, V) for the Stem sparse-prefill path.

This module only draws and shapes input tensors.  It contains none of the
method's arithmetic (no pooling, scoring, budgeting, selection or attention),
so both the GPU path and the CPU oracle can consume what it produces without
sharing any of the method's code.

Recipe (the same for every workload):
  * Q[t, h, :] ~ N(0, I_d) and K[t, g, :] ~ N(0, I_d), float32 draws from
    NumPy's PCG64 ``default_rng(seed)``;
  * rotary position embedding applied to Q and K when a RoPE base is given:
    rotate-half pairing (element k with element k + d/2), inverse frequency
    base**(-2k/d), position = token index *within its own sequence*;
  * the first 4 tokens of every sequence have K multiplied by 3 (attention
    sinks; scaling commutes with the rotation);
  * V[t, g, :] = z * s with z ~ N(0, I_d) and one s ~ LogNormal(0, 0.5)
    (sigma of the underlying normal) per (token, KV head);
  * bf16 workloads round every value to bfloat16 with round-to-nearest-even
    on the host, and both paths read those exact values.

Draw order is fixed: Q, then K, then z, then s, each over the whole packed
token range, so a workload is reproducible from its seed alone.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

SINK_TOKENS_SCALED = 4
SINK_K_SCALE = 3.0
V_LOGNORMAL_SIGMA = 0.5


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, dtype and Stem parameters of one prefill layer."""

    name: str
    seqlens: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    rope_theta: Optional[float]
    block: int
    sink_blocks: int
    k_min: int
    rho0: float
    tau: float            # decay length, in blocks
    seed: int = 0
    budget_mode: str = "exp"          # "exp" (rho0, tau), "linear" or "linear_fraction" (k_start, mu)
    k_start: float = 0.0              # linear budget: dynamic blocks at the first row
    mu: float = 0.0                   # linear budget: k_end / k_start
    metric: str = "output_aware"      # "output_aware", "additive" or "routing"
    beta: float = 0.2                 # additive metric weight (the pages' value)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of this path.  Seeds are 1000 + position in this list.
WORKLOADS = {
    "single-head-1k-fp32": Workload(
        "single-head-1k-fp32", (1024,), 1, 1, 64, "f32", None,
        block=64, sink_blocks=1, k_min=2, rho0=1.0, tau=4.0, seed=1001),
    "llama3-8b-32k-b64": Workload(
        "llama3-8b-32k-b64", (32768,), 32, 8, 128, "bf16", 5.0e5,
        block=64, sink_blocks=2, k_min=8, rho0=0.5, tau=64.0, seed=1002),
    "llama3-8b-128k-b128": Workload(
        "llama3-8b-128k-b128", (131072,), 32, 8, 128, "bf16", 5.0e5,
        block=128, sink_blocks=2, k_min=16, rho0=0.3, tau=128.0, seed=1003),
    "qwen2.5-7b-64k-b64": Workload(
        "qwen2.5-7b-64k-b64", (65536,), 28, 4, 128, "bf16", 1.0e6,
        block=64, sink_blocks=4, k_min=8, rho0=0.25, tau=256.0, seed=1004),
    "llama3-8b-varlen-120k-b64": Workload(
        "llama3-8b-varlen-120k-b64", (8192, 16384, 32768, 65536), 32, 8, 128,
        "bf16", 5.0e5, block=64, sink_blocks=2, k_min=8, rho0=0.4, tau=128.0,
        seed=1005),
}

HEADLINE = "llama3-8b-128k-b128"


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Inputs here are finite; NaN/Inf are not produced by the generator."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _rope_tables(positions: np.ndarray, d: int, theta: float):
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _apply_rope_inplace(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> None:
    """x: [n, H, d] float32; cos/sin: [n, d/2]."""
    half = x.shape[-1] // 2
    c = cos[:, None, :]
    s = sin[:, None, :]
    x1 = x[..., :half].copy()
    x2 = x[..., half:]
    x[..., :half] = x1 * c - x2 * s
    x[..., half:] = x2 * c + x1 * s


def positions_of(seqlens) -> np.ndarray:
    return np.concatenate([np.arange(n, dtype=np.int64) for n in seqlens]) \
        if len(seqlens) else np.zeros(0, dtype=np.int64)


@dataclasses.dataclass
class Inputs:
    """Generated tensors.  ``q``, ``k``, ``v`` are float32 arrays holding the
    exact values both paths consume; for bf16 workloads ``*_bits`` hold the
    bfloat16 patterns to upload (uint16, same shapes)."""

    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None


def generate(w: Workload, seed: Optional[int] = None, chunk: int = 8192) -> Inputs:
    """Draw Q, K, V for workload ``w`` (seed defaults to ``w.seed``)."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    T, Hq, Hkv, d = w.total_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim
    q = rng.standard_normal((T, Hq, d), dtype=np.float32)
    k = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    s = rng.lognormal(0.0, V_LOGNORMAL_SIGMA, size=(T, Hkv)).astype(np.float32)
    v *= s[:, :, None]

    cu = w.cu_seqlens
    if w.rope_theta is not None:
        pos = positions_of(w.seqlens)
        for a in range(0, T, chunk):
            b = min(T, a + chunk)
            cos, sin = _rope_tables(pos[a:b], d, w.rope_theta)
            _apply_rope_inplace(q[a:b], cos, sin)
            _apply_rope_inplace(k[a:b], cos, sin)
    for si in range(len(w.seqlens)):
        a = int(cu[si])
        n = min(SINK_TOKENS_SCALED, int(w.seqlens[si]))
        k[a:a + n] *= np.float32(SINK_K_SCALE)

    if w.dtype == "bf16":
        out = Inputs(w, q, k, v)
        for name in ("q", "k", "v"):
            x = getattr(out, name)
            bits = np.empty(x.shape, dtype=np.uint16)
            flat_x = x.reshape(-1)
            flat_b = bits.reshape(-1)
            step = 1 << 24
            for a in range(0, flat_x.size, step):
                flat_b[a:a + step] = bf16_bits(flat_x[a:a + step])
                flat_x[a:a + step] = bf16_bits_to_f32(flat_b[a:a + step])
            setattr(out, name + "_bits", bits)
        return out
    if w.dtype != "f32":
        raise ValueError(f"unsupported dtype {w.dtype}")
    return Inputs(w, q, k, v)


def custom(seqlens: List[int], num_q_heads: int, num_kv_heads: int,
           head_dim: int, dtype: str, block: int, *, sink_blocks: int = 2,
           k_min: int = 4, rho0: float = 0.5, tau: float = 8.0,
           rope_theta: Optional[float] = 5.0e5, seed: int = 7,
           name: str = "custom", **params) -> Workload:
    """A small workload of the same distribution, for tests (``params`` sets
    budget_mode, k_start, mu, metric or beta)."""
    return Workload(name, tuple(int(x) for x in seqlens), num_q_heads,
                    num_kv_heads, head_dim, dtype, rope_theta, block,
                    sink_blocks, k_min, float(rho0), float(tau), seed, **params)


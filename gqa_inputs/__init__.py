"""Seeded synthetic inputs for GroupQueryAttention over a shared-buffer KV cache.

This module only draws numbers and lays them out. It holds none of the
attention method's arithmetic, so both the fp64 CPU oracle and the HIP path
can consume its output without sharing any computation.

Everything is returned as raw bit patterns in numpy arrays (uint32 for fp32,
uint16 for fp16 and bf16) so that cache contents, including NaN poison with a
payload, survive round trips bit for bit.

Workloads (by name; the seed of each is fixed):
  worked-example            fp32 prefill-then-decode example (prompt 32, head
                            size 8, buffer 64); the prefill/decode GEMM shapes
                            come from the worked example of the rocMLIR
                            "KV Cache" discussion.
  split-kv-decode-fp16      B=16, H=32, Hkv=8, D=128, M=4096, past lengths
                            U{512..4095}.
  causal-prefill-bf16       B=4, H=32, Hkv=8, D=128, S=2048, rotary theta=1e4.
  ragged-continuation-fp16  B=8, H=28, Hkv=4, D=128, S=128, past U{0..3072}.
  window-decode-bf16        B=8, H=32, Hkv=8, D=128, M=W=4096, full cache.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")

# NaN with a payload, written into every cache slot past the valid length.
POISON = {"fp32": np.uint32(0x7FC00ABC), "fp16": np.uint16(0x7E5A), "bf16": np.uint16(0x7FC5)}


def bits_dtype(dtype: str):
    return np.uint32 if dtype == "fp32" else np.uint16


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws to the storage dtype (nearest-even) and return bits.

    Used only to materialise synthetic values; bf16 goes through fp32 first.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp32":
        return x.astype(np.float32).view(np.uint32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    raise ValueError(dtype)


def rope_tables(rows: int, half_dim: int, theta: float = 10000.0):
    """cos/sin tables [rows, half_dim] for rotary embedding, computed in fp64
    and rounded once to fp32. The op takes them as inputs (like the ONNX
    op's cos_cache/sin_cache), so both sides read exactly these numbers."""
    d = 2 * half_dim
    inv = theta ** (-(2.0 * np.arange(half_dim, dtype=np.float64)) / d)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclasses.dataclass
class Case:
    """One call's worth of inputs (bits) plus its shape and options."""
    name: str
    dtype: str
    batch: int
    new_tokens: int
    num_heads: int
    kv_num_heads: int
    head_size: int
    max_seq_len: int
    seqlens_k: np.ndarray                 # int32 [B] past lengths
    q: np.ndarray                         # bits [B, S, H*D]
    k_new: np.ndarray                     # bits [B, S, Hkv*D]
    v_new: np.ndarray                     # bits [B, S, Hkv*D]
    k_cache: np.ndarray                   # bits [B, Hkv, M, D]
    v_cache: np.ndarray                   # bits [B, Hkv, M, D]
    scale: float = 0.0                    # 0 -> 1/sqrt(D)
    local_window_size: int = -1
    cos: Optional[np.ndarray] = None      # fp32 [P, D/2] or None
    sin: Optional[np.ndarray] = None
    rotary_interleaved: int = 0
    greedy_eviction: int = 0              # 1: evict only on overflow, keep the latest W
    attention_bias: Optional[np.ndarray] = None   # bits [B or 1, H or 1, S, T] or None
    position_offset: Optional[np.ndarray] = None  # int32 [B]: absolute position of buffer row 0
    seed: int = 0
    extra: dict = dataclasses.field(default_factory=dict)

    def copy(self) -> "Case":
        c = dataclasses.replace(self)
        for f in ("seqlens_k", "q", "k_new", "v_new", "k_cache", "v_cache"):
            setattr(c, f, getattr(self, f).copy())
        if self.position_offset is not None:
            c.position_offset = self.position_offset.copy()
        c.extra = dict(self.extra)
        return c


def _normal_bits(rng, shape, dtype):
    return to_bits(rng.standard_normal(shape), dtype)


def fill_cache(rng, B, Hkv, M, D, lens, dtype, valid=None):
    """A [B, Hkv, M, D] cache: N(0,1) in rows [0, valid_b), poison after."""
    bits = _normal_bits(rng, (B, Hkv, M, D), dtype)
    valid = lens if valid is None else valid
    rows = np.arange(M)[None, :]
    dead = rows >= np.asarray(valid, dtype=np.int64)[:, None]          # [B, M]
    bits[np.broadcast_to(dead[:, None, :, None], bits.shape)] = POISON[dtype]
    return bits


def make_case(name, dtype, B, S, H, Hkv, D, M, lens, seed, *, window=-1,
              rotary=False, theta=10000.0, rotary_rows=None, interleaved=0,
              scale=0.0, rng=None, extra=None) -> Case:
    """Draw order: (lengths are given) Q, K_new, V_new, then cache contents."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = np.asarray(lens, dtype=np.int32)
    q = _normal_bits(rng, (B, S, H * D), dtype)
    k_new = _normal_bits(rng, (B, S, Hkv * D), dtype)
    v_new = _normal_bits(rng, (B, S, Hkv * D), dtype)
    k_cache = fill_cache(rng, B, Hkv, M, D, lens, dtype)
    v_cache = fill_cache(rng, B, Hkv, M, D, lens, dtype)
    cos = sin = None
    if rotary:
        P = rotary_rows if rotary_rows is not None else max(M, int(lens.max(initial=0)) + S)
        cos, sin = rope_tables(P, D // 2, theta)
    return Case(name, dtype, B, S, H, Hkv, D, M, lens, q, k_new, v_new, k_cache, v_cache,
                scale=scale, local_window_size=window, cos=cos, sin=sin,
                rotary_interleaved=interleaved, seed=seed, extra=dict(extra or {}))


def _uniform_int(rng, lo, hi, n):
    # inclusive at both ends
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


WORKLOAD_SEEDS = {
    "worked-example": 1,
    "split-kv-decode-fp16": 2,
    "causal-prefill-bf16": 3,
    "ragged-continuation-fp16": 4,
    "window-decode-bf16": 5,
}


def workload(name: str, step: int = 1, seed: Optional[int] = None) -> Case:
    """One of the named workloads; seed defaults to the workload's own.

    The worked example has two steps: step 1 is the 32-token prefill from an
    empty cache and step 2 the one-token decode at past length 32 (to chain
    step 2 onto the cache a real step 1 produced, replace its caches)."""
    if name not in WORKLOAD_SEEDS:
        raise ValueError(f"unknown workload {name!r}; known: {sorted(WORKLOAD_SEEDS)}")
    seed = WORKLOAD_SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "worked-example":
        if step == 1:
            return make_case("worked-example-prefill", "fp32", 1, 32, 4, 2, 8, 64, [0], seed,
                             scale=1.0 / math.sqrt(8.0), rng=rng)
        return make_case("worked-example-decode", "fp32", 1, 1, 4, 2, 8, 64, [32], seed,
                         scale=1.0 / math.sqrt(8.0), rng=rng)
    if name == "split-kv-decode-fp16":
        lens = _uniform_int(rng, 512, 4095, 16)
        return make_case(name, "fp16", 16, 1, 32, 8, 128, 4096, lens, seed, rng=rng)
    if name == "causal-prefill-bf16":
        lens = np.zeros(4, np.int32)
        return make_case(name, "bf16", 4, 2048, 32, 8, 128, 4096, lens, seed,
                         rotary=True, theta=10000.0, rotary_rows=4096, rng=rng)
    if name == "ragged-continuation-fp16":
        lens = _uniform_int(rng, 0, 3072, 8)
        return make_case(name, "fp16", 8, 128, 28, 4, 128, 4096, lens, seed, rng=rng)
    totals = _uniform_int(rng, 4096, 16384, 8)
    lens = np.full(8, 4096, np.int32)
    return make_case(name, "bf16", 8, 1, 32, 8, 128, 4096, lens, seed,
                     window=4096, rng=rng, extra={"total_lengths": totals})


def next_decode_tokens(case: Case, rng) -> Case:
    """Same cache, fresh one-token Q/K/V (for rolling decode steps)."""
    c = case.copy()
    B, H, Hkv, D = c.batch, c.num_heads, c.kv_num_heads, c.head_size
    c.new_tokens = 1
    c.q = _normal_bits(rng, (B, 1, H * D), c.dtype)
    c.k_new = _normal_bits(rng, (B, 1, Hkv * D), c.dtype)
    c.v_new = _normal_bits(rng, (B, 1, Hkv * D), c.dtype)
    return c

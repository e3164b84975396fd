"""Shared plumbing for the GPU parity tests: move seeded bit arrays to the GPU,
call the library through its binding, and bring results back as bits/fp64."""
from __future__ import annotations

import numpy as np

from oracle import gqa_oracle as O

TOL = {"fp32": 1e-4, "fp16": 2e-2, "bf16": 2e-2}


def torch_dtype(dtype):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_dev(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    signed = bits.view(np.int32 if bits.dtype == np.uint32 else np.int16)
    return torch.from_numpy(np.ascontiguousarray(signed)).to(device).view(torch_dtype(dtype))


def to_bits(t) -> np.ndarray:
    import torch
    if t.dtype == torch.float32:
        return t.detach().view(torch.int32).cpu().numpy().view(np.uint32)
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class DevCase:
    """A Case's tensors on the GPU."""

    def __init__(self, case, device="cuda"):
        import torch
        self.case = case
        dt = case.dtype
        self.q = to_dev(case.q, dt, device)
        self.k_new = to_dev(case.k_new, dt, device)
        self.v_new = to_dev(case.v_new, dt, device)
        self.k_cache = to_dev(case.k_cache, dt, device)
        self.v_cache = to_dev(case.v_cache, dt, device)
        self.lens_host = np.asarray(case.seqlens_k, np.int32).copy()
        self.lens_dev = torch.from_numpy(self.lens_host.copy()).to(device)
        self.bias = None
        if getattr(case, "attention_bias", None) is not None:
            self.bias = to_dev(case.attention_bias, dt, device)
        self.off_host = self.off_dev = None
        if getattr(case, "position_offset", None) is not None:
            self.off_host = np.asarray(case.position_offset, np.int32).copy()
            self.off_dev = torch.from_numpy(self.off_host.copy()).to(device)
        self.cos = self.sin = None
        if case.cos is not None:
            self.cos = torch.from_numpy(case.cos).to(device)
            self.sin = torch.from_numpy(case.sin).to(device)

    def set_lengths(self, lens):
        import torch
        self.lens_host = np.asarray(lens, np.int32).copy()
        self.lens_dev = torch.from_numpy(self.lens_host.copy()).to(self.k_cache.device)

    def set_offsets(self, offsets):
        import torch
        self.off_host = np.asarray(offsets, np.int32).copy()
        self.off_dev = torch.from_numpy(self.off_host.copy()).to(self.k_cache.device)

    def run(self, entry="prefill", out=None, workspace=None):
        import grouped_query_kv_amd as gqa
        c = self.case
        fn = gqa.gqa_attention_decode if entry == "decode" else gqa.gqa_attention_prefill
        return fn(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache, self.lens_host,
                  self.lens_dev, out, scale=c.scale, local_window_size=c.local_window_size,
                  cos_cache=self.cos, sin_cache=self.sin, rotary_interleaved=c.rotary_interleaved,
                  workspace=workspace, greedy_eviction=bool(c.greedy_eviction),
                  attention_bias=self.bias, position_offset=self.off_host,
                  position_offset_dev=self.off_dev)

    def append(self):
        import grouped_query_kv_amd as gqa
        c = self.case
        gqa.gqa_append_kv(self.k_new, self.v_new, self.k_cache, self.v_cache, self.lens_host,
                          self.lens_dev, cos_cache=self.cos, sin_cache=self.sin,
                          rotary_interleaved=c.rotary_interleaved, position_offset=self.off_host,
                          position_offset_dev=self.off_dev)

    def caches(self):
        return to_bits(self.k_cache), to_bits(self.v_cache)


def out_f64(t, dtype) -> np.ndarray:
    return O.to_f64(to_bits(t), dtype)


def assert_close(got: np.ndarray, want: np.ndarray, dtype: str, what=""):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= TOL[dtype], f"{what}: max abs error {worst:.3e} > {TOL[dtype]:.0e}"
    return worst


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what=""):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} elements differ, first at {tuple(bad[0])}: "
                             f"got {got[tuple(bad[0])]:#x}, want {want[tuple(bad[0])]:#x}")

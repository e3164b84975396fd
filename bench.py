#!/usr/bin/env python3
"""Throughput of GroupQueryAttention over a shared KV buffer on one MI355X.

Prints ONE JSON line. The headline step is the fp16 split-KV decode
(B=16, H=32, Hkv=8, D=128, M=4096, past lengths U{512..4095}, seed 2):
`value` is its algorithmic HBM bytes per step / wall time per step (GB/s).
The same line carries the bf16 causal prefill (B=4, H=32, Hkv=8, D=128,
S=2048, rotary; TFLOP/s over causal pairs), the fp16 ragged continuation
(B=8, H=28, Hkv=4, S=128) and the bf16 sliding-window decode (B=8, M=W=4096,
cache full, evict one row per step), each with its roofline fraction, then
the secondary legs (windowed chunks, separate past/present, greedy eviction,
attention bias, and the decode and causal prefill at head size 64).

Timing: inputs are resident in HBM before the timed region; each step rotates
over enough independent input sets (>= 1 GiB) that the 256 MB Infinity Cache
cannot serve repeated reads. Wall time over K back-to-back steps
(synchronised on both sides) gives ms_per_step and `value`; a second pass of
the same K steps between one pair of HIP events on the launch stream, queued
behind a spin kernel so that the device runs the calls back to back, gives
the device time per call used for the roofline fraction.

The CPU baseline times the fp64 oracle (as it stands) on a bounded sample of
the decode workload on this host's cores.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, 2.5 PFLOP/s
METRIC = "decode attn HBM GB/s + prefill TFLOP/s (fraction of MI355X peak), 1 GPU"
# HBM traffic of the decode kernel on the headline workload, per dispatch, from
# two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),
# each scaled by what the same counter reads for a plain 512 MiB device-to-device
# copy: FETCH_SIZE reads 262157 KiB for 524288 KiB moved (x2.0), WRITE_SIZE reads
# 524288 KiB (x1.0). Valid only for the kernel sources the counters were taken
# on; any change to them makes the figure null until the passes are repeated.
DECODE_TRAFFIC = {
    "sources": {"grouped_query_kv_amd/csrc/decode.hip":
                "bd13273628e645f22c93f0a05b9da027d612a8adf8e743e40b7862c819c56b2a",
                "grouped_query_kv_amd/csrc/gqa_internal.h":
                "4b62ef6cda1715062c2911657a2c20031b59281584c6ee04135249d3f3439172"},
    "fetch_kib": 73715.043, "write_kib": 1050.310,
    "fetch_scale": 524288.0 / 262157.088, "write_scale": 1.0,
}
POISON16 = {"fp16": 0x7E5A, "bf16": 0x7FC5}
MIN_ROTATION_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# input sets
# ----------------------------------------------------------------------------

class DevSet:
    """One independent set of device inputs for a case (same lengths)."""

    def __init__(self, case, seed, torch, canonical=False):
        import gpu_helpers as H
        dt = H.torch_dtype(case.dtype)
        self.case = case
        if canonical:
            d = H.DevCase(case)
            self.q, self.k_new, self.v_new = d.q, d.k_new, d.v_new
            self.k_cache, self.v_cache = d.k_cache, d.v_cache
            self.cos, self.sin = d.cos, d.sin
        else:
            g = torch.Generator(device="cuda").manual_seed(seed)

            def rnd(shape):
                return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dt)

            B, S, H_, Hkv, D, M = (case.batch, case.new_tokens, case.num_heads, case.kv_num_heads,
                                   case.head_size, case.max_seq_len)
            self.q, self.k_new, self.v_new = rnd((B, S, H_ * D)), rnd((B, S, Hkv * D)), rnd((B, S, Hkv * D))
            self.k_cache, self.v_cache = rnd((B, Hkv, M, D)), rnd((B, Hkv, M, D))
            lens = torch.as_tensor(case.seqlens_k, device="cuda").long()
            dead = torch.arange(M, device="cuda")[None, :] >= lens[:, None]
            for c in (self.k_cache, self.v_cache):
                c.view(torch.int16)[dead[:, None, :, None].expand_as(c)] = np.int16(
                    np.uint16(POISON16[case.dtype]).view(np.int16))
            self.cos = self.sin = None
            if case.cos is not None:
                self.cos = torch.from_numpy(case.cos).cuda()
                self.sin = torch.from_numpy(case.sin).cuda()
        self.lens_host = np.asarray(case.seqlens_k, np.int32).copy()
        self.lens_dev = torch.from_numpy(self.lens_host.copy()).cuda()
        self.out = torch.empty_like(self.q)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in (self.q, self.k_new, self.v_new,
                                                           self.k_cache, self.v_cache))


def make_sets(case, torch, base_seed):
    first = DevSet(case, base_seed, torch, canonical=True)
    n = max(4, math.ceil(MIN_ROTATION_BYTES / first.nbytes()))
    return [first] + [DevSet(case, base_seed * 1000 + i, torch) for i in range(1, n)]


# ----------------------------------------------------------------------------
# algorithmic work (what the method must move or compute per call)
# ----------------------------------------------------------------------------

def decode_bytes(case, lens_attended, window=-1):
    """K and V rows attended (incl. the new token), new rows written, Q read, O written."""
    e = 4 if case.dtype == "fp32" else 2
    B, H, Hkv, D = case.batch, case.num_heads, case.kv_num_heads, case.head_size
    rows = 0
    for L in lens_attended:
        n = L + 1 if window <= 0 else min(L + 1, window)
        rows += n
    return rows * Hkv * D * e * 2 + B * Hkv * D * e * 2 + 2 * B * H * D * e


def prefill_flops(case):
    """4*D flops (QK^T and PV) per visible (query, key) pair."""
    S, D, H = case.new_tokens, case.head_size, case.num_heads
    W = case.local_window_size
    pairs = 0
    for L in case.seqlens_k:
        L = int(L)
        for i in range(S):
            p = L + i
            lo = max(0, p - W + 1) if W > 0 else 0
            pairs += p - lo + 1
    return 4.0 * D * pairs * H


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------

def time_calls(torch, sets, call, steps, warmup):
    """Warmup, then three passes of `steps` calls rotating over the input sets.

    Pass 1 (the timed region): barrier + synchronize, the calls back to back,
    synchronize; gives the wall ms per step. Pass 2: one pair of HIP events
    on the launch stream around the same calls back to back, queued behind a
    spin kernel that outlasts the host's enqueue time, so the device runs
    them without gaps from the host; gives the device ms per call the
    roofline uses (the figure a kernel trace reports, plus the few hundred
    ns between dispatches). Pass 3: an event pair around each call, for the
    spread (each pair adds its own dispatch overhead).
    Returns (wall ms per step, device ms per call, per-call event ms list).
    """
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        call(sets[i % len(sets)])
    torch.cuda.synchronize()
    gc_was = gc.isenabled()
    gc.disable()                 # no collector pause inside the timed region
    t0 = time.perf_counter()
    for i in range(steps):
        call(sets[(warmup + i) % len(sets)])
    enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    log(f"[bench]   wall {wall:.4f} ms/step, host enqueue {enq * 1e3 / steps:.4f} ms/step")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(spin_cycles(torch, 2.0 * enq + 2e-3))
    e0.record(stream)
    for i in range(steps):
        call(sets[(warmup + i) % len(sets)])
    e1.record(stream)
    torch.cuda.synchronize()
    dev = e0.elapsed_time(e1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda._sleep(spin_cycles(torch, 2.0 * enq + 2e-3))
    for i in range(steps):
        ev[i][0].record(stream)
        call(sets[(warmup + i) % len(sets)])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    if gc_was:
        gc.enable()
    per = [x.elapsed_time(y) for x, y in ev]
    return wall, dev, per


_SPIN_RATE = []


def spin_cycles(torch, seconds):
    """Argument for torch.cuda._sleep that spins about `seconds` (rate measured once)."""
    if not _SPIN_RATE:
        n = 1 << 20
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(n)
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        _SPIN_RATE.append(n / max(a.elapsed_time(b) * 1e-3, 1e-6))
    return int(min(seconds, 1.0) * _SPIN_RATE[0]) + 1


def decode_traffic_bytes():
    """Counter-derived HBM bytes per decode dispatch, or None if the kernel changed."""
    import hashlib
    for rel, digest in DECODE_TRAFFIC["sources"].items():
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    t = DECODE_TRAFFIC
    return int(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]))


def stats(dev, per):
    a = np.sort(np.asarray(per))
    return {"mean_ms": float(dev), "per_call_event_median_ms": float(np.median(a)),
            "per_call_event_p10_ms": float(a[int(0.1 * (len(a) - 1))]),
            "per_call_event_p90_ms": float(a[int(0.9 * (len(a) - 1))])}


def read_yardstick(torch, gqa, nbytes, steps, warmup, decode_ms):
    """A plain streaming read (gqa_stream_read, the decode's launch shape) of
    the decode's byte count, rotating over buffers that together exceed the
    last-level cache like the decode's input sets: the time any kernel that
    reads those bytes once can reach here, and the decode's time against it."""
    nbytes16 = (nbytes + 15) // 16 * 16
    n = max(4, math.ceil(MIN_ROTATION_BYTES / nbytes16))
    bufs = [torch.ones(nbytes16, dtype=torch.uint8, device="cuda") for _ in range(n)]
    log(f"[bench] read yardstick: {n} buffers of {nbytes16} bytes")
    _, dev, per = time_calls(torch, bufs, lambda b: gqa.gqa_stream_read(b), steps, warmup)
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes16, "us": dev * 1e3, "gbs": nbytes16 / (dev * 1e-3) / 1e9,
            "frac_hbm_peak": nbytes16 / (dev * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "decode_time_over_read_time": decode_ms / dev,
            "per_call_event_median_us": float(np.median(per)) * 1e3}


def decode_call(gqa):
    def call(s):
        c = s.case
        gqa.gqa_attention_decode(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.lens_host, s.lens_dev,
                                 s.out, scale=c.scale, local_window_size=c.local_window_size,
                                 cos_cache=s.cos, sin_cache=s.sin)
    return call


def biased_call(gqa):
    """Either entry with the set's additive bias (`s.bias`)."""
    def call(s):
        c = s.case
        gqa.gqa_attention_prefill(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.lens_host, s.lens_dev,
                                  s.out, scale=c.scale, local_window_size=c.local_window_size,
                                  cos_cache=s.cos, sin_cache=s.sin, attention_bias=s.bias)
    return call


def prefill_call(gqa):
    def call(s):
        c = s.case
        gqa.gqa_attention_prefill(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.lens_host, s.lens_dev,
                                  s.out, scale=c.scale, local_window_size=c.local_window_size,
                                  cos_cache=s.cos, sin_cache=s.sin,
                                  rotary_interleaved=c.rotary_interleaved,
                                  greedy_eviction=bool(c.greedy_eviction))
    return call


def present_call(gqa):
    """Separate past (the set's caches) and present buffers."""
    def call(s):
        c = s.case
        gqa.gqa_attention_prefill(s.q, s.k_new, s.v_new, s.k_cache, s.v_cache, s.lens_host, s.lens_dev,
                                  s.out, scale=c.scale, local_window_size=c.local_window_size,
                                  present_key=s.present_k, present_value=s.present_v)
    return call


def run_leg(torch, name, case, call, steps, warmup, prepare=None):
    log(f"[bench] {name} sets: building")
    sets = make_sets(case, torch, case.seed or 7)
    for x in sets:
        if prepare:
            prepare(x)
    log(f"[bench] {name}: {len(sets)} input sets, timing {steps} steps")
    w, d, p_ = time_calls(torch, sets, call, steps, warmup)
    del sets
    torch.cuda.empty_cache()
    return w, stats(d, p_)


def device_info(torch):
    """The GPU as torch sees it, and its clocks as rocm-smi reports them right
    after a timed leg (a child process with a time limit; None if unavailable)."""
    import subprocess
    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2**30, 1), "clocks": None}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        if r.returncode == 0:
            data = json.loads(r.stdout)
            card = next(iter(data.values())) if isinstance(data, dict) and data else {}
            info["clocks"] = {k: v for k, v in card.items() if "clk" in k.lower()} or card
    except Exception as e:  # noqa: BLE001
        info["clocks"] = f"unavailable: {type(e).__name__}"
    return info


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the decode workload
# ----------------------------------------------------------------------------

def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return 1


def cpu_baseline_prefill(case, nb=1):
    """The fp64 oracle on the first `nb` sequences of the causal prefill
    (all heads, all 2048 new tokens): TFLOP/s over the causal pairs it
    computes (the oracle itself works on the dense masked matrix)."""
    from oracle import gqa_oracle as O
    sub = case.copy()
    sub.batch = nb
    for f in ("seqlens_k", "q", "k_new", "v_new", "k_cache", "v_cache"):
        setattr(sub, f, getattr(case, f)[:nb].copy())
    t0 = time.perf_counter()
    st, out, *_ = O.gqa_attention(sub, "prefill")
    el = time.perf_counter() - t0
    assert st == O.OK
    fl = prefill_flops(sub)
    return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle, causal prefill of the first {nb} of {case.batch} "
                       f"sequences (S=2048, 32 heads, rotary), one run of {el:.1f} s, "
                       f"{fl:.3e} causal-pair flop; {len(os.sched_getaffinity(0))} host cores "
                       f"visible, {blas_threads()} BLAS threads; "
                       f"{platform.processor() or platform.machine()}")}


def cpu_baseline(case, budget_s=12.0):
    from oracle import gqa_oracle as O
    blas = blas_threads()
    nb = 4
    sub = case.copy()
    sub.batch = nb
    for f in ("seqlens_k", "q", "k_new", "v_new", "k_cache", "v_cache"):
        setattr(sub, f, getattr(case, f)[:nb].copy())
    reps, t0 = 0, time.perf_counter()
    while True:
        st, out, *_ = O.gqa_attention(sub, "decode")
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 200:
            break
    byts = decode_bytes(sub, [int(x) for x in sub.seqlens_k]) * reps
    return {"value": byts / el / 1e9, "unit": "GB/s", "cores": int(blas), "kind": "oracle",
            "sample": (f"fp64 numpy oracle, decode of the first {nb} of 16 sequences "
                       f"(past lengths {sub.seqlens_k.tolist()}), {reps} repetitions in {el:.1f} s; "
                       f"{len(os.sched_getaffinity(0))} host cores visible, {blas} BLAS threads; "
                       f"{platform.processor() or platform.machine()}")}


# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="decode,prefill,continuation,window,chunks,present,greedy,bias,"
                                      "head64",
                    help="workloads to run, comma-separated; the split-KV decode (the headline) "
                         "always runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device-to-device copies of MIB MiB (the reference "
                         "for scaling memory-traffic counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the op is not sharded across "
                                   "GPUs (run with --gpus 1)"}))
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_copy": n, "copies": 5}), flush=True)
        return
    import gqa_inputs as gi
    import grouped_query_kv_amd as gqa
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    which = set(args.only.split(","))
    unknown = which - {"decode", "prefill", "continuation", "window", "chunks", "present", "greedy",
                       "bias", "head64"}
    if unknown:
        sys.exit(f"--only: unknown workloads {sorted(unknown)}")
    result = {}

    # --- headline: fp16 split-KV decode -------------------------------------
    dec = gi.workload("split-kv-decode-fp16")
    log(f"[bench] split-KV decode sets: building (lens={dec.seqlens_k.tolist()})")
    sets = make_sets(dec, torch, gi.WORKLOAD_SEEDS[dec.name])
    log(f"[bench] split-KV decode: {len(sets)} input sets, timing {args.steps} steps")
    wall, dev, per = time_calls(torch, sets, decode_call(gqa), args.steps, args.warmup)
    dec_bytes = decode_bytes(dec, [int(x) for x in dec.seqlens_k])
    st_dec = stats(dev, per)
    achieved = dec_bytes / (st_dec["mean_ms"] * 1e-3) / 1e9
    value = dec_bytes / (wall * 1e-3) / 1e9
    del sets
    torch.cuda.empty_cache()
    yardstick = read_yardstick(torch, gqa, dec_bytes, args.steps, args.warmup,
                               st_dec["mean_ms"])
    device = device_info(torch)

    extra = {}
    if "prefill" in which:
        pre = gi.workload("causal-prefill-bf16")
        log("[bench] causal prefill sets: building")
        sets = make_sets(pre, torch, gi.WORKLOAD_SEEDS[pre.name])
        steps = max(5, args.steps // 2)
        log(f"[bench] causal prefill: {len(sets)} input sets, timing {steps} steps")
        w, d, p_ = time_calls(torch, sets, prefill_call(gqa), steps, max(2, args.warmup // 2))
        fl = prefill_flops(pre)
        st = stats(d, p_)
        tf = fl / (st["mean_ms"] * 1e-3) / 1e12
        extra["causal_prefill"] = {"workload": "bf16 causal prefill B=4 H=32 Hkv=8 D=128 S=2048 rotary",
                                   "tflops": tf, "frac_mfma_peak": tf / MFMA_PEAK_TFLOPS,
                                   "ms_per_call_wall": w, "flops": fl, **st}
        del sets
        torch.cuda.empty_cache()
    if "continuation" in which:
        cont = gi.workload("ragged-continuation-fp16")
        log("[bench] ragged continuation sets: building")
        sets = make_sets(cont, torch, gi.WORKLOAD_SEEDS[cont.name])
        log(f"[bench] ragged continuation: {len(sets)} input sets")
        w, d, p_ = time_calls(torch, sets, prefill_call(gqa), args.steps, args.warmup)
        fl = prefill_flops(cont)
        st = stats(d, p_)
        tf = fl / (st["mean_ms"] * 1e-3) / 1e12
        extra["ragged_continuation"] = {"workload": "fp16 ragged continuation B=8 H=28 Hkv=4 D=128 S=128",
                                        "tflops": tf, "frac_mfma_peak": tf / MFMA_PEAK_TFLOPS,
                                        "ms_per_call_wall": w, "flops": fl,
                                        "lens": cont.seqlens_k.tolist(), **st}
        del sets
        torch.cuda.empty_cache()
    if "window" in which:
        win = gi.workload("window-decode-bf16")
        log("[bench] window decode sets: building")
        sets = make_sets(win, torch, gi.WORKLOAD_SEEDS[win.name])
        log(f"[bench] window decode: {len(sets)} input sets")
        w, d, p_ = time_calls(torch, sets, decode_call(gqa), args.steps, args.warmup)
        st = stats(d, p_)
        att = decode_bytes(win, [4095] * 8, window=4096)
        shift = 8 * 8 * 4095 * 128 * 2 * 2 * 2      # read + write of every kept row, K and V
        del sets
        torch.cuda.empty_cache()
        # attention alone: the same shapes one row short of full (4095 past
        # rows), so the step appends at row 4095 and attends over 4096 keys
        # without moving anything
        att_case = gi.workload("window-decode-bf16")
        att_case.seqlens_k = np.full(8, 4095, np.int32)
        w2, st2 = run_leg(torch, "window decode, attention only", att_case, decode_call(gqa),
                          args.steps, args.warmup)
        extra["window_decode"] = {
            "workload": "bf16 sliding-window decode B=8 H=32 Hkv=8 D=128 M=W=4096, full cache",
            "step_gbs_vs_fused_minimum": (att + shift // 2) / (st["mean_ms"] * 1e-3) / 1e9,
            "step_bytes_unfused": att + shift, "attention_bytes": att,
            "ms_per_call_wall": w, **st,
            "attention_only": {
                "workload": "the same shapes with 4095 past rows: append at row 4095, attend over "
                            "4096 keys, no eviction",
                "gbs": att / (st2["mean_ms"] * 1e-3) / 1e9,
                "frac_hbm_peak": att / (st2["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "ms_per_call_wall": w2, **st2}}

    if "chunks" in which:
        # chunks of 128 tokens into the full window caches: attention over
        # past ++ new (staging frames), then eviction of 128 rows and append
        ch = gi.make_case("window-chunks-bf16", "bf16", 8, 128, 32, 8, 128, 4096, [4096] * 8, 6,
                          window=4096)
        w, st = run_leg(torch, "windowed chunks", ch, prefill_call(gqa), max(5, args.steps // 2),
                        max(2, args.warmup // 2))
        fl = prefill_flops(ch)
        kept = 8 * 8 * (4096 - 128) * 128 * 2 * 2          # K and V rows that move, bytes
        extra["windowed_chunks"] = {
            "workload": "bf16 windowed chunks B=8 H=32 Hkv=8 D=128 M=W=4096, full cache, S=128",
            "tflops": fl / (st["mean_ms"] * 1e-3) / 1e12, "flops": fl,
            "kept_rows_move_bytes_rw": 2 * kept, "ms_per_call_wall": w, **st}
    if "present" in which:
        pc = gi.workload("split-kv-decode-fp16")

        def with_present(x):
            x.present_k = torch.empty_like(x.k_cache)
            x.present_v = torch.empty_like(x.v_cache)
        w, st = run_leg(torch, "present-mode decode", pc, present_call(gqa), args.steps, args.warmup,
                        with_present)
        # the op's minimum: every past row read once (the attention's read)
        # and written once into present, plus the decode's own traffic
        copy = sum(int(L) for L in pc.seqlens_k) * 8 * 128 * 2 * 2   # past rows written
        byts = decode_bytes(pc, [int(x) for x in pc.seqlens_k]) + copy
        extra["present_decode"] = {
            "workload": "fp16 decode as the split-KV decode, past and present in separate buffers",
            "gbs": byts / (st["mean_ms"] * 1e-3) / 1e9, "bytes_per_call": byts,
            "frac_hbm_peak": byts / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_per_call_wall": w, **st}
    if "greedy" in which:
        # capacity 4608 rows, window 4096: a step that fits only attends
        # (4096 keys); one step in 512 overflows and first keeps the 4095
        # newest rows
        M, W = 4608, 4096
        plain = gi.make_case("greedy-window-bf16", "bf16", 8, 1, 32, 8, 128, M, [4096] * 8, 8,
                             window=W)
        plain.greedy_eviction = 1
        full = gi.make_case("greedy-window-bf16", "bf16", 8, 1, 32, 8, 128, M, [M] * 8, 8, window=W)
        full.greedy_eviction = 1
        w1, st1 = run_leg(torch, "greedy window decode (fits)", plain, prefill_call(gqa), args.steps,
                          args.warmup)
        w2, st2 = run_leg(torch, "greedy window decode (overflows)", full, prefill_call(gqa),
                          max(5, args.steps // 2), max(2, args.warmup // 2))
        att = decode_bytes(plain, [4095] * 8, window=W)
        amort = (st2["mean_ms"] + (M - W - 1) * st1["mean_ms"]) / (M - W)
        extra["greedy_window_decode"] = {
            "workload": "bf16 window decode B=8 H=32 Hkv=8 D=128 W=4096, capacity 4608, greedy eviction",
            "fits_ms": st1["mean_ms"], "overflow_ms": st2["mean_ms"],
            "amortized_ms_per_step": amort, "attention_bytes": att,
            "attention_gbs_when_fits": att / (st1["mean_ms"] * 1e-3) / 1e9,
            "fits_wall_ms": w1, "overflow_wall_ms": w2}

    if "bias" in which:
        # additive bias [B, H, S, T], T >= the longest past + new: both the
        # split-KV decode and the prefill kernel read it in their tile loops
        def add_bias(T):
            def prep(x):
                c = x.case
                x.bias = torch.randn((c.batch, c.num_heads, c.new_tokens, T), device="cuda",
                                     dtype=torch.float32).to(x.q.dtype)
            return prep
        bd = gi.workload("split-kv-decode-fp16")
        T = int(bd.seqlens_k.max()) + 1
        w, st = run_leg(torch, "decode with bias", bd, biased_call(gqa), args.steps, args.warmup,
                        add_bias(T))
        bias_read = sum(int(L) + 1 for L in bd.seqlens_k) * bd.num_heads * 2
        byts = decode_bytes(bd, [int(x) for x in bd.seqlens_k]) + bias_read
        extra["decode_with_bias"] = {
            "workload": "fp16 split-KV decode as the headline plus a [16, 32, 1, T] fp16 bias",
            "gbs": byts / (st["mean_ms"] * 1e-3) / 1e9, "bytes_per_call": byts,
            "frac_hbm_peak": byts / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_per_call_wall": w, **st}
        bc = gi.workload("ragged-continuation-fp16")
        T = -(-(int(bc.seqlens_k.max()) + bc.new_tokens) // 4) * 4   # a multiple of 4: MFMA kernel
        w, st = run_leg(torch, "continuation with bias", bc, biased_call(gqa), args.steps,
                        args.warmup, add_bias(T))
        fl = prefill_flops(bc)
        extra["continuation_with_bias"] = {
            "workload": "fp16 ragged continuation B=8 H=28 Hkv=4 S=128 plus a [8, 28, 128, T] fp16 "
                        "bias, T a multiple of 4",
            "tflops": fl / (st["mean_ms"] * 1e-3) / 1e12,
            "frac_mfma_peak": fl / (st["mean_ms"] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
            "ms_per_call_wall": w, **st}

    if "head64" in which:
        # the headline decode and the causal prefill at head size 64 (the same
        # past lengths; fresh draws of the values)
        d64 = gi.make_case("split-kv-decode-fp16-d64", "fp16", 16, 1, 32, 8, 64, 4096,
                           dec.seqlens_k, 12)
        w, st = run_leg(torch, "decode, head size 64", d64, decode_call(gqa), args.steps, args.warmup)
        byts = decode_bytes(d64, [int(x) for x in d64.seqlens_k])
        extra["decode_head64"] = {
            "workload": "fp16 decode B=16 H=32 Hkv=8 D=64 M=4096, the headline's past lengths",
            "gbs": byts / (st["mean_ms"] * 1e-3) / 1e9, "bytes_per_call": byts,
            "frac_hbm_peak": byts / (st["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_per_call_wall": w, **st}
        p64 = gi.make_case("causal-prefill-bf16-d64", "bf16", 4, 2048, 32, 8, 64, 4096, [0] * 4, 13,
                           rotary=True, rotary_rows=4096)
        w, st = run_leg(torch, "causal prefill, head size 64", p64, prefill_call(gqa),
                        max(5, args.steps // 2), max(2, args.warmup // 2))
        fl = prefill_flops(p64)
        extra["causal_prefill_head64"] = {
            "workload": "bf16 causal prefill B=4 H=32 Hkv=8 D=64 S=2048 rotary",
            "tflops": fl / (st["mean_ms"] * 1e-3) / 1e12,
            "frac_mfma_peak": fl / (st["mean_ms"] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
            "flops": fl, "ms_per_call_wall": w, **st}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        cpu = cpu_baseline(dec)
        if "causal_prefill" in extra:
            log("[bench] CPU baseline of the causal prefill (oracle)")
            extra["causal_prefill"]["cpu_baseline"] = cpu_baseline_prefill(
                gi.workload("causal-prefill-bf16"))

    line = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "fp16 decode, B=16 H=32 Hkv=8 D=128 M=4096, past lengths U{512..4095} "
                               "(seed 2), 1 new token per sequence",
                   "global_batch": 16, "seq_len": 4096, "parallelism": "none (1 GPU)",
                   "seqlens_k": dec.seqlens_k.tolist()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": decode_traffic_bytes(),
                     "kernel": "decode call (all launches of gqa_attention_decode)",
                     "bytes_per_call": dec_bytes, **st_dec},
        "cpu_baseline": cpu,
        "hbm_read_yardstick": yardstick,
        "device": device,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Caches must match bit for bit (every byte outside the appended rows included,
so a stray write or a read of the NaN poison past the length shows up);
outputs must be finite and within max abs error 1e-4 (fp32) or 2e-2
(fp16/bf16) of the oracle.
"""
import sys

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import gqa_oracle as O

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_kv_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch


from gpu_helpers import (DevCase, assert_bits_equal, assert_close, out_f64, to_bits,  # noqa: E402
                         to_dev)


def check_full(case, entry="prefill", what=""):
    """Run one call on the GPU and compare everything with the oracle."""
    say(f"[gpu] {what or case.name}: B={case.batch} S={case.new_tokens} H={case.num_heads} "
        f"Hkv={case.kv_num_heads} D={case.head_size} M={case.max_seq_len} dt={case.dtype} "
        f"W={case.local_window_size} rot={case.cos is not None} lens={list(case.seqlens_k)[:8]}")
    st, want, kc, vc, lens_after = O.gqa_attention(case, entry)
    assert st == O.OK
    dev = DevCase(case)
    out = dev.run(entry)
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, f"{what} k_cache")
    assert_bits_equal(gv, vc, f"{what} v_cache")
    err = assert_close(out_f64(out, case.dtype), want, case.dtype, what)
    say(f"[gpu]   max abs error {err:.3e}")
    return dev, kc, vc, lens_after, err


# --------------------------------------------------------------------------
# the worked example (prefill 32, then decode to 33)
# --------------------------------------------------------------------------

def test_worked_example_prefill_then_decode():
    c1 = gi.workload("worked-example", step=1)
    dev, kc, vc, lens, _ = check_full(c1, "prefill", "worked example step 1")
    c2 = gi.workload("worked-example", step=2)
    c2.k_cache, c2.v_cache = kc, vc                 # continue from step 1's cache
    st, want, kc2, vc2, _ = O.gqa_attention(c2, "decode")
    d2 = DevCase(c2)
    d2.k_cache, d2.v_cache = dev.k_cache, dev.v_cache  # same buffer, stays in place
    ptr = dev.k_cache.data_ptr()
    out = d2.run("decode")
    assert dev.k_cache.data_ptr() == ptr
    gk, gv = d2.caches()
    assert_bits_equal(gk, kc2, "worked example step 2 k_cache")
    assert_bits_equal(gv, vc2, "worked example step 2 v_cache")
    assert_close(out_f64(out, "fp32"), want, "fp32", "worked example step 2")


# --------------------------------------------------------------------------
# small randomised shapes: tile edges, ragged lengths, groups, windows, rotary
# --------------------------------------------------------------------------

SMALL = [
    # dtype, B, S, H, Hkv, D, M, lens, window, rotary, interleaved, entry
    ("fp16", 3, 1, 8, 2, 128, 300, [0, 63, 257], -1, False, 0, "decode"),
    ("bf16", 2, 1, 32, 8, 128, 600, [64, 511], -1, False, 0, "decode"),
    ("fp16", 4, 1, 28, 4, 128, 1100, [127, 128, 129, 1099], -1, False, 0, "decode"),
    ("bf16", 2, 1, 8, 8, 128, 200, [5, 199], -1, True, 0, "decode"),
    ("fp16", 2, 1, 16, 2, 128, 300, [299, 17], 64, False, 0, "decode"),
    ("bf16", 2, 1, 16, 1, 128, 256, [256, 256], 256, False, 0, "decode"),     # full: evict 1
    ("fp32", 2, 1, 6, 3, 64, 80, [0, 79], -1, True, 1, "decode"),
    ("fp16", 2, 1, 4, 2, 64, 100, [10, 99], -1, False, 0, "decode"),
    ("bf16", 2, 37, 8, 2, 128, 400, [0, 200], -1, False, 0, "prefill"),
    ("fp16", 2, 64, 28, 4, 128, 300, [63, 1], -1, False, 0, "prefill"),
    ("bf16", 1, 130, 32, 8, 128, 512, [0], -1, True, 0, "prefill"),
    ("fp16", 3, 17, 8, 1, 128, 128, [0, 50, 111], -1, True, 1, "prefill"),
    ("bf16", 2, 33, 16, 2, 128, 200, [100, 0], 40, False, 0, "prefill"),
    ("fp16", 2, 5, 12, 4, 64, 64, [3, 59], -1, False, 0, "prefill"),
    ("fp32", 2, 9, 4, 2, 8, 40, [0, 31], 7, False, 0, "prefill"),
    ("bf16", 2, 3, 2, 1, 256, 40, [10, 0], -1, True, 0, "prefill"),
    ("fp16", 1, 1, 1, 1, 8, 1, [0], -1, False, 0, "prefill"),               # M = 1
    # few row blocks and a long buffer: key ranges sized to the lengths and
    # split over up to 4 workgroups, including ranges in which some rows see
    # no key (their causal limit lies before the range) and an unsplit L = 0
    ("fp16", 3, 40, 8, 2, 128, 2048, [0, 700, 1999], -1, True, 0, "prefill"),
    ("bf16", 2, 33, 16, 2, 128, 2048, [1500, 0], 100, False, 0, "prefill"),
    ("bf16", 2, 7, 8, 8, 128, 1024, [1017, 300], -1, False, 0, "prefill"),
    # more than 16 query heads per kv head: several head groups per kv head
    # in the decode (G = 32: two groups of 16; G = 20: two groups of 10)
    ("fp16", 3, 1, 32, 1, 128, 700, [699, 5, 300], -1, False, 0, "decode"),
    ("bf16", 2, 1, 40, 2, 128, 520, [100, 518], -1, True, 0, "decode"),
    ("bf16", 2, 1, 40, 2, 128, 520, [519, 519], 64, False, 0, "decode"),
    ("fp16", 2, 9, 32, 1, 128, 300, [0, 250], -1, True, 0, "prefill"),
    # more sequences than travel in the kernel arguments: lengths read on the device
    ("bf16", 66, 3, 4, 2, 128, 64, [(7 * i) % 62 for i in range(66)], -1, True, 0, "prefill"),
    ("fp16", 66, 1, 4, 2, 128, 64, [(5 * i) % 64 for i in range(66)], -1, False, 0, "decode"),
    # 33-64 sequences on the split-KV decode: per-sequence values held one
    # per lane, including lanes 32-63 (plain, and with the fused eviction)
    ("fp16", 48, 1, 8, 2, 128, 256, [(37 * i) % 256 for i in range(48)], -1, False, 0, "decode"),
    ("bf16", 64, 1, 4, 1, 128, 192, [192 if i % 3 == 0 else (29 * i) % 192 for i in range(64)],
     192, True, 0, "decode"),
    # windowed chunks that evict: attention over past ++ new in the staging
    # frames, then eviction and append in the cache (some sequences evict,
    # some not; the window below, at and above the chunk; S = M drops the
    # whole past; the split plan on a long buffer; the generic kernel)
    ("bf16", 2, 33, 16, 2, 128, 200, [190, 100], 200, False, 0, "prefill"),
    ("fp16", 3, 64, 28, 4, 128, 300, [300, 280, 0], 128, True, 0, "prefill"),
    ("bf16", 2, 130, 32, 8, 128, 512, [500, 512], 512, True, 0, "prefill"),
    ("fp16", 1, 64, 8, 1, 128, 64, [64], 64, False, 0, "prefill"),
    ("bf16", 2, 40, 8, 2, 128, 2048, [2040, 1000], 1024, False, 0, "prefill"),
    ("fp16", 2, 70, 8, 2, 128, 256, [255, 256], 16, True, 1, "prefill"),
    ("fp32", 2, 9, 4, 2, 8, 40, [35, 40], 40, False, 0, "prefill"),
    ("bf16", 2, 5, 6, 3, 64, 48, [48, 44], 20, True, 0, "prefill"),
    # head size 64 on the split-KV decode: half a row per lane group, the
    # rotation's pairs at the half-size table stride, one head group and two
    # (G = 32), the fused eviction of a full window and the eviction kernel
    ("bf16", 3, 1, 16, 2, 64, 700, [699, 5, 300], -1, True, 0, "decode"),
    ("fp16", 2, 1, 32, 1, 64, 520, [519, 100], -1, True, 1, "decode"),
    ("bf16", 2, 1, 16, 2, 64, 300, [300, 17], 300, False, 0, "decode"),
    ("fp16", 2, 1, 8, 2, 64, 300, [299, 17], 64, True, 0, "decode"),
    ("bf16", 64, 1, 4, 1, 64, 192, [192 if i % 3 == 0 else (29 * i) % 192 for i in range(64)],
     192, True, 0, "decode"),
    # head size 64 on the MFMA prefill: 128-byte tile rows, four products per
    # score tile and two output tiles; several row blocks, G = 7, the
    # key-split plan (plain and windowed), both rotary pair orders and a
    # windowed chunk that evicts (staging frame)
    ("bf16", 2, 130, 32, 8, 64, 512, [0, 300], -1, True, 0, "prefill"),
    ("fp16", 2, 64, 28, 4, 64, 300, [63, 1], -1, False, 0, "prefill"),
    ("fp16", 3, 40, 8, 2, 64, 2048, [0, 700, 1999], -1, True, 1, "prefill"),
    ("bf16", 2, 33, 16, 2, 64, 2048, [1500, 0], 100, False, 0, "prefill"),
    ("fp16", 2, 70, 8, 2, 64, 256, [255, 256], 16, True, 1, "prefill"),
    ("bf16", 2, 40, 8, 2, 64, 2048, [2040, 1000], 1024, True, 0, "prefill"),
]


@pytest.mark.parametrize("spec", SMALL, ids=[f"{s[0]}-{s[-1]}-{i}" for i, s in enumerate(SMALL)])
def test_small_shapes(spec):
    dt, B, S, H, Hkv, D, M, lens, W, rot, inter, entry = spec
    case = gi.make_case("small", dt, B, S, H, Hkv, D, M, lens, seed=sum(map(ord, repr(spec))) % 1000,
                        window=W, rotary=rot, interleaved=inter,
                        rotary_rows=(M + S if rot else None))
    check_full(case, entry, f"small {spec}")


# --------------------------------------------------------------------------
# separate past and present buffers: present = past ++ new, then the op
# --------------------------------------------------------------------------

PRESENT = [
    # dtype, B, S, H, Hkv, D, past_rows, present rows M, lens, window, rotary, entry
    ("fp16", 3, 1, 32, 8, 128, 700, 701, [0, 350, 700], -1, False, "decode"),
    ("bf16", 2, 64, 16, 2, 128, 300, 364, [300, 17], -1, True, "prefill"),
    ("fp32", 2, 5, 4, 2, 8, 20, 25, [20, 3], -1, False, "prefill"),
    ("bf16", 2, 40, 8, 2, 128, 256, 256, [256, 200], 128, False, "prefill"),   # present evicts
    ("fp16", 2, 1, 8, 2, 128, 512, 512, [512, 100], 512, True, "decode"),     # decode evicts
    # one new token on the split-KV decode, which copies the past rows into
    # present as it reads them: head size 64 with a window reaching row 0,
    # more than 64 sequences (the launches of 64 offset the past buffers
    # too), two head groups (only the first writes), and a window that does
    # not reach row 0 (the separate copy)
    ("bf16", 4, 1, 16, 2, 64, 300, 400, [299, 0, 150, 17], 301, True, "decode"),
    ("fp16", 70, 1, 8, 2, 128, 96, 128, [(13 * i) % 97 for i in range(70)], -1, False, "decode"),
    ("bf16", 2, 1, 64, 2, 128, 200, 256, [199, 64], -1, True, "decode"),
    ("fp16", 2, 1, 8, 2, 128, 256, 300, [255, 10], 100, False, "decode"),
]


@pytest.mark.parametrize("spec", PRESENT, ids=[f"{s[0]}-{s[-1]}-{i}" for i, s in enumerate(PRESENT)])
def test_present_mode(spec):
    import torch
    dt, B, S, H, Hkv, D, P, M, lens, W, rot, entry = spec
    seed = sum(map(ord, repr(spec))) % 1000
    case = gi.make_case("present", dt, B, S, H, Hkv, D, M, [0] * B, seed, window=W, rotary=rot,
                        rotary_rows=(M + S if rot else None))
    case.seqlens_k = np.asarray(lens, np.int32)
    rng = np.random.default_rng(seed + 1)
    past_k = gi.fill_cache(rng, B, Hkv, P, D, lens, dt)
    past_v = gi.fill_cache(rng, B, Hkv, P, D, lens, dt)
    say(f"[gpu] present mode {spec}")
    st, want, kc, vc, after = O.gqa_attention_present(case, past_k, past_v)
    assert st == O.OK
    dev = DevCase(case)                       # k_cache / v_cache: the present buffers
    pk, pv = to_dev(past_k, dt), to_dev(past_v, dt)
    import grouped_query_kv_amd as gqa
    fn = gqa.gqa_attention_decode if entry == "decode" else gqa.gqa_attention_prefill
    out = fn(dev.q, dev.k_new, dev.v_new, pk, pv, dev.lens_host, dev.lens_dev, scale=case.scale,
             local_window_size=W, cos_cache=dev.cos, sin_cache=dev.sin,
             present_key=dev.k_cache, present_value=dev.v_cache)
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, "present k")
    assert_bits_equal(gv, vc, "present v")
    assert_bits_equal(to_bits(pk), past_k, "past k (never written)")
    assert_bits_equal(to_bits(pv), past_v, "past v (never written)")
    err = assert_close(out_f64(out, dt), want, dt, f"present {spec}")
    say(f"[gpu]   max abs error {err:.3e}")
    # the filled present buffer then serves as a shared buffer
    if all(int(a) < M for a in after) or W > 0:
        nxt = gi.next_decode_tokens(case, rng)
        nxt.k_cache, nxt.v_cache, nxt.seqlens_k = kc, vc, after.astype(np.int32)
        st2, want2, kc2, vc2, _ = O.gqa_attention(nxt, "decode")
        assert st2 == O.OK
        d2 = DevCase(nxt)
        d2.k_cache, d2.v_cache = dev.k_cache, dev.v_cache
        out2 = d2.run("decode")
        gk2, gv2 = d2.caches()
        assert_bits_equal(gk2, kc2, "present then shared k")
        assert_bits_equal(gv2, vc2, "present then shared v")
        assert_close(out_f64(out2, dt), want2, dt, "present then shared decode")
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# greedy eviction (capacity M > window W): move rows only on overflow
# --------------------------------------------------------------------------

GREEDY = [
    # dtype, B, H, Hkv, D, M, W, lens, chunk sizes per step, rotary
    ("bf16", 4, 32, 8, 128, 1024, 768, [1024, 1000, 500, 1024], [1, 1, 1, 1], False),
    ("fp16", 3, 28, 4, 128, 512, 200, [512, 480, 100], [64, 1, 64, 1], True),
    ("fp16", 2, 8, 2, 128, 256, 40, [256, 250], [64, 1, 1], False),          # S > W
    ("fp32", 2, 4, 2, 8, 40, 10, [40, 30], [1, 5, 1, 1], True),
]


@pytest.mark.parametrize("spec", GREEDY, ids=[f"{s[0]}-{i}" for i, s in enumerate(GREEDY)])
def test_greedy_eviction_rolling(spec):
    dt, B, H, Hkv, D, M, W, lens, chunks, rot = spec
    seed = sum(map(ord, repr(spec))) % 1000
    rng = np.random.default_rng(seed)
    case = gi.make_case("greedy", dt, B, chunks[0], H, Hkv, D, M, lens, seed, window=W,
                        rotary=rot, rotary_rows=(M + max(chunks) if rot else None))
    case.greedy_eviction = 1
    dev = DevCase(case)
    cache_k, cache_v = dev.k_cache, dev.v_cache
    for step, S in enumerate(chunks):
        entry = "decode" if S == 1 else "prefill"
        say(f"[gpu] greedy {spec[:7]} step {step}: S={S} lens={case.seqlens_k.tolist()}")
        st, want, kc, vc, after = O.gqa_attention(case, entry)
        assert st == O.OK
        out = dev.run(entry)
        gk, gv = dev.caches()
        assert_bits_equal(gk, kc, f"greedy step {step} k_cache")
        assert_bits_equal(gv, vc, f"greedy step {step} v_cache")
        err = assert_close(out_f64(out, dt), want, dt, f"greedy step {step}")
        say(f"[gpu]   max abs error {err:.3e}, lengths after {after.tolist()}")
        if step + 1 == len(chunks):
            break
        nxt = case.copy()
        nxt.new_tokens = chunks[step + 1]
        nxt.q = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, H * D)), dt)
        nxt.k_new = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, Hkv * D)), dt)
        nxt.v_new = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, Hkv * D)), dt)
        nxt.k_cache, nxt.v_cache, nxt.seqlens_k = kc, vc, after.astype(np.int32)
        case = nxt
        dev = DevCase(case)
        dev.k_cache, dev.v_cache = cache_k, cache_v


# --------------------------------------------------------------------------
# additive attention bias: column = the key's position in past ++ new
# --------------------------------------------------------------------------

BIAS = [
    # dtype, B, S, H, Hkv, D, M, lens, window, rotary, bias (batch, heads), extra columns, greedy
    ("fp16", 4, 1, 32, 8, 128, 1024, [0, 100, 700, 1023], -1, False, "BH", 5, 0),    # fast decode
    ("bf16", 2, 1, 16, 4, 128, 512, [512, 300], 512, False, "1H", 0, 0),             # fused eviction
    ("bf16", 2, 1, 8, 2, 128, 300, [300, 17], 64, True, "B1", 3, 0),                 # eviction kernel
    ("fp16", 2, 1, 8, 2, 128, 256, [256, 50], 100, False, "BH", 0, 1),               # greedy: drop 157
    ("fp32", 2, 1, 4, 2, 8, 40, [40, 3], 40, False, "BH", 0, 0),                     # generic decode
    ("fp16", 2, 33, 8, 2, 128, 200, [0, 100], -1, True, "BH", 2, 0),                 # prefill (generic)
    ("bf16", 2, 20, 8, 2, 128, 128, [128, 120], 128, False, "11", 0, 0),             # chunk, staging
    # T % 4 == 0: the MFMA prefill kernel reads the bias (four columns per load)
    ("fp16", 2, 33, 8, 2, 128, 200, [0, 100], -1, True, "BH", 3, 0),
    ("bf16", 3, 40, 8, 2, 128, 2048, [0, 700, 1999], -1, True, "1H", 1, 0),       # key-split plan
    ("bf16", 2, 33, 16, 2, 128, 200, [100, 0], 40, False, "B1", 3, 0),            # window
    ("fp16", 2, 130, 28, 4, 128, 512, [380, 0], -1, False, "BH", 2, 0),           # several row blocks
    ("bf16", 2, 20, 8, 2, 128, 128, [128, 120], 128, False, "11", 1, 0),          # staging, plain kernel
    ("fp16", 3, 1, 16, 2, 64, 600, [0, 300, 599], -1, True, "BH", 2, 0),          # D = 64 decode
    ("bf16", 2, 1, 8, 2, 64, 256, [256, 100], 256, False, "1H", 0, 0),            # D = 64 fused
    ("fp16", 2, 33, 8, 2, 64, 200, [0, 100], -1, True, "BH", 3, 0),               # D = 64 prefill
    ("bf16", 3, 40, 8, 2, 64, 2048, [0, 700, 1999], -1, False, "1H", 1, 0),       # D = 64 split
]


def _attach_bias(case, kind, extra, rng):
    B, H, S = case.batch, case.num_heads, case.new_tokens
    Bb = B if kind[0] == "B" else 1
    Hb = H if kind[1] == "H" else 1
    T = int((np.asarray(case.seqlens_k) + S).max()) + extra
    case.attention_bias = gi.to_bits(rng.standard_normal((Bb, Hb, S, T)), case.dtype)
    return case


@pytest.mark.parametrize("spec", BIAS, ids=[f"{s[0]}-{s[10]}-{i}" for i, s in enumerate(BIAS)])
def test_attention_bias(spec):
    dt, B, S, H, Hkv, D, M, lens, W, rot, kind, extra, greedy = spec
    seed = sum(map(ord, repr(spec))) % 1000
    case = gi.make_case("bias", dt, B, S, H, Hkv, D, M, lens, seed, window=W, rotary=rot,
                        rotary_rows=(M + S if rot else None))
    case.greedy_eviction = greedy
    _attach_bias(case, kind, extra, np.random.default_rng(seed))
    check_full(case, "decode" if S == 1 else "prefill", f"bias {spec}")


# More sequences than one split-KV decode launch plans (64): one-token calls
# that evict run the eviction (fused when the window covers the buffer) and
# then the split-KV decode in launches of 64 sequences, which must keep the
# same rows as the eviction (W - 1 with greedy eviction) and read the bias
# column of a kept key at its buffer row plus the dropped count.
MANY = [
    # dtype, H, Hkv, M, W, greedy, bias kind
    ("bf16", 8, 2, 96, 64, 1, None),
    ("fp16", 8, 2, 96, 96, 0, "BH"),
    ("fp16", 4, 1, 80, 48, 1, "1H"),
]


@pytest.mark.parametrize("spec", MANY, ids=[f"{s[0]}-g{s[5]}-{s[6]}" for s in MANY])
def test_many_sequences_evicting_decode(spec):
    dt, H, Hkv, M, W, greedy, kind = spec
    B = 66
    lens = [M if i % 3 else (11 * i) % M for i in range(B)]
    seed = sum(map(ord, repr(spec))) % 1000
    case = gi.make_case("many", dt, B, 1, H, Hkv, 128, M, lens, seed, window=W)
    case.greedy_eviction = greedy
    if kind:
        _attach_bias(case, kind, 2, np.random.default_rng(seed))
    check_full(case, "decode", f"{B} sequences evicting {spec}")


@pytest.mark.parametrize("spec", [
    # dtype, B, H, Hkv, D, M, W, rotary: more than 64 sequences run the
    # split-KV decode as consecutive launches of 64 (here 64 + 64 + 2, and
    # 64 + 6 with the fused eviction of a full window)
    ("fp16", 130, 8, 2, 128, 256, -1, True),
    ("bf16", 70, 8, 8, 128, 128, 128, False),
    ("fp16", 70, 8, 2, 64, 128, 128, True),
], ids=["fp16-B130", "bf16-B70-window", "fp16-B70-D64-window"])
def test_decode_more_than_64_sequences(spec):
    dt, B, H, Hkv, D, M, W, rot = spec
    seed = sum(map(ord, repr(spec))) % 1000
    rng = np.random.default_rng(seed)
    if W > 0:
        lens = [M if i % 4 else int(rng.integers(0, M)) for i in range(B)]
    else:
        lens = rng.integers(0, M, B).tolist()
    case = gi.make_case("many-decode", dt, B, 1, H, Hkv, D, M, lens, seed, window=W, rotary=rot,
                        rotary_rows=2 * M)
    check_full(case, "decode", f"decode {B} sequences {spec}")


def test_attention_bias_decode_full_size():
    case = gi.workload("split-kv-decode-fp16")
    _attach_bias(case, "BH", 1, np.random.default_rng(77))
    check_full(case, "decode", "split-KV decode with a [B, H, 1, T] bias")


# one-token calls with separate past and present buffers on the split-KV
# decode, which moves the past rows itself: random shapes with bias, rotary
# position offsets, several head groups and more than 64 sequences
@pytest.mark.parametrize("k", range(12))
def test_present_decode_fused_copy_random(k):
    import grouped_query_kv_amd as gqa
    rng = np.random.default_rng(9000 + k)
    dt = ["fp16", "bf16"][int(rng.integers(0, 2))]
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 4, 7, 20]))
    B = int(rng.choice([1, 3, 17, 66]))
    P = int(rng.choice([64, 200, 513]))
    M = P + int(rng.integers(1, 40))
    lens = rng.integers(0, P + 1, B).tolist()
    W = -1 if rng.random() < 0.6 else max(lens) + 1 + int(rng.integers(0, 5))
    rot = bool(rng.random() < 0.5)
    case = gi.make_case("present-fused", dt, B, 1, G * Hkv, Hkv, D, M, [0] * B, 9100 + k, window=W,
                        rotary=rot, rotary_rows=(M + 41 if rot else None))
    case.seqlens_k = np.asarray(lens, np.int32)
    if rot and rng.random() < 0.5:
        case.position_offset = rng.integers(0, 40, B).astype(np.int32)
    if rng.random() < 0.4:
        T = max(lens) + 1 + int(rng.integers(0, 5))
        case.attention_bias = gi.to_bits(rng.standard_normal((B, G * Hkv, 1, T)), dt)
    past_k = gi.fill_cache(rng, B, Hkv, P, D, lens, dt)
    past_v = gi.fill_cache(rng, B, Hkv, P, D, lens, dt)
    desc = f"present fused {k}: {dt} B={B} G={G} Hkv={Hkv} D={D} P={P} M={M} W={W} rot={rot}"
    say(f"[gpu] {desc}")
    st, want, kc, vc, _ = O.gqa_attention_present(case, past_k, past_v)
    assert st == O.OK
    dev = DevCase(case)
    pk, pv = to_dev(past_k, dt), to_dev(past_v, dt)
    out = gqa.gqa_attention_decode(dev.q, dev.k_new, dev.v_new, pk, pv, dev.lens_host, dev.lens_dev,
                                   scale=case.scale, local_window_size=W, cos_cache=dev.cos,
                                   sin_cache=dev.sin, present_key=dev.k_cache,
                                   present_value=dev.v_cache, attention_bias=dev.bias,
                                   position_offset=dev.off_host, position_offset_dev=dev.off_dev)
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, f"{desc} present k")
    assert_bits_equal(gv, vc, f"{desc} present v")
    assert_bits_equal(to_bits(pk), past_k, f"{desc} past k (never written)")
    assert_bits_equal(to_bits(pv), past_v, f"{desc} past v (never written)")
    err = assert_close(out_f64(out, dt), want, dt, desc)
    say(f"[gpu]   max abs error {err:.3e}")


# --------------------------------------------------------------------------
# the halves: append and eviction on their own
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dt,D,rot,offsets", [("fp16", 128, False, None), ("bf16", 64, True, None),
                                              ("fp32", 8, True, None), ("fp16", 6, False, None),
                                              ("bf16", 128, True, [9, 0, 24]),
                                              ("fp32", 8, True, [3, 1, 2])])
def test_append_by_index_code(dt, D, rot, offsets):
    B, S, Hkv, M = 3, 5, 2, 40
    case = gi.make_case("append", dt, B, S, 2 * Hkv, Hkv, D, M, [0, 17, 35], 3, rotary=rot,
                        rotary_rows=M + 24)
    if offsets is not None:
        case.position_offset = np.array(offsets, np.int32)
    code = np.arange(B * S * Hkv * D, dtype=np.float64).reshape(B, S, Hkv * D) % 1000
    case.k_new = gi.to_bits(code, dt)
    case.v_new = gi.to_bits(-code, dt)
    say(f"[gpu] append {dt} D={D} rot={rot} offsets={offsets}")
    st, kc, vc = O.gqa_append_kv(case)
    dev = DevCase(case)
    dev.append()
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, "append k_cache")
    assert_bits_equal(gv, vc, "append v_cache")


@pytest.mark.parametrize("dt,D,M,lens,incoming", [
    ("bf16", 128, 4096, [4096, 4095, 100, 0], 1),        # one-row drop, halo path
    ("fp16", 128, 700, [700, 690, 650, 10], 30),         # several rows, halo path
    ("fp32", 8, 3000, [3000, 2999, 1500, 2990], 200),    # large drop, serial path
    ("fp16", 6, 513, [513, 300, 513, 0], 1),             # 12-byte rows
    ("bf16", 64, 64, [64, 64, 10, 64], 64),              # drop everything
])
def test_evict_window_half(dt, D, M, lens, incoming):
    import grouped_query_kv_amd as gqa
    case = gi.make_case("evict", dt, len(lens), 1, 2, 2, D, M, lens, 4)
    say(f"[gpu] evict {dt} D={D} M={M} lens={lens} incoming={incoming}")
    st, kc, vc, after = O.gqa_evict_window(case, incoming)
    dev = DevCase(case)
    got_after = gqa.gqa_evict_window(dev.k_cache, dev.v_cache, dev.lens_host, dev.lens_dev, incoming)
    assert got_after.tolist() == after.tolist()
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, "evict k_cache")
    assert_bits_equal(gv, vc, "evict v_cache")


# --------------------------------------------------------------------------
# the five workloads at full size
# --------------------------------------------------------------------------

def test_split_kv_decode_full_size():
    check_full(gi.workload("split-kv-decode-fp16"), "decode", "split-KV decode")


def test_window_decode_rolling_steps():
    import grouped_query_kv_amd as gqa
    case = gi.workload("window-decode-bf16")
    rng = np.random.default_rng(55)
    dev = DevCase(case)
    ptr = dev.k_cache.data_ptr()
    for step in range(4):
        say(f"[gpu] window decode rolling step {step}")
        st, want, kc, vc, lens = O.gqa_attention(case, "decode")
        assert st == O.OK and lens.tolist() == [4096] * 8
        out = dev.run("decode")
        gk, gv = dev.caches()
        assert_bits_equal(gk, kc, f"window decode step {step} k_cache")
        assert_bits_equal(gv, vc, f"window decode step {step} v_cache")
        assert_close(out_f64(out, "bf16"), want, "bf16", f"window decode step {step}")
        assert dev.k_cache.data_ptr() == ptr
        nxt = gi.next_decode_tokens(case, rng)
        nxt.k_cache, nxt.v_cache = kc, vc
        case = nxt
        dev.case = case
        for name in ("q", "k_new", "v_new"):
            getattr(dev, name).copy_(to_dev(getattr(case, name), "bf16"))
    # the same full cache with the window off has no room
    case.local_window_size = -1
    dev.case = case
    with pytest.raises(gqa.GQAError) as e:
        dev.run("decode")
    assert e.value.status == gqa.GQA_ERR_NO_ROOM


@pytest.mark.parametrize("dt,M,lens,S,greedy", [
    ("bf16", 1024, [1024, 1000, 1024], 40, 0),   # split key ranges: partial slots poisoned too
    ("fp16", 256, [256, 199, 131], 37, 1),       # greedy: only the first overflows
])
def test_windowed_chunk_poisoned_workspace(dt, M, lens, S, greedy):
    """A windowed chunk (S > 1 into full W-slot caches) whose workspace holds
    NaN bits in every byte except the merge counters (which the library keeps
    at zero between calls). The staging frames then hold NaN in the rows past
    each sequence's L + S up to the end of its last 64-key tile, and in every
    row no step writes: outputs and caches must still match the oracle, so the
    prefill's tile loads stop at the valid length and nothing reads a row the
    call did not write."""
    import torch
    from test_prefill_plan import align256, cdiv, layout, lib_workspace
    B, H, Hkv, D = 3, 8, 2, 128
    case = gi.make_case("poisoned-workspace", dt, B, S, H, Hkv, D, M, lens, 41 + S, window=M,
                        rotary=True, rotary_rows=M + S)
    case.greedy_eviction = greedy
    total, _, (c_off, c_bytes), _ = layout(B, S, H, Hkv, D, M, 2, M)
    assert total == lib_workspace(B, S, H, Hkv, M, M, {"fp16": 1, "bf16": 2}[dt])
    ws = torch.full((total,), 0xFF, dtype=torch.uint8, device="cuda")   # 0xFFFF: NaN in fp16, bf16
    ws[:align256(B * Hkv * cdiv(H // Hkv, 16) * 4)] = 0                  # decode merge counters
    ws[c_off:c_off + c_bytes] = 0                                        # prefill split counters
    say(f"[gpu] poisoned workspace {dt} lens={lens} S={S} greedy={greedy}: {total} bytes")
    st, want, kc, vc, _ = O.gqa_attention(case, "prefill")
    assert st == O.OK
    dev = DevCase(case)
    out = dev.run("prefill", workspace=ws)
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, "poisoned workspace k_cache")
    assert_bits_equal(gv, vc, "poisoned workspace v_cache")
    err = assert_close(out_f64(out, dt), want, dt, "poisoned workspace")
    say(f"[gpu]   max abs error {err:.3e}")


@pytest.mark.parametrize("dt,W", [("fp16", -1), ("bf16", 512)])
def test_decode_poisoned_workspace(dt, W):
    """The split-KV decode (with a window: full caches, so the fused eviction
    and its halo rows run too) on a workspace that holds NaN bits everywhere
    but the merge counters: the cross-workgroup merge reads only partials this
    call wrote."""
    import torch
    from test_prefill_plan import align256, cdiv, lib_workspace
    B, H, Hkv, D, M = 16, 32, 8, 128, 512
    lens = [M if W > 0 else M - 1] * 8 + list(range(37, M, 60))   # no window: room for one
    case = gi.make_case("poisoned-decode", dt, B, 1, H, Hkv, D, M, lens, 77, window=W,
                        rotary=True, rotary_rows=M + 1)
    total = lib_workspace(B, 1, H, Hkv, M, W, {"fp16": 1, "bf16": 2}[dt])
    ws = torch.full((total,), 0xFF, dtype=torch.uint8, device="cuda")
    ws[:align256(B * Hkv * cdiv(H // Hkv, 16) * 4)] = 0                  # decode merge counters
    say(f"[gpu] poisoned workspace decode {dt} W={W}: {total} bytes")
    st, want, kc, vc, _ = O.gqa_attention(case, "decode")
    assert st == O.OK
    dev = DevCase(case)
    out = dev.run("decode", workspace=ws)
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, "poisoned decode k_cache")
    assert_bits_equal(gv, vc, "poisoned decode v_cache")
    err = assert_close(out_f64(out, dt), want, dt, "poisoned decode")
    say(f"[gpu]   max abs error {err:.3e}")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_windowed_chunks_rolling(dt):
    """Chunks of S > 1 tokens into full W-slot caches, continued in place on
    the GPU; each step against the oracle run on the previous oracle state."""
    rng = np.random.default_rng(31)
    B, H, Hkv, D, M = 4, 16, 4, 128, 1024
    lens = [1024, 1000, 600, 1024]
    case = gi.make_case("chunks", dt, B, 96, H, Hkv, D, M, lens, 12, window=M, rotary=True,
                        rotary_rows=M + 4 * 128 + 300)
    # buffer row 0 holds absolute position 300 + (rows the windows dropped before)
    case.position_offset = np.array([300, 0, 17, 5], np.int32)
    dev = DevCase(case)
    ptr = dev.k_cache.data_ptr()
    for step in range(3):
        S = [96, 128, 40][step]
        say(f"[gpu] windowed chunks {dt} step {step}: S={S} lens={case.seqlens_k.tolist()}")
        st, want, kc, vc, after = O.gqa_attention(case, "prefill")
        assert st == O.OK
        out = dev.run("prefill")
        gk, gv = dev.caches()
        assert_bits_equal(gk, kc, f"chunk step {step} k_cache")
        assert_bits_equal(gv, vc, f"chunk step {step} v_cache")
        err = assert_close(out_f64(out, dt), want, dt, f"chunk step {step}")
        say(f"[gpu]   max abs error {err:.3e}")
        assert dev.k_cache.data_ptr() == ptr
        # next chunk: fresh Q/K/V, the lengths the call left
        nxt = case.copy()
        nxt.new_tokens = [96, 128, 40, 1][step + 1]
        nxt.q = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, H * D)), dt)
        nxt.k_new = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, Hkv * D)), dt)
        nxt.v_new = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, Hkv * D)), dt)
        # the rows this step dropped move the absolute position of row 0
        nxt.position_offset = (case.position_offset + case.seqlens_k + S - after).astype(np.int32)
        nxt.k_cache, nxt.v_cache, nxt.seqlens_k = kc, vc, after.astype(np.int32)
        case = nxt
        cache_k, cache_v = dev.k_cache, dev.v_cache
        dev = DevCase(case)
        dev.k_cache, dev.v_cache = cache_k, cache_v


POSITION_OFFSETS = [
    # dtype, B, H, Hkv, D, M, W, lens, chunk sizes per step, greedy
    ("bf16", 3, 16, 4, 128, 256, 256, [256, 256, 100], [1, 1, 1, 1], 0),       # fused eviction decode
    ("fp16", 2, 8, 2, 128, 300, 200, [300, 280], [1, 1, 1], 1),                # greedy, eviction kernel
    ("fp16", 2, 28, 4, 128, 512, 512, [512, 400], [64, 1, 33, 1], 0),         # chunks and decodes
    ("fp32", 2, 4, 2, 8, 40, 40, [40, 33], [1, 7, 1], 0),                      # plain kernel
    ("bf16", 66, 4, 2, 128, 64, 64, [64 if i % 2 else (7 * i) % 60 for i in range(66)], [3, 1], 0),
]


@pytest.mark.parametrize("spec", POSITION_OFFSETS,
                         ids=[f"{s[0]}-B{s[1]}-{i}" for i, s in enumerate(POSITION_OFFSETS)])
def test_rolling_window_with_rotary_position_offsets(spec):
    """Rolling steps into full window caches with rotary on throughout: row 0
    of each buffer holds absolute position offset_b, which grows by the rows
    each step drops, so new tokens keep rotating at their positions in the
    whole history ([P2] para 1 positions with the sliding-window follow-up's
    eviction). Every step against the oracle on the previous oracle state;
    66 sequences take the prefill kernel's device-read offsets."""
    dt, B, H, Hkv, D, M, W, lens, chunks, greedy = spec
    seed = sum(map(ord, repr(spec))) % 1000
    rng = np.random.default_rng(seed)
    case = gi.make_case("offsets", dt, B, chunks[0], H, Hkv, D, M, lens, seed, window=W,
                        rotary=True, rotary_rows=2000)
    case.greedy_eviction = greedy
    case.position_offset = rng.integers(0, 500, B).astype(np.int32)
    dev = DevCase(case)
    cache_k, cache_v = dev.k_cache, dev.v_cache
    for step, S in enumerate(chunks):
        entry = "decode" if S == 1 else "prefill"
        say(f"[gpu] offsets {spec[:7]} step {step}: S={S} lens={case.seqlens_k.tolist()[:6]} "
            f"offsets={case.position_offset.tolist()[:6]}")
        st, want, kc, vc, after = O.gqa_attention(case, entry)
        assert st == O.OK
        out = dev.run(entry)
        gk, gv = dev.caches()
        assert_bits_equal(gk, kc, f"offsets step {step} k_cache")
        assert_bits_equal(gv, vc, f"offsets step {step} v_cache")
        err = assert_close(out_f64(out, dt), want, dt, f"offsets step {step}")
        say(f"[gpu]   max abs error {err:.3e}")
        if step + 1 == len(chunks):
            break
        nxt = case.copy()
        nxt.new_tokens = chunks[step + 1]
        nxt.q = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, H * D)), dt)
        nxt.k_new = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, Hkv * D)), dt)
        nxt.v_new = gi.to_bits(rng.standard_normal((B, nxt.new_tokens, Hkv * D)), dt)
        nxt.position_offset = (case.position_offset + case.seqlens_k + S - after).astype(np.int32)
        nxt.k_cache, nxt.v_cache, nxt.seqlens_k = kc, vc, after.astype(np.int32)
        case = nxt
        dev = DevCase(case)
        dev.k_cache, dev.v_cache = cache_k, cache_v


def test_causal_prefill_full_size():
    """The causal prefill workload in full: every output row of every
    sequence and head (all 32 row blocks of each (sequence, kv head)) against
    the oracle, and both caches bit for bit."""
    check_full(gi.workload("causal-prefill-bf16"), "prefill", "causal prefill (every row)")


def test_ragged_continuation_full_size():
    """The ragged continuation workload in full: every output row (each
    (sequence, kv head) has 128 x 7 query rows in 4 row blocks, whose key
    ranges the split plan cuts over up to 4 workgroups) against the oracle,
    and both caches bit for bit."""
    case = gi.workload("ragged-continuation-fp16")
    check_full(case, "prefill", f"ragged continuation (every row) lens={case.seqlens_k.tolist()}")


# the shapes of the decode, window, causal prefill and continuation
# workloads at head size 64: every output against the oracle, both caches
# bit for bit
HEAD64_FULL = [
    ("decode", "fp16", 16, 1, 32, 8, 4096, "U512-4095", -1, False),
    ("decode", "bf16", 8, 1, 32, 8, 4096, "full", 4096, False),
    ("prefill", "bf16", 4, 2048, 32, 8, 4096, "empty", -1, True),
    ("prefill", "fp16", 8, 128, 28, 4, 4096, "U0-3072", -1, False),
]


@pytest.mark.parametrize("spec", HEAD64_FULL, ids=["decode", "window", "causal", "continuation"])
def test_head_size_64_full_shapes(spec):
    entry, dt, B, S, H, Hkv, M, kind, W, rot = spec
    seed = sum(map(ord, repr(spec))) % 1000
    rng = np.random.default_rng(seed)
    if kind == "full":
        lens = [M] * B
    elif kind == "empty":
        lens = [0] * B
    else:
        lo, hi = (int(x) for x in kind[1:].split("-"))
        lens = rng.integers(lo, hi + 1, B).tolist()
    case = gi.make_case("head64-full", dt, B, S, H, Hkv, 64, M, lens, seed, window=W, rotary=rot,
                        rotary_rows=(M if rot else None))
    check_full(case, entry, f"head size 64 {spec} lens={lens}")


# --------------------------------------------------------------------------
# no shared state: two calls in flight on two streams, own workspaces
# --------------------------------------------------------------------------

def test_concurrent_streams_with_own_workspaces():
    """The library keeps no state between calls: two decodes and two
    prefills enqueued on two streams (default priority) at once, each with
    its own workspace, give exactly the outputs and caches of the same calls
    made one after the other."""
    import torch
    import grouped_query_kv_amd as gqa
    cases = [gi.make_case("streams", "fp16", 4, 1, 32, 8, 128, 2048, [2047, 5, 900, 1500], 61),
             gi.make_case("streams", "bf16", 3, 1, 16, 4, 128, 1024, [100, 1023, 512], 62),
             gi.make_case("streams", "bf16", 2, 40, 8, 2, 128, 2048, [1900, 0], 63, rotary=True,
                          rotary_rows=2100),
             gi.make_case("streams", "fp16", 2, 70, 28, 4, 128, 512, [300, 17], 64)]
    entries = ["decode", "decode", "prefill", "prefill"]

    def ws_for(c):
        n = gqa.gqa_workspace_bytes(c.batch, c.new_tokens, c.num_heads, c.kv_num_heads, c.head_size,
                                    c.max_seq_len, gqa.GQA_FP16 if c.dtype == "fp16" else gqa.GQA_BF16)
        return torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")

    # one after the other on the current stream
    ref = []
    for c, e in zip(cases, entries):
        d = DevCase(c)
        out = d.run(e, workspace=ws_for(c))
        torch.cuda.synchronize()
        ref.append((to_bits(out), *d.caches()))
    # all four in flight, alternating between two streams
    say("[gpu] four calls on two streams")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    devs = [DevCase(c) for c in cases]
    wss = [ws_for(c) for c in cases]
    torch.cuda.synchronize()
    outs = []
    for k, (d, e, w) in enumerate(zip(devs, entries, wss)):
        with torch.cuda.stream(streams[k % 2]):
            outs.append(d.run(e, workspace=w))
    torch.cuda.synchronize()
    for k, d in enumerate(devs):
        gk, gv = d.caches()
        assert_bits_equal(to_bits(outs[k]), ref[k][0], f"stream call {k} out")
        assert_bits_equal(gk, ref[k][1], f"stream call {k} k_cache")
        assert_bits_equal(gv, ref[k][2], f"stream call {k} v_cache")


# --------------------------------------------------------------------------
# prefill then decodes equals a one-shot prefill (the worked example's story)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64), ("fp32", 8)])
def test_prefill_then_decodes_match_one_shot(dt, D):
    import torch
    n, k = 70, 5
    full = gi.make_case("inc", dt, 2, n + k, 8, 2, D, 128, [0, 0], 77, rotary=True, rotary_rows=128)
    st, ref, _, _, _ = O.gqa_attention(full)
    part = full.copy()
    part.new_tokens = n
    part.q, part.k_new, part.v_new = full.q[:, :n], full.k_new[:, :n], full.v_new[:, :n]
    say(f"[gpu] incremental {dt}: prefill {n} then {k} decodes")
    dev = DevCase(part)
    out = dev.run("prefill")
    assert_close(out_f64(out, dt), ref[:, :n], dt, "prefill part")
    for s in range(k):
        step = full.copy()
        step.new_tokens = 1
        step.q, step.k_new, step.v_new = (x[:, n + s:n + s + 1].copy() for x in (full.q, full.k_new, full.v_new))
        dev.case = step
        dev.q, dev.k_new, dev.v_new = (to_dev(getattr(step, a), dt) for a in ("q", "k_new", "v_new"))
        dev.set_lengths([n + s, n + s])
        out = dev.run("decode")
        assert_close(out_f64(out, dt)[:, 0], ref[:, n + s], dt, f"decode {s}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("dt,D,lens", [("fp16", 128, [0, 0]), ("bf16", 128, [0, 0]),
                                       ("bf16", 64, [0, 0]), ("fp32", 8, [0, 0])])
def test_prefill_then_chunks_match_one_shot(dt, D, lens):
    """A prefill of n tokens followed by continuation chunks of 37 and 90
    tokens gives, for each chunk, the same rows as a one-shot prefill of all
    of them (chunked continuation, as in the ragged continuation workload)."""
    import torch
    n, chunks = 200, [37, 90]
    tot = n + sum(chunks)
    full = gi.make_case("inc-chunks", dt, 2, tot, 28, 4, D, 512, lens, 78, rotary=True,
                        rotary_rows=512)
    st, ref, kc_ref, vc_ref, _ = O.gqa_attention(full)
    assert st == O.OK
    part = full.copy()
    part.new_tokens = n
    part.q, part.k_new, part.v_new = full.q[:, :n], full.k_new[:, :n], full.v_new[:, :n]
    say(f"[gpu] incremental {dt}: prefill {n} then chunks {chunks}")
    dev = DevCase(part)
    out = dev.run("prefill")
    assert_close(out_f64(out, dt), ref[:, :n], dt, "prefill part")
    start = n
    for c in chunks:
        step = full.copy()
        step.new_tokens = c
        step.q, step.k_new, step.v_new = (x[:, start:start + c].copy()
                                          for x in (full.q, full.k_new, full.v_new))
        dev.case = step
        dev.q, dev.k_new, dev.v_new = (to_dev(getattr(step, a), dt) for a in ("q", "k_new", "v_new"))
        dev.set_lengths([start, start])
        out = dev.run("prefill")
        assert_close(out_f64(out, dt), ref[:, start:start + c], dt, f"chunk at {start}")
        start += c
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc_ref, "chunked k_cache")
    assert_bits_equal(gv, vc_ref, "chunked v_cache")
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# split prefill: the workspace counters return to zero, repeated calls agree
# --------------------------------------------------------------------------

def test_split_prefill_repeated_calls_share_workspace(gpu):
    torch = gpu
    import grouped_query_kv_amd as gqa
    case = gi.make_case("split-repeat", "fp16", 3, 40, 8, 2, 128, 2048, [0, 700, 1999], seed=11,
                        rotary=True, rotary_rows=2048 + 40)
    st, want, kc, vc, _ = O.gqa_attention(case, "prefill")
    assert st == O.OK
    dev = DevCase(case)
    n = gqa.gqa_workspace_bytes(3, 40, 8, 2, 128, 2048, gqa.GQA_FP16)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    outs = []
    for i in range(3):
        say(f"[gpu] split prefill, call {i} on one workspace of {n} bytes")
        outs.append(out_f64(dev.run("prefill", workspace=ws), case.dtype))
        torch.cuda.synchronize()
        # the per-row-block split counters sit at the end of the workspace
        assert int(ws[-256:].count_nonzero()) == 0, "split counters not back to zero"
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, "k_cache")
    assert_bits_equal(gv, vc, "v_cache")
    for o in outs:
        assert_close(o, want, case.dtype, "split prefill")
        assert np.array_equal(o, outs[0]), "the merge order depends on arrival"


# --------------------------------------------------------------------------
# seeded random combinations of the features (fixed seeds: a regular test)
# --------------------------------------------------------------------------

def _random_case(k, head_size=None, salt=0):
    """Case k of the random feature mix; with `head_size`, a 2-byte dtype at
    that head size (its own seeds through `salt`)."""
    k = k + salt
    rng = np.random.default_rng(1000 + k)
    if head_size is None:
        dt = ["fp16", "bf16", "fp32"][rng.integers(0, 3)]
        D = 128 if dt != "fp32" and rng.random() < 0.8 else int(rng.choice([8, 64, 128]))
    else:
        dt = ["fp16", "bf16"][rng.integers(0, 2)]
        D = head_size
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 7]))
    B = int(rng.integers(1, 5))
    M = int(rng.choice([64, 96, 200, 320]))
    S = 1 if rng.random() < 0.4 else int(rng.integers(2, min(M, 80) + 1))
    window = -1
    greedy = 0
    if rng.random() < 0.5:
        window = int(rng.integers(max(1, S), M + 1))
        greedy = int(rng.random() < 0.4 and window < M)
    if window > 0:
        lens = [int(rng.integers(0, M + 1)) for _ in range(B)]
    else:
        lens = [int(rng.integers(0, M - S + 1)) for _ in range(B)]
    rot = bool(rng.random() < 0.5)
    inter = int(rot and rng.random() < 0.3)
    case = gi.make_case("random", dt, B, S, G * Hkv, Hkv, D, M, lens, 2000 + k, window=window,
                        rotary=rot, interleaved=inter, rotary_rows=(M + S if rot else None))
    case.greedy_eviction = greedy
    if rng.random() < 0.3:
        T = int((np.asarray(lens) + S).max()) + int(rng.integers(0, 5))
        Bb = B if rng.random() < 0.5 else 1
        Hb = G * Hkv if rng.random() < 0.5 else 1
        case.attention_bias = gi.to_bits(rng.standard_normal((Bb, Hb, S, T)), dt)
    present_rows = int(max(lens)) + int(rng.integers(0, 8)) if rng.random() < 0.25 else None
    orng = np.random.default_rng(5000 + k)     # own generator: the draws above stay as they were
    if rot and orng.random() < 0.5:
        case.position_offset = orng.integers(0, 40, B).astype(np.int32)
        case.cos, case.sin = gi.rope_tables(M + S + 40, D // 2)
    return case, present_rows


@pytest.mark.parametrize("k", range(40))
def test_random_feature_combinations(k):
    _check_random(k, 0, *_random_case(k))


# the same mix at head size 64, where fp16/bf16 run the MFMA kernels too
@pytest.mark.parametrize("k", range(24))
def test_random_feature_combinations_head_size_64(k):
    _check_random(k, 10000, *_random_case(k, head_size=64, salt=10000))


def _check_random(k, salt, case, present_rows):
    import grouped_query_kv_amd as gqa
    entry = "decode" if case.new_tokens == 1 else "prefill"
    desc = (f"random {k} (salt {salt}): {case.dtype} B={case.batch} S={case.new_tokens} H={case.num_heads} "
            f"Hkv={case.kv_num_heads} D={case.head_size} M={case.max_seq_len} W={case.local_window_size} "
            f"greedy={case.greedy_eviction} rot={case.cos is not None} "
            f"bias={None if case.attention_bias is None else case.attention_bias.shape} "
            f"offsets={None if case.position_offset is None else case.position_offset.tolist()} "
            f"present={present_rows} lens={list(case.seqlens_k)}")
    if present_rows is None:
        check_full(case, entry, desc)
        return
    say(f"[gpu] {desc}")
    rng = np.random.default_rng(3000 + k + salt)
    past_k = gi.fill_cache(rng, case.batch, case.kv_num_heads, present_rows, case.head_size,
                           case.seqlens_k, case.dtype)
    past_v = gi.fill_cache(rng, case.batch, case.kv_num_heads, present_rows, case.head_size,
                           case.seqlens_k, case.dtype)
    st, want, kc, vc, _ = O.gqa_attention_present(case, past_k, past_v)
    assert st == O.OK
    dev = DevCase(case)
    fn = gqa.gqa_attention_decode if entry == "decode" else gqa.gqa_attention_prefill
    out = fn(dev.q, dev.k_new, dev.v_new, to_dev(past_k, case.dtype), to_dev(past_v, case.dtype),
             dev.lens_host, dev.lens_dev, scale=case.scale, local_window_size=case.local_window_size,
             cos_cache=dev.cos, sin_cache=dev.sin, rotary_interleaved=case.rotary_interleaved,
             present_key=dev.k_cache, present_value=dev.v_cache,
             greedy_eviction=bool(case.greedy_eviction), attention_bias=dev.bias,
             position_offset=dev.off_host, position_offset_dev=dev.off_dev)
    gk, gv = dev.caches()
    assert_bits_equal(gk, kc, f"{desc} present k")
    assert_bits_equal(gv, vc, f"{desc} present v")
    err = assert_close(out_f64(out, case.dtype), want, case.dtype, desc)
    say(f"[gpu]   max abs error {err:.3e}")


def test_stream_read_yardstick_runs():
    """The read yardstick (not part of the op) runs on a device buffer and
    leaves it as it was."""
    import torch
    import grouped_query_kv_amd as gqa
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")
    before = buf.clone()
    gqa.gqa_stream_read(buf)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)

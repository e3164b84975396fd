"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties the oracle to something it does not compute: a scalar-loop
brute force, torch's float64 scaled_dot_product_attention on the special
case past = 0, closed forms, textbook rounding cases, the shapes of the
worked example in the rocMLIR "KV Cache" discussion, and the invariants the
op pages state (one buffer stays in place, overflow fails, the window keeps
the most recent tokens contiguously).
"""
import json
import math
import os

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import brute
from oracle import gqa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(dtype="fp32", B=2, S=3, H=4, Hkv=2, D=4, M=12, lens=(0, 5), seed=0, **kw):
    return gi.make_case("tiny", dtype, B, S, H, Hkv, D, M, list(lens), seed, **kw)


def f64_cache(case, bits):
    return O.to_f64(bits, case.dtype)


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

TINY = [
    dict(dtype="fp32"),
    dict(dtype="fp16", H=6, Hkv=2, lens=(7, 0)),
    dict(dtype="bf16", H=3, Hkv=3, D=2, lens=(1, 9)),
    dict(dtype="fp32", H=4, Hkv=1, S=1, lens=(11, 0)),
    dict(dtype="fp16", rotary=True, lens=(2, 6)),
    dict(dtype="bf16", rotary=True, interleaved=1, D=6, H=2, Hkv=1, lens=(4, 3)),
    dict(dtype="fp32", window=3, lens=(6, 2)),
    dict(dtype="fp16", window=12, S=1, lens=(12, 12)),          # full cache: evict 1
    dict(dtype="bf16", window=5, S=4, lens=(12, 10)),           # S>1 with eviction
    dict(dtype="fp32", window=12, S=12, lens=(12, 3)),          # whole buffer turns over
    dict(dtype="fp32", scale=0.37, lens=(3, 3)),
]


@pytest.mark.parametrize("kw", TINY, ids=[str(i) for i in range(len(TINY))])
def test_brute_force_matches_oracle(kw):
    case = tiny(**kw)
    st, out, kc, vc, _ = O.gqa_attention(case)
    assert st == O.OK
    bout, bkc, bvc = brute.brute_attention(case)
    np.testing.assert_allclose(out.reshape(case.batch, case.new_tokens, -1), np.array(bout),
                               rtol=0, atol=1e-12)
    assert np.array_equal(kc, np.array(bkc, dtype=kc.dtype))
    assert np.array_equal(vc, np.array(bvc, dtype=vc.dtype))


@pytest.mark.parametrize("step", [1, 2])
def test_brute_force_matches_oracle_on_worked_example(step):
    case = gi.workload("worked-example", step=step)
    st, out, kc, vc, _ = O.gqa_attention(case)
    assert st == O.OK
    bout, bkc, bvc = brute.brute_attention(case)
    np.testing.assert_allclose(out, np.array(bout), rtol=0, atol=1e-12)
    assert np.array_equal(kc, np.array(bkc, dtype=kc.dtype))


# --------------------------------------------------------------------------
# library routine on the special case past = 0
# --------------------------------------------------------------------------

@pytest.mark.parametrize("H,Hkv,S,D", [(4, 2, 9, 8), (6, 3, 17, 16), (7, 7, 5, 4), (8, 1, 12, 32)])
def test_past_zero_equals_torch_sdpa(H, Hkv, S, D):
    torch = pytest.importorskip("torch")
    case = tiny("fp32", B=2, S=S, H=H, Hkv=Hkv, D=D, M=S + 3, lens=(0, 0), seed=H * 100 + S)
    st, out, _, _, _ = O.gqa_attention(case)
    assert st == O.OK
    q = torch.from_numpy(O.to_f64(case.q, "fp32")).view(2, S, H, D).transpose(1, 2)
    k = torch.from_numpy(O.to_f64(case.k_new, "fp32")).view(2, S, Hkv, D).transpose(1, 2)
    v = torch.from_numpy(O.to_f64(case.v_new, "fp32")).view(2, S, Hkv, D).transpose(1, 2)
    k = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    v = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(q.contiguous(), k, v, is_causal=True)
    ref = ref.transpose(1, 2).reshape(2, S, H * D).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms and invariants of the softmax
# --------------------------------------------------------------------------

def test_weights_sum_to_one_and_masked_are_zero():
    rng = np.random.default_rng(3)
    S, T, D, past = 5, 9, 6, 4
    allowed = O.allowed_mask(S, T, past, W=3)
    _, p = O.attend_one(rng.standard_normal((S, D)), rng.standard_normal((T, D)),
                        rng.standard_normal((T, D)), allowed, 0.5, return_weights=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(p[~allowed] == 0.0)
    assert np.all(p[allowed] > 0.0)
    # each query sees itself and the W - 1 keys before it: the mask's structure
    assert allowed.sum(axis=1).tolist() == [3] * S
    assert all(allowed[i, past + i] and not allowed[i, past + i + 1] for i in range(S - 1))


def test_two_keys_closed_form():
    # scores 0 and ln 3 (scale 1): weights 1/4, 3/4
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    v = np.array([[4.0, 0.0], [0.0, 8.0]])
    o = O.attend_one(q, k, v, np.ones((1, 2), bool), 1.0)
    np.testing.assert_allclose(o, [[1.0, 6.0]], rtol=0, atol=1e-14)


def test_constant_values_give_that_value():
    case = tiny("fp16", S=4, lens=(3, 7), window=5)
    D = case.head_size
    row = gi.to_bits(np.linspace(-1, 1, D), "fp16")
    case.v_new[:] = np.tile(row, case.kv_num_heads)
    case.v_cache[:, :, :] = np.where(np.isnan(O.to_f64(case.v_cache, "fp16")), case.v_cache, row)
    st, out, _, _, _ = O.gqa_attention(case)
    want = np.tile(O.to_f64(row, "fp16"), case.num_heads)
    np.testing.assert_allclose(out, np.broadcast_to(want, out.shape), rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_visible_values():
    case = tiny("fp32", S=3, lens=(4, 8), window=4)
    case.q[:] = 0
    st, out, kc, vc, _ = O.gqa_attention(case)
    B, S, H, Hkv, D = 2, 3, 4, 2, 4
    G = H // Hkv
    vf = O.to_f64(vc, "fp32")
    for b in range(B):
        L = int(case.seqlens_k[b])
        for i in range(S):
            p = L + i
            lo = max(0, p - 4 + 1)
            for h in range(H):
                want = vf[b, h // G, lo:p + 1].mean(axis=0)
                np.testing.assert_allclose(out[b, i, h * D:(h + 1) * D], want, rtol=0, atol=1e-14)


def test_first_token_sees_only_itself():
    case = tiny("bf16", S=4, lens=(0, 0))
    st, out, _, _, _ = O.gqa_attention(case)
    D, G = case.head_size, case.num_heads // case.kv_num_heads
    v0 = O.to_f64(case.v_new[:, 0], "bf16")          # [B, Hkv*D]
    for h in range(case.num_heads):
        g = h // G
        assert np.array_equal(out[:, 0, h * D:(h + 1) * D], v0[:, g * D:(g + 1) * D])


def test_gqa_equals_mha_on_expanded_kv():
    case = tiny("fp32", B=2, S=3, H=6, Hkv=2, D=4, M=10, lens=(2, 5), seed=11)
    G = 3
    mha = case.copy()
    mha.kv_num_heads = 6
    kn = case.k_new.reshape(2, 3, 2, 4)
    vn = case.v_new.reshape(2, 3, 2, 4)
    mha.k_new = np.repeat(kn, G, axis=2).reshape(2, 3, 24)
    mha.v_new = np.repeat(vn, G, axis=2).reshape(2, 3, 24)
    mha.k_cache = np.repeat(case.k_cache, G, axis=1)
    mha.v_cache = np.repeat(case.v_cache, G, axis=1)
    _, a, _, _, _ = O.gqa_attention(case)
    _, b, _, _, _ = O.gqa_attention(mha)
    assert np.array_equal(a, b)


def test_lse_merge_of_any_partition_equals_unsplit():
    rng = np.random.default_rng(5)
    T, D = 37, 8
    q, k, v = rng.standard_normal(D), rng.standard_normal((T, D)), rng.standard_normal((T, D))
    allowed = np.ones(T, bool)
    allowed[:4] = False                                   # a window start
    ref = O.attend_one(q[None], k, v, allowed[None], 0.3)[0]
    for trial in range(20):
        cuts = np.sort(rng.choice(np.arange(1, T), size=rng.integers(1, 8), replace=False))
        parts = []
        for lo, hi in zip(np.r_[0, cuts], np.r_[cuts, T]):
            a = np.zeros(T, bool)
            a[lo:hi] = allowed[lo:hi]
            parts.append(O.partial_attention(q, k, v, a, 0.3))
        np.testing.assert_allclose(O.lse_merge(parts), ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# rotary
# --------------------------------------------------------------------------

def test_rotary_position_zero_is_identity_and_roundtrip_exact():
    cos, sin = gi.rope_tables(8, 4)
    assert cos[0].tolist() == [1.0] * 4 and sin[0].tolist() == [0.0] * 4
    case = tiny("bf16", rotary=True, lens=(0, 0), S=1)
    q0 = O.rotated_bits(case, case.q, case.num_heads)
    assert np.array_equal(q0, case.q.reshape(2, 1, 4, 4).transpose(0, 2, 1, 3))


def test_rotary_closed_form_two_dims():
    # D = 2: (1, 0) rotated by angle a is (cos a, sin a); (0, 1) -> (-sin a, cos a)
    a = 0.7
    cos = np.array([[1.0], [math.cos(a)]])
    sin = np.array([[0.0], [math.sin(a)]])
    y = O.rotary_f64(np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([1, 1]), cos, sin, 0)
    np.testing.assert_allclose(y, [[math.cos(a), math.sin(a)], [-math.sin(a), math.cos(a)]],
                               rtol=0, atol=1e-16)


def test_rotary_preserves_pair_norms_and_relative_positions():
    rng = np.random.default_rng(9)
    D, P = 16, 64
    inv = 10000.0 ** (-(2.0 * np.arange(D // 2)) / D)
    ang = np.arange(P)[:, None] * inv[None]
    cos, sin = np.cos(ang), np.sin(ang)            # fp64 tables for exact identities
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m in (0, 5, 17):
        y = O.rotary_f64(q[None], np.array([m]), cos, sin, 0)[0]
        np.testing.assert_allclose(y[:8] ** 2 + y[8:] ** 2, q[:8] ** 2 + q[8:] ** 2, rtol=1e-13)
    dots = {}
    for m, n in [(3, 1), (10, 8), (40, 38), (7, 7), (30, 30)]:
        rq = O.rotary_f64(q[None], np.array([m]), cos, sin, 0)[0]
        rk = O.rotary_f64(k[None], np.array([n]), cos, sin, 0)[0]
        dots.setdefault(m - n, []).append(rq @ rk)
    for vals in dots.values():
        np.testing.assert_allclose(vals, vals[0], rtol=1e-12)


def test_rotary_interleaved_is_permuted_rotate_half():
    rng = np.random.default_rng(4)
    D = 8
    cos, sin = gi.rope_tables(16, D // 2)
    x = rng.standard_normal((3, D))
    pos = np.array([2, 9, 15])
    perm = np.r_[np.arange(0, D, 2), np.arange(1, D, 2)]        # interleaved -> halves
    a = O.rotary_f64(x, pos, cos, sin, 1)
    b = O.rotary_f64(x[:, perm], pos, cos, sin, 0)
    assert np.array_equal(a[:, perm], b)


def test_rounding_chain_textbook_cases():
    with open(os.path.join(GOLDEN, "rne_cases.json")) as f:
        cases = json.load(f)
    for dt in ("bf16", "fp16"):
        for c in cases[dt]:
            got = int(O.round_f64_to_dtype(np.array([c["x"]]), dt)[0])
            assert got == int(c["bits"], 16), (dt, c)
            assert O.to_f64(np.array([got], np.uint16), dt)[0] == O.to_f64(
                np.array([int(c["bits"], 16)], np.uint16), dt)[0]


def test_rotary_products_are_exact_in_fp64():
    # every dtype significand (<= 24 bits) times an fp32 significand fits in 53 bits,
    # so x*c in fp64 equals the exact rational product: check with fractions
    from fractions import Fraction
    rng = np.random.default_rng(2)
    xs = rng.standard_normal(50).astype(np.float32).astype(np.float64)
    cs = rng.standard_normal(50).astype(np.float32).astype(np.float64)
    for x, c in zip(xs, cs):
        assert Fraction(x * c) == Fraction(x) * Fraction(c)


# --------------------------------------------------------------------------
# shared buffer: append, overflow, eviction
# --------------------------------------------------------------------------

def test_append_writes_exactly_the_new_rows_by_index_code():
    B, S, Hkv, D, M = 2, 3, 2, 4, 10
    case = tiny("fp16", B=B, S=S, H=4, Hkv=Hkv, D=D, M=M, lens=(0, 7))
    code = np.zeros((B, S, Hkv * D))
    for b in range(B):
        for i in range(S):
            for g in range(Hkv):
                for d in range(D):
                    code[b, i, g * D + d] = ((b * S + i) * Hkv + g) * D + d
    case.k_new = gi.to_bits(code, "fp16")
    case.v_new = gi.to_bits(-code, "fp16")
    st, kc, vc = O.gqa_append_kv(case)
    assert st == O.OK
    kf, vf = O.to_f64(kc, "fp16"), O.to_f64(vc, "fp16")
    for b in range(B):
        L = int(case.seqlens_k[b])
        for g in range(Hkv):
            for t in range(M):
                if L <= t < L + S:
                    i = t - L
                    want = np.array([((b * S + i) * Hkv + g) * D + d for d in range(D)], float)
                    assert np.array_equal(kf[b, g, t], want)
                    assert np.array_equal(vf[b, g, t], -want)
                else:
                    assert np.array_equal(kc[b, g, t], case.k_cache[b, g, t])
                    assert np.array_equal(vc[b, g, t], case.v_cache[b, g, t])


@pytest.mark.parametrize("entry", ["append", "prefill"])
def test_overflow_fails_and_leaves_buffer(entry):
    case = tiny("bf16", S=3, M=12, lens=(9, 4))          # 9 + 3 == M: fits
    st = O.gqa_append_kv(case)[0] if entry == "append" else O.gqa_attention(case)[0]
    assert st == O.OK
    case.seqlens_k = np.array([10, 4], np.int32)          # 10 + 3 > M
    if entry == "append":
        st, kc, vc = O.gqa_append_kv(case)
    else:
        st, _, kc, vc, _ = O.gqa_attention(case)
    assert st == O.NO_ROOM
    assert np.array_equal(kc, case.k_cache) and np.array_equal(vc, case.v_cache)


def test_validation_rules():
    base = tiny("fp32")
    bad = [
        dict(num_heads=3),                      # H % Hkv != 0
        dict(new_tokens=0, _entry="prefill"),
        dict(local_window_size=0),
        dict(local_window_size=13),             # W > M
        dict(seqlens_k=np.array([-1, 0], np.int32)),
        dict(seqlens_k=np.array([13, 0], np.int32)),
        dict(head_size=257),
        dict(new_tokens=2, _entry="decode"),
    ]
    for kw in bad:
        c = base.copy()
        entry = kw.pop("_entry", "prefill")
        for k, v in kw.items():
            setattr(c, k, v)
        assert O.validate(c, entry) == O.INVALID, kw
    c = tiny("fp16", D=5, H=2, Hkv=1, rotary=False)
    c.cos = np.ones((20, 2), np.float32)
    c.sin = np.zeros((20, 2), np.float32)
    assert O.validate(c, "prefill") == O.INVALID          # odd head size with rotary
    c = tiny("fp16", rotary=True, M=12, lens=(0, 10), S=2, rotary_rows=11)
    assert O.validate(c, "prefill") == O.INVALID          # position 11 not in the table
    e = tiny("fp32", B=0, lens=())
    assert O.validate(e, "prefill") == O.OK               # empty batch: a no-op


def test_window_keeps_most_recent_tokens_contiguously():
    """Rolling steps against a host-side full history of token codes."""
    rng = np.random.default_rng(21)
    B, Hkv, D, M = 2, 1, 2, 8
    history = [[] for _ in range(B)]
    case = tiny("fp32", B=B, S=1, H=2, Hkv=Hkv, D=D, M=M, lens=(0, 0), window=M)
    serial = 0
    for step in range(30):
        S = int(rng.integers(1, M + 1))
        c = case.copy()
        c.new_tokens = S
        codes = np.zeros((B, S, Hkv * D))
        for b in range(B):
            for i in range(S):
                serial += 1
                codes[b, i, :] = serial
                history[b].append(serial)
        c.k_new = gi.to_bits(codes, "fp32")
        c.v_new = gi.to_bits(-codes, "fp32")
        c.q = gi.to_bits(np.zeros((B, S, 2 * D)), "fp32")
        st, out, kc, vc, lens = O.gqa_attention(c)
        assert st == O.OK
        for b in range(B):
            keep = history[b][-M:]
            assert int(lens[b]) == len(keep)
            got = O.to_f64(kc[b, 0, :len(keep), 0], "fp32")
            assert got.tolist() == [float(x) for x in keep]
            assert (O.to_f64(vc[b, 0, :len(keep), 0], "fp32") == -got).all()
        case.k_cache, case.v_cache, case.seqlens_k = kc, vc, lens.astype(np.int32)


def test_evict_half_then_append_half_equals_whole_op():
    case = tiny("bf16", S=1, M=12, lens=(12, 11), window=12)
    st, out, kc, vc, lens = O.gqa_attention(case, "decode")
    st1, kc1, vc1, l1 = O.gqa_evict_window(case, 1)
    assert st1 == O.OK and l1.tolist() == [11, 11]
    c2 = case.copy()
    c2.k_cache, c2.v_cache, c2.seqlens_k = kc1, vc1, l1
    c2.local_window_size = -1
    st2, kc2, vc2 = O.gqa_append_kv(c2)
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)


def test_windowed_decode_equals_full_history_window_attention():
    """Rolling window decode (cache of M = W slots) vs attention over the whole
    history kept in a large buffer with the same window mask."""
    rng = np.random.default_rng(8)
    W, T0 = 6, 6
    small = tiny("fp32", B=1, S=1, H=2, Hkv=1, D=4, M=W, lens=(T0,), window=W, seed=1)
    big = small.copy()
    big.max_seq_len = 64
    big.k_cache = np.zeros((1, 1, 64, 4), np.uint32)
    big.v_cache = np.zeros((1, 1, 64, 4), np.uint32)
    big.k_cache[:, :, :T0] = small.k_cache[:, :, :T0]
    big.v_cache[:, :, :T0] = small.v_cache[:, :, :T0]
    for step in range(10):
        toks = gi.next_decode_tokens(small, rng)
        for c in (small, big):
            c.q, c.k_new, c.v_new = toks.q, toks.k_new, toks.v_new
        s1, o1, kc1, vc1, l1 = O.gqa_attention(small, "decode")
        s2, o2, kc2, vc2, l2 = O.gqa_attention(big, "decode")
        assert s1 == s2 == O.OK
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
        small.k_cache, small.v_cache, small.seqlens_k = kc1, vc1, l1.astype(np.int32)
        big.k_cache, big.v_cache, big.seqlens_k = kc2, vc2, l2.astype(np.int32)


def _rolling_window_vs_history(steps, S_of, W, T0, rng, use_offset=True, D=4):
    """Chunks into a full W-slot cache (attention before the eviction drops
    the keys early queries still see) vs the same chunks into a buffer long
    enough to keep the whole history, with the same window mask and rotary
    on throughout. The window cache's buffer row 0 holds absolute position
    total - length, which is its position offset; the history buffer's is 0.
    Returns the largest output difference and whether every kept row equals
    the history's row at the same position, bit for bit."""
    small = tiny("fp32", B=2, S=1, H=4, Hkv=2, D=D, M=W, lens=(T0, 3), window=W, seed=2)
    big = small.copy()
    big.max_seq_len = 160
    for name in ("k_cache", "v_cache"):
        arr = np.zeros((2, 2, 160, D), np.uint32)
        arr[:, :, :W] = getattr(small, name)
        setattr(big, name, arr)
    cos, sin = gi.rope_tables(160, D // 2)
    for c in (small, big):
        c.cos, c.sin = cos, sin
    total = np.array([T0, 3])
    worst, rows_equal = 0.0, True
    for step in range(steps):
        S = S_of(step)
        q = gi.to_bits(rng.standard_normal((2, S, 4 * D)), "fp32")
        k = gi.to_bits(rng.standard_normal((2, S, 2 * D)), "fp32")
        v = gi.to_bits(rng.standard_normal((2, S, 2 * D)), "fp32")
        for c in (small, big):
            c.new_tokens, c.q, c.k_new, c.v_new = S, q, k, v
        small.position_offset = (total - small.seqlens_k).astype(np.int32) if use_offset else None
        entry = "decode" if S == 1 else "prefill"
        s1, o1, kc1, vc1, l1 = O.gqa_attention(small, entry)
        s2, o2, kc2, vc2, l2 = O.gqa_attention(big, entry)
        assert s1 == s2 == O.OK
        worst = max(worst, float(np.abs(o1 - o2).max()))
        total = total + S
        assert l1.tolist() == np.minimum(total, W).tolist()
        for b in range(2):
            n = int(l1[b])
            rows_equal &= bool(np.array_equal(kc1[b, :, :n], kc2[b, :, int(l2[b]) - n:int(l2[b])]))
            rows_equal &= bool(np.array_equal(vc1[b, :, :n], vc2[b, :, int(l2[b]) - n:int(l2[b])]))
        small.k_cache, small.v_cache, small.seqlens_k = kc1, vc1, l1.astype(np.int32)
        big.k_cache, big.v_cache, big.seqlens_k = kc2, vc2, l2.astype(np.int32)
    return worst, rows_equal


def test_windowed_chunks_equal_full_history_window_attention():
    """Rolling chunks of 2..W tokens into a full window cache, rotary on at
    every step (absolute positions through the position offset): outputs
    equal full-history window attention, and the kept rows are the history's
    newest rows, rotated at the same positions, bit for bit."""
    rng = np.random.default_rng(9)
    W = 8
    worst, rows_equal = _rolling_window_vs_history(8, lambda _: int(rng.integers(2, W + 1)), W, 8,
                                                   np.random.default_rng(10))
    assert worst <= 1e-13 and rows_equal


def test_windowed_decode_with_rotary_equals_full_history():
    """One-token steps into a full window cache (one row dropped per step),
    rotary on: equal to full-history window attention at the same absolute
    positions."""
    worst, rows_equal = _rolling_window_vs_history(12, lambda _: 1, 6, 6, np.random.default_rng(12))
    assert worst <= 1e-13 and rows_equal


def test_dropping_the_position_offset_breaks_the_history_equivalence():
    """Negative control for the two pins above: rotating at L_b + i alone
    (no offset) once rows have been dropped rotates the new keys at wrong
    positions, and the comparison with the history catches it."""
    worst, rows_equal = _rolling_window_vs_history(6, lambda _: 1, 6, 6, np.random.default_rng(12),
                                                   use_offset=False)
    assert not rows_equal and worst > 1e-6


def test_position_offset_validation():
    base = tiny("fp16", S=2, M=12, lens=(3, 5), rotary=True, rotary_rows=20)
    ok = base.copy()
    ok.position_offset = np.array([0, 13], np.int32)           # 13 + 5 + 2 = 20 rows: fits
    assert O.validate(ok, "prefill") == O.OK
    over = base.copy()
    over.position_offset = np.array([0, 14], np.int32)         # position 20 is past the table
    assert O.validate(over, "prefill") == O.INVALID
    neg = base.copy()
    neg.position_offset = np.array([-1, 0], np.int32)
    assert O.validate(neg, "prefill") == O.INVALID
    short = base.copy()
    short.position_offset = np.array([0], np.int32)            # not one per sequence
    assert O.validate(short, "prefill") == O.INVALID
    # an offset moves every rotary position by the same amount: the rotated K
    # rows of (offset o, past L) are those of (offset 0, past L + o)
    a = tiny("bf16", B=1, S=3, M=16, lens=(2,), rotary=True, rotary_rows=32, seed=5)
    a.position_offset = np.array([7], np.int32)
    b = a.copy()
    b.position_offset = None
    b.seqlens_k = np.array([9], np.int32)
    assert np.array_equal(O.rotated_bits(a, a.k_new, 2), O.rotated_bits(b, b.k_new, 2))


def test_present_mode_by_index_code_and_equals_shared_mode():
    """Separate past/present: present rows [0, L_b) are the past rows, then
    the new rows at L_b.., every other present row untouched, past unchanged
    (each row checked by decoding its index code); the outputs equal the
    shared-mode op on a buffer that holds the same past."""
    B, S, Hkv, D, P, M = 2, 3, 2, 4, 5, 11
    lens = (5, 2)
    case = tiny("fp32", B=B, S=S, H=4, Hkv=Hkv, D=D, M=M, lens=(0, 0), seed=4)
    case.seqlens_k = np.asarray(lens, np.int32)

    def code(b, g, j, d, new):
        return 1000 * b + 100 * g + 10 * j + d + (0.5 if new else 0.0)

    past = np.zeros((B, Hkv, P, D))
    for b, g, j, d in np.ndindex(B, Hkv, P, D):
        past[b, g, j, d] = code(b, g, j, d, False)
    new = np.zeros((B, S, Hkv * D))
    for b, i, g, d in np.ndindex(B, S, Hkv, D):
        new[b, i, g * D + d] = code(b, g, i, d, True)
    pk, pv = gi.to_bits(past, "fp32"), gi.to_bits(-past, "fp32")
    case.k_new, case.v_new = gi.to_bits(new, "fp32"), gi.to_bits(-new, "fp32")
    poison = case.k_cache.copy()
    before = (pk.copy(), pv.copy())
    st, out, kc, vc, after = O.gqa_attention_present(case, pk, pv)
    assert st == O.OK and after.tolist() == [L + S for L in lens]
    assert np.array_equal(pk, before[0]) and np.array_equal(pv, before[1])
    for b, g, j, d in np.ndindex(B, Hkv, M, D):
        L = lens[b]
        got = kc[b, g, j, d]
        if j < L:
            want = O.to_f64(gi.to_bits(np.array(code(b, g, j, d, False)), "fp32"), "fp32")
            assert O.to_f64(got, "fp32") == want
        elif j < L + S:
            assert O.to_f64(got, "fp32") == code(b, g, j - L, d, True)
        else:
            assert got == poison[b, g, j, d]
        assert O.to_f64(vc[b, g, j, d], "fp32") == -O.to_f64(got, "fp32") or j >= L + S
    shared = case.copy()
    shared.k_cache[:, :, :P] = pk
    shared.v_cache[:, :, :P] = pv
    st2, out2, kc2, vc2, _ = O.gqa_attention(shared)
    assert st2 == O.OK
    np.testing.assert_array_equal(out, out2)
    for b in range(B):
        n = lens[b] + S
        assert np.array_equal(kc[b, :, :n], kc2[b, :, :n])
    # a past row count below some length is rejected, present untouched
    short = pk[:, :, :4].copy()
    st3, _, kc3, _, _ = O.gqa_attention_present(case, short, short)
    assert st3 == O.INVALID and np.array_equal(kc3, case.k_cache)


def test_greedy_eviction_matches_default_outputs_and_moves_less():
    """Greedy eviction (cache capacity M > window W): the attention outputs
    equal the default mode's at every step (both keep every key a window can
    reach), the buffer always holds the most recent tokens of the history,
    oldest first, and rows move only in steps whose append would overflow,
    which then leave exactly the W most recent tokens (all new ones if S > W)."""
    rng = np.random.default_rng(17)
    B, Hkv, D, M, W = 2, 1, 2, 12, 5
    history = [[] for _ in range(B)]
    base = tiny("fp32", B=B, S=1, H=2, Hkv=Hkv, D=D, M=M, lens=(0, 0), window=W)
    greedy, default = base.copy(), base.copy()
    greedy.greedy_eviction = 1
    serial, moves = 0, 0
    for step in range(40):
        S = int(rng.integers(1, 7 if step % 5 else 2))
        codes = np.zeros((B, S, Hkv * D))
        for b in range(B):
            for i in range(S):
                serial += 1
                codes[b, i, :] = serial
                history[b].append(serial)
        q = gi.to_bits(rng.standard_normal((B, S, 2 * D)), "fp32")
        outs = []
        for c in (greedy, default):
            c.new_tokens, c.q = S, q
            c.k_new, c.v_new = gi.to_bits(codes, "fp32"), gi.to_bits(-codes, "fp32")
            before = np.asarray(c.seqlens_k).copy()
            st, out, kc, vc, lens = O.gqa_attention(c)
            assert st == O.OK
            outs.append(out)
            if c is greedy:
                for b in range(B):
                    n = int(lens[b])
                    overflow = int(before[b]) + S > M
                    moves += overflow
                    want = max(W, S) if overflow else int(before[b]) + S
                    assert n == min(want, len(history[b]))
                    got = O.to_f64(kc[b, 0, :n, 0], "fp32").tolist()
                    assert got == [float(x) for x in history[b][-n:]]
            c.k_cache, c.v_cache, c.seqlens_k = kc, vc, lens.astype(np.int32)
        np.testing.assert_allclose(outs[0], outs[1], rtol=1e-13, atol=1e-12)
    assert 0 < moves < 40 * B // 2
    # without a window there is nothing to keep: rejected
    bad = base.copy()
    bad.greedy_eviction, bad.local_window_size = 1, -1
    assert O.validate(bad, "prefill") == O.INVALID


# --------------------------------------------------------------------------
# additive attention bias ([P1] sliding-window follow-up gives its shape)
# --------------------------------------------------------------------------

def _with_bias(case, shape_bh=None, T=None, values=None, rng=None):
    B, H, S = case.batch, case.num_heads, case.new_tokens
    Bb, Hb = shape_bh or (B, H)
    T = T or int((np.asarray(case.seqlens_k) + S).max())
    if values is None:
        values = (rng or np.random.default_rng(5)).standard_normal((Bb, Hb, S, T))
    c = case.copy()
    c.attention_bias = gi.to_bits(values, case.dtype)
    return c


@pytest.mark.parametrize("kw,bh", [
    (dict(dtype="fp32"), None),
    (dict(dtype="fp16", H=6, Hkv=2, lens=(7, 0)), (1, 6)),
    (dict(dtype="bf16", S=1, M=8, lens=(8, 3), window=8), (2, 1)),     # decode with eviction
    (dict(dtype="fp32", S=3, M=8, lens=(8, 6), window=5), (1, 1)),     # chunk with eviction
])
def test_bias_brute_force_matches_oracle(kw, bh):
    base = tiny(**kw)
    case = _with_bias(base, bh, T=int((np.asarray(base.seqlens_k) + base.new_tokens).max()) + 2)
    st, out, kc, vc, _ = O.gqa_attention(case, "decode" if case.new_tokens == 1 else "prefill")
    assert st == O.OK
    bout, bk, bv = brute.brute_attention(case)
    np.testing.assert_allclose(out, np.asarray(bout), rtol=0, atol=1e-12)


def test_bias_zero_and_row_constants_change_nothing():
    case = tiny("fp32", S=4, lens=(3, 9), window=6, rotary=True)
    st0, ref, *_ = O.gqa_attention(case)
    T = 13
    zero = _with_bias(case, T=T, values=np.zeros((2, 4, 4, T)))
    np.testing.assert_array_equal(O.gqa_attention(zero)[1], ref)
    # softmax is shift invariant: a constant per (b, h, query) row cancels
    row = np.broadcast_to(np.arange(2 * 4 * 4, dtype=float).reshape(2, 4, 4, 1) - 7.0, (2, 4, 4, T))
    np.testing.assert_allclose(O.gqa_attention(_with_bias(case, T=T, values=row))[1], ref,
                               rtol=0, atol=1e-12)


def test_bias_of_minus_infinity_outside_a_window_is_that_window():
    """-inf on every column below p - W' + 1 equals the window-W' op: the
    bias columns are the keys' positions in past ++ new."""
    case = tiny("fp32", S=5, H=4, Hkv=2, lens=(2, 7), M=16)
    Wp = 3
    T = 12
    _, wanted, *_ = O.gqa_attention(_win(case, Wp))
    # the past lengths differ per sequence: one bias row block per sequence
    vals = np.zeros((2, 1, 5, T))
    for b, L in enumerate(case.seqlens_k):
        for i in range(5):
            vals[b, 0, i, :max(0, L + i - Wp + 1)] = -np.inf
    got = O.gqa_attention(_with_bias(case, (2, 1), T=T, values=vals))[1]
    np.testing.assert_allclose(got, wanted, rtol=0, atol=1e-13)


def _win(case, W):
    c = case.copy()
    c.local_window_size = W
    return c


def test_bias_column_is_the_position_before_eviction():
    """A full window cache takes one token (the oldest row is dropped); a
    large bias on the column of one kept key makes the output that key's V
    row (the weights of the others are below e^-60)."""
    case = tiny("fp32", B=1, S=1, H=2, Hkv=1, D=4, M=6, lens=(6,), window=6, seed=3)
    T = 7
    target = 4                     # position 4 of past ++ new = buffer row 3 after the drop
    vals = np.zeros((1, 1, 1, T))
    vals[0, 0, 0, target] = 80.0
    st, out, kc, vc, lens = O.gqa_attention(_with_bias(case, (1, 1), T=T, values=vals), "decode")
    assert st == O.OK and lens.tolist() == [6]
    want_v = O.to_f64(case.v_cache[0, 0, target], "fp32")
    np.testing.assert_allclose(out[0, 0, :4], want_v, rtol=0, atol=1e-20)
    np.testing.assert_array_equal(O.to_f64(vc[0, 0, target - 1], "fp32"), want_v)


def test_bias_broadcast_equals_expanded_and_bad_shapes_are_rejected():
    case = tiny("bf16", S=2, H=4, Hkv=2, lens=(4, 1))
    rng = np.random.default_rng(8)
    one = rng.standard_normal((1, 1, 2, 7))
    a = O.gqa_attention(_with_bias(case, (1, 1), T=7, values=one))[1]
    b = O.gqa_attention(_with_bias(case, (2, 4), T=7, values=np.broadcast_to(one, (2, 4, 2, 7))))[1]
    np.testing.assert_array_equal(a, b)
    assert O.validate(_with_bias(case, (3, 1), T=7), "prefill") == O.INVALID
    assert O.validate(_with_bias(case, (1, 2), T=7), "prefill") == O.INVALID
    assert O.validate(_with_bias(case, (1, 1), T=5), "prefill") == O.INVALID   # L + S = 6 > 5


def test_prefill_then_decodes_equals_one_shot_prefill():
    n, k = 7, 4
    full = tiny("fp32", B=1, S=n + k, H=4, Hkv=2, D=8, M=16, lens=(0,), seed=12, rotary=True)
    _, ref, _, _, _ = O.gqa_attention(full)
    part = full.copy()
    part.new_tokens = n
    part.q, part.k_new, part.v_new = full.q[:, :n], full.k_new[:, :n], full.v_new[:, :n]
    _, out, kc, vc, lens = O.gqa_attention(part)
    np.testing.assert_allclose(out, ref[:, :n], rtol=0, atol=1e-13)
    for s in range(k):
        step = full.copy()
        step.new_tokens = 1
        step.q, step.k_new, step.v_new = (x[:, n + s:n + s + 1] for x in (full.q, full.k_new, full.v_new))
        step.k_cache, step.v_cache, step.seqlens_k = kc, vc, lens.astype(np.int32)
        _, out, kc, vc, lens = O.gqa_attention(step, "decode")
        np.testing.assert_allclose(out[:, 0], ref[:, n + s], rtol=0, atol=1e-13)


def test_prefill_then_chunks_equals_one_shot_prefill():
    n, chunks = 5, [3, 4]
    tot = n + sum(chunks)
    full = tiny("fp32", B=2, S=tot, H=4, Hkv=2, D=8, M=16, lens=(0, 0), seed=13, rotary=True)
    _, ref, kc_ref, vc_ref, _ = O.gqa_attention(full)
    part = full.copy()
    part.new_tokens = n
    part.q, part.k_new, part.v_new = full.q[:, :n], full.k_new[:, :n], full.v_new[:, :n]
    _, out, kc, vc, lens = O.gqa_attention(part)
    np.testing.assert_allclose(out, ref[:, :n], rtol=0, atol=1e-13)
    start = n
    for c in chunks:
        step = full.copy()
        step.new_tokens = c
        step.q, step.k_new, step.v_new = (x[:, start:start + c] for x in (full.q, full.k_new, full.v_new))
        step.k_cache, step.v_cache, step.seqlens_k = kc, vc, lens.astype(np.int32)
        _, out, kc, vc, lens = O.gqa_attention(step)
        np.testing.assert_allclose(out, ref[:, start:start + c], rtol=0, atol=1e-13)
        start += c
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref)


# --------------------------------------------------------------------------
# the worked example's shapes (rocMLIR "KV Cache")
# --------------------------------------------------------------------------

def test_worked_example_shapes():
    with open(os.path.join(GOLDEN, "p3_worked_example.json")) as f:
        ex = json.load(f)
    P, D, M = ex["prompt_length"], ex["head_size"], ex["max_seq_len"]
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((P, D)), rng.standard_normal((P, D)), rng.standard_normal((P, D))
    o, p = O.attend_one(q, k, v, O.allowed_mask(P, P, 0, -1), 1 / math.sqrt(D), return_weights=True)
    assert list(p.shape) == ex["prefill"]["softmax"]
    assert list(o.shape) == ex["prefill"]["gemm1"][2]
    # decode: one token at past length 32 inside an M-slot buffer sees 33 keys
    case = gi.make_case("ex", "fp32", 1, 1, 1, 1, D, M, [P], 0)
    st, out, kc, _, lens = O.gqa_attention(case, "decode")
    assert st == O.OK and int(lens[0]) == ex["decode"]["softmax"][1]
    qd = O.to_f64(case.q, "fp32").reshape(1, D)
    kd = O.to_f64(kc[0, 0, :int(lens[0])], "fp32")
    _, pd = O.attend_one(qd, kd, kd, O.allowed_mask(1, kd.shape[0], P, -1), 1.0, return_weights=True)
    assert list(pd.shape) == ex["decode"]["softmax"]
    assert list(out.shape[1:]) == [1, D]

"""The C-ABI boundary without a GPU: the library loads, exports every symbol
the header declares, and validation rejects bad calls before any launch.

Every call here fails validation, so no device memory is ever touched (the
"device" pointers are dummies). The expected status of each case follows the
oracle's validation rules where the oracle has one.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import gqa_inputs as gi
from oracle import gqa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def g():
    import grouped_query_kv_amd as gqa
    return gqa


def declared_functions():
    with open(os.path.join(ROOT, "include", "gqa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(gqa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol(g):
    names = declared_functions()
    assert set(names) == {"gqa_workspace_bytes", "gqa_append_kv", "gqa_attention_prefill",
                          "gqa_attention_decode", "gqa_attention_present", "gqa_evict_window",
                          "gqa_attention_decode_noalloc", "gqa_stream_read", "gqa_status_string",
                          "gqa_last_error"}
    assert set(names) == set(g.EXPORTED)
    lib = ctypes.CDLL(g.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(g):
    for code in range(6):
        assert g.lib.gqa_status_string(code)
    assert b"no room" in g.lib.gqa_status_string(g.GQA_ERR_NO_ROOM)


def _shape(g, B=2, S=3, H=4, Hkv=2, D=8, M=16, dtype=0):
    return g.Shape(B, S, H, Hkv, D, M, dtype)


def _call(g, entry, shape, opts=None, lens=(0, 0), ws_bytes=1 << 30, ws=FAKE, incoming=1):
    opts = opts or g.Options(0.0, -1, None, None, 0, 0)
    hl = np.asarray(lens, np.int32)
    hp = hl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if entry == "append":
        return g.lib.gqa_append_kv(ctypes.byref(shape), ctypes.byref(opts), FAKE, FAKE, FAKE, FAKE,
                                   hp, FAKE, None)
    if entry == "evict":
        after = np.zeros(max(1, len(lens)), np.int32)
        return g.lib.gqa_evict_window(ctypes.byref(shape), incoming, FAKE, FAKE, hp, FAKE,
                                      after.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      ws, ws_bytes, None)
    fn = g.lib.gqa_attention_decode if entry == "decode" else g.lib.gqa_attention_prefill
    return fn(ctypes.byref(shape), ctypes.byref(opts), FAKE, FAKE, FAKE, FAKE, FAKE, hp, FAKE,
              FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("entry", ["append", "prefill"])
def test_no_room_when_past_plus_new_exceeds_buffer(g, entry):
    st = _call(g, entry, _shape(g, S=3, M=16), lens=(13, 14))
    assert st == g.GQA_ERR_NO_ROOM
    assert b"sequence 1" in g.lib.gqa_last_error()


@pytest.mark.parametrize("entry", ["append", "prefill"])
def test_no_room_without_integer_overflow(g, entry):
    # past + new computed in 64 bits: a huge new_tokens is no room, not a wrap
    st = _call(g, entry, _shape(g, S=2**31 - 1, M=16), lens=(5, 0))
    assert st == g.GQA_ERR_NO_ROOM


def test_no_room_in_decode_without_window(g):
    st = _call(g, "decode", _shape(g, S=1, M=16), lens=(16, 0))
    assert st == g.GQA_ERR_NO_ROOM


def test_no_room_matches_oracle_rule():
    # the oracle agrees on which of these fit: L + S == M fits, M + 1 does not
    fits = gi.make_case("x", "fp32", 2, 3, 4, 2, 8, 16, [13, 0], 0)
    assert O.validate(fits, "prefill") == O.OK
    over = gi.make_case("x", "fp32", 2, 3, 4, 2, 8, 16, [14, 0], 0)
    assert O.validate(over, "prefill") == O.NO_ROOM


INVALID = [
    ("prefill", dict(H=3), {}),                         # H % Hkv
    ("prefill", dict(S=0), {}),
    ("decode", dict(S=2), {}),
    ("prefill", dict(D=0), {}),
    ("prefill", dict(D=257), {}),
    ("prefill", dict(M=0), {}),
    ("prefill", dict(dtype=7), {}),
    ("prefill", dict(B=-1), {}),
    ("prefill", {}, dict(window=0)),
    ("prefill", {}, dict(window=17)),
    ("prefill", {}, dict(lens=(-1, 0))),
    ("prefill", {}, dict(lens=(17, 0))),
    ("prefill", {}, dict(scale=float("nan"))),
    ("prefill", dict(D=7), dict(rotary=True)),          # odd D with rotary
    ("prefill", {}, dict(rotary=True, rows=4, lens=(2, 0))),   # positions beyond the table
    ("append", dict(S=-1), {}),
]


@pytest.mark.parametrize("entry,shape_kw,kw", INVALID)
def test_invalid_arguments(g, entry, shape_kw, kw):
    shape = _shape(g, **shape_kw)
    rot = kw.get("rotary", False)
    opts = g.Options(kw.get("scale", 0.0), kw.get("window", -1), FAKE if rot else None,
                     FAKE if rot else None, kw.get("rows", 64), 0)
    st = _call(g, entry, shape, opts, lens=kw.get("lens", (0, 0)))
    assert st == g.GQA_ERR_INVALID_ARG, g.lib.gqa_last_error()
    assert g.lib.gqa_last_error()


def test_windowed_chunk_needs_the_staging_workspace(g):
    # S > 1 with a window: the workspace holds two staging frames of
    # B * Hkv * (M + S) rows, and a workspace sized without the window is
    # rejected before any launch
    shape = _shape(g, S=3, M=16)
    opts = g.Options(0.0, 16, None, None, 0, 0)
    plain = g.lib.gqa_workspace_bytes(ctypes.byref(shape), None)
    staged = g.lib.gqa_workspace_bytes(ctypes.byref(shape), ctypes.byref(opts))
    assert staged >= plain + 2 * 2 * 2 * (16 + 3) * 8 * 4
    st = _call(g, "prefill", shape, opts, lens=(15, 0), ws_bytes=staged - 1)
    assert st == g.GQA_ERR_WORKSPACE
    # one token per sequence needs no staging
    one = _shape(g, S=1, M=16)
    assert (g.lib.gqa_workspace_bytes(ctypes.byref(one), ctypes.byref(opts))
            == g.lib.gqa_workspace_bytes(ctypes.byref(one), None))


def test_greedy_eviction_needs_a_window(g):
    opts = g.Options(0.0, -1, None, None, 0, 0, 1)
    assert _call(g, "prefill", _shape(g, S=3, M=16), opts, lens=(3, 2)) == g.GQA_ERR_INVALID_ARG
    assert "window" in g.lib.gqa_last_error().decode()
    assert _call(g, "decode", _shape(g, S=1, M=16), opts, lens=(3, 2)) == g.GQA_ERR_INVALID_ARG


def test_bias_validation(g):
    sh = _shape(g, S=3, M=16)              # B = 2, H = 4
    def opts(bb, bh, bt):
        o = g.Options(0.0, -1, None, None, 0, 0, 0)
        o.attention_bias, o.bias_batch, o.bias_heads, o.bias_total = FAKE, bb, bh, bt
        return o
    assert _call(g, "prefill", sh, opts(3, 1, 16), lens=(3, 2)) == g.GQA_ERR_INVALID_ARG
    assert _call(g, "prefill", sh, opts(1, 2, 16), lens=(3, 2)) == g.GQA_ERR_INVALID_ARG
    # past + new reaches 6 columns
    assert _call(g, "prefill", sh, opts(2, 4, 5), lens=(3, 2)) == g.GQA_ERR_INVALID_ARG
    assert "bias_total" in g.lib.gqa_last_error().decode()
    assert _call(g, "decode", _shape(g, S=1, M=16), opts(1, 1, 3), lens=(3, 2)) == g.GQA_ERR_INVALID_ARG


def test_workspace_too_small(g):
    need = g.lib.gqa_workspace_bytes(ctypes.byref(_shape(g, S=1, D=128, dtype=1)), None)
    assert need > 0
    st = _call(g, "decode", _shape(g, S=1, D=128, dtype=1), lens=(3, 4), ws_bytes=need - 1)
    assert st == g.GQA_ERR_WORKSPACE
    st = _call(g, "decode", _shape(g, S=1, D=128, dtype=1), lens=(3, 4), ws=None)
    assert st == g.GQA_ERR_WORKSPACE


def test_workspace_bound_is_independent_of_lengths(g):
    a = g.gqa_workspace_bytes(16, 1, 32, 8, 128, 4096, g.GQA_FP16)
    b = g.gqa_workspace_bytes(16, 1, 32, 8, 128, 4096, g.GQA_FP16)
    assert a == b and a % 256 == 0
    assert g.gqa_workspace_bytes(0, 1, 32, 8, 128, 4096, g.GQA_FP16) == 0


def test_evict_validation(g):
    sh = _shape(g, S=0, M=16)
    assert _call(g, "evict", sh, lens=(3, 4), incoming=17) == g.GQA_ERR_INVALID_ARG
    assert _call(g, "evict", sh, lens=(3, 4), incoming=-1) == g.GQA_ERR_INVALID_ARG
    assert _call(g, "evict", sh, lens=(3, 20), incoming=1) == g.GQA_ERR_INVALID_ARG
    assert _call(g, "evict", sh, lens=(16, 4), incoming=2, ws=None) == g.GQA_ERR_WORKSPACE


def test_evict_without_drops_is_a_host_only_noop(g):
    # nothing to drop: returns the new lengths and launches nothing
    hl = np.array([3, 4], np.int32)
    after = np.zeros(2, np.int32)
    st = g.lib.gqa_evict_window(ctypes.byref(_shape(g, S=0, M=16)), 5, FAKE, FAKE,
                                hl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), FAKE,
                                after.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), FAKE, 1 << 30,
                                None)
    assert st == g.GQA_OK and after.tolist() == [3, 4]


def test_empty_batch_is_a_noop(g):
    assert _call(g, "prefill", _shape(g, B=0), lens=()) == g.GQA_OK
    assert _call(g, "append", _shape(g, B=0), lens=()) == g.GQA_OK
    assert _call(g, "append", _shape(g, S=0), lens=(1, 2)) == g.GQA_OK


def _present(g, shape, lens, past_rows, past_k=FAKE + 0x1000, past_v=FAKE + 0x2000,
             present_k=FAKE + 0x3000, present_v=FAKE + 0x4000):
    # every case below must fail validation: the pointers are dummies
    opts = g.Options(0.0, -1, None, None, 0, 0)
    hl = np.asarray(lens, np.int32)
    hp = hl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return g.lib.gqa_attention_present(ctypes.byref(shape), ctypes.byref(opts), FAKE, FAKE, FAKE,
                                       past_k, past_v, past_rows, present_k, present_v,
                                       hp, FAKE, FAKE, FAKE, 1 << 30, None)


def test_present_mode_validation(g):
    sh = _shape(g, S=3, M=16)
    # a length beyond the past's rows
    assert _present(g, sh, (6, 2), 5) == g.GQA_ERR_INVALID_ARG
    assert _present(g, sh, (3, 2), -1) == g.GQA_ERR_INVALID_ARG
    # present too short for past + new: no room, as in shared mode
    assert _present(g, sh, (14, 2), 20) == g.GQA_ERR_NO_ROOM
    # the same buffers with another row count
    assert _present(g, sh, (3, 2), 8, past_k=FAKE, past_v=FAKE + 8, present_k=FAKE,
                    present_v=FAKE + 8) == g.GQA_ERR_INVALID_ARG
    # only K shared, or only V
    assert _present(g, sh, (3, 2), 16, past_k=FAKE, present_k=FAKE) == g.GQA_ERR_INVALID_ARG
    assert _present(g, sh, (3, 2), 16, past_v=FAKE, present_v=FAKE) == g.GQA_ERR_INVALID_ARG
    # a missing past
    assert _present(g, sh, (3, 2), 8, past_k=0) == g.GQA_ERR_INVALID_ARG
    # workspace checked before any launch
    opts = g.Options(0.0, 16, None, None, 0, 0)
    hl = np.asarray((3, 2), np.int32)
    st = g.lib.gqa_attention_present(ctypes.byref(sh), ctypes.byref(opts), FAKE, FAKE, FAKE, FAKE,
                                     FAKE + 64, 8, FAKE + 128, FAKE + 192,
                                     hl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), FAKE, FAKE,
                                     None, 0, None)
    assert st == g.GQA_ERR_WORKSPACE


def test_binding_routes_separate_present_to_present_mode(g):
    torch = pytest.importorskip("torch")
    past_k, past_v = torch.zeros(1, 1, 4, 8), torch.zeros(1, 1, 4, 8)
    pres_k, pres_v = torch.zeros(1, 1, 16, 8), torch.zeros(1, 1, 16, 8)
    q, kn = torch.zeros(1, 2, 16), torch.zeros(1, 2, 8)
    # length 5 exceeds the 4 past rows: only the present entry point checks
    # that (validation, before any launch)
    lens_dev = torch.zeros(1, dtype=torch.int32)   # never read: validation fails first
    with pytest.raises(g.GQAError) as e:
        g.gqa_attention_prefill(q, kn, kn, past_k, past_v, np.array([5], np.int32), lens_dev,
                                present_key=pres_k, present_value=pres_v, stream=0)
    assert e.value.status == g.GQA_ERR_INVALID_ARG and "past_rows" in str(e.value)
    with pytest.raises(g.GQAError):
        g.gqa_attention_prefill(q, kn, kn, past_k, past_v, np.array([1], np.int32), None,
                                present_key=pres_k, stream=0)


def test_binding_rejects_separate_past_and_present(g):
    torch = pytest.importorskip("torch")
    kc = torch.zeros(1, 1, 8, 4)
    vc = torch.zeros(1, 1, 8, 4)
    other = torch.zeros(1, 1, 8, 4)
    kn = torch.zeros(1, 1, 4)
    with pytest.raises(g.GQAError) as e:
        g.gqa_append_kv(kn, kn, kc, vc, np.zeros(1, np.int32), None, present_key=other, stream=0)
    assert e.value.status == g.GQA_ERR_INVALID_ARG


def test_binding_surfaces_no_room(g):
    torch = pytest.importorskip("torch")
    kc = torch.zeros(1, 1, 8, 4)
    kn = torch.zeros(1, 2, 4)
    with pytest.raises(g.GQAError) as e:
        g.gqa_append_kv(kn, kn, kc, kc.clone(), np.array([7], np.int32),
                        torch.zeros(1, dtype=torch.int32), stream=0)
    assert e.value.status == g.GQA_ERR_NO_ROOM


def test_binding_checks_lengths_and_rotary_tables(g):
    # the kernels read these with a fixed layout: the binding refuses others
    torch = pytest.importorskip("torch")
    kc, vc = torch.zeros(2, 1, 8, 4), torch.zeros(2, 1, 8, 4)
    q, kn = torch.zeros(2, 1, 8), torch.zeros(2, 1, 4)
    lens = np.zeros(2, np.int32)
    good = torch.zeros(2, dtype=torch.int32)
    cos = torch.ones(9, 2)
    bad_calls = [
        dict(seqlens_k_dev=torch.zeros(2, dtype=torch.int64)),
        dict(seqlens_k_dev=torch.zeros(3, dtype=torch.int32)),
        dict(cos_cache=cos.half(), sin_cache=cos.half()),
        dict(cos_cache=torch.ones(9, 4), sin_cache=torch.ones(9, 4)),
        dict(cos_cache=cos, sin_cache=torch.ones(8, 2)),
        dict(cos_cache=cos),
    ]
    for kw in bad_calls:
        dev = kw.pop("seqlens_k_dev", good)
        with pytest.raises(g.GQAError) as e:
            g.gqa_attention_decode(q, kn, kn, kc, vc, lens, dev, stream=0, **kw)
        assert e.value.status == g.GQA_ERR_INVALID_ARG, kw
        with pytest.raises(g.GQAError):
            g.gqa_append_kv(kn, kn, kc, vc, lens, dev, stream=0, **kw)


# --------------------------------------------------------------------------
# alignment: the vector kernels move 16-byte units of every tensor
# --------------------------------------------------------------------------

@pytest.mark.parametrize("entry", ["append", "prefill", "decode"])
@pytest.mark.parametrize("which", range(6))
def test_misaligned_tensors_are_rejected(g, entry, which):
    # pointer order of the attention calls: q, k_new, v_new, k_cache, v_cache, out
    ptrs = [FAKE] * 6
    ptrs[which] = FAKE + 8
    shape = _shape(g, S=1 if entry == "decode" else 3)
    opts = g.Options(0.0, -1, None, None, 0, 0)
    hl = np.zeros(2, np.int32)
    hp = hl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if entry == "append":
        if which in (0, 5):          # no q / out in the append half
            return
        st = g.lib.gqa_append_kv(ctypes.byref(shape), ctypes.byref(opts), *ptrs[1:5], hp, FAKE, None)
    else:
        fn = g.lib.gqa_attention_decode if entry == "decode" else g.lib.gqa_attention_prefill
        st = fn(ctypes.byref(shape), ctypes.byref(opts), *ptrs[:5], hp, FAKE, ptrs[5], FAKE, 1 << 30,
                None)
    assert st == g.GQA_ERR_INVALID_ARG
    assert b"aligned" in g.lib.gqa_last_error()


def test_misaligned_past_and_evict_buffers_are_rejected(g):
    shape = _shape(g, S=3, M=16)
    st = _present(g, shape, (5, 2), 8, past_k=FAKE + 0x1004)
    assert st == g.GQA_ERR_INVALID_ARG and b"aligned" in g.lib.gqa_last_error()
    after = np.zeros(2, np.int32)
    hl = np.asarray((16, 3), np.int32)
    st = g.lib.gqa_evict_window(ctypes.byref(_shape(g, S=0, M=16)), 1, FAKE + 2, FAKE,
                                hl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), FAKE,
                                after.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), FAKE, 1 << 30,
                                None)
    assert st == g.GQA_ERR_INVALID_ARG and b"aligned" in g.lib.gqa_last_error()


# --------------------------------------------------------------------------
# the entry point without a workspace: validated before any device call
# --------------------------------------------------------------------------

def _noalloc(g, shape, lens, opts=None):
    opts = opts or g.Options(0.0, -1, None, None, 0, 0)
    hl = np.asarray(lens, np.int32)
    return g.lib.gqa_attention_decode_noalloc(ctypes.byref(shape), ctypes.byref(opts), FAKE, FAKE,
                                              FAKE, FAKE, FAKE,
                                              hl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                              FAKE, FAKE, None)


def test_noalloc_validates_like_decode(g):
    assert _noalloc(g, _shape(g, S=2), (0, 0)) == g.GQA_ERR_INVALID_ARG       # one token only
    assert _noalloc(g, _shape(g, S=1, M=16), (16, 0)) == g.GQA_ERR_NO_ROOM
    assert _noalloc(g, _shape(g, S=1, D=257), (0, 0)) == g.GQA_ERR_INVALID_ARG
    assert _noalloc(g, _shape(g, B=0, S=1), ()) == g.GQA_OK                   # nothing to do


def test_noalloc_rejects_calls_beyond_its_scratch(g):
    # a shape whose workspace exceeds the static scratch is refused with a
    # message naming both sizes, before any device call
    big = g.Shape(64, 1, 256, 32, 128, 8192, g.GQA_FP16)
    need = g.lib.gqa_workspace_bytes(ctypes.byref(big), None)
    assert need > g.NOALLOC_SCRATCH_BYTES
    st = _noalloc(g, big, [0] * 64)
    assert st == g.GQA_ERR_WORKSPACE
    assert b"static scratch" in g.lib.gqa_last_error()


@pytest.mark.parametrize("B,H,Hkv,M,dt,W", [(16, 32, 8, 4096, 1, -1), (8, 32, 8, 4096, 2, 4096),
                                           (64, 32, 8, 4096, 1, -1)])
def test_decode_workloads_fit_the_static_scratch(g, B, H, Hkv, M, dt, W):
    # the split-KV and window decode workloads (and 64 sequences of 4096 rows)
    # need less workspace than the static scratch holds, counters apart
    shape = g.Shape(B, 1, H, Hkv, 128, M, dt)
    opts = g.Options(0.0, W, None, None, 0, 0)
    need = g.lib.gqa_workspace_bytes(ctypes.byref(shape), ctypes.byref(opts))
    assert need + (64 << 10) <= g.NOALLOC_SCRATCH_BYTES


# --------------------------------------------------------------------------
# position offsets: validated against the rotary table before any launch
# --------------------------------------------------------------------------

def _with_offsets(g, host, dev=FAKE, rows=16, rot=True):
    o = g.Options(0.0, -1, FAKE if rot else None, FAKE if rot else None, rows, 0)
    keep = None
    if host is not None:
        keep = np.asarray(host, np.int32)
        o.position_offset_host = keep.ctypes.data
    o.position_offset_dev = dev
    return o, keep


@pytest.mark.parametrize("host,dev,lens,msg", [
    ([0, 0], None, (0, 0), b"position_offset"),     # host copy without the device copy
    (None, FAKE, (0, 0), b"position_offset"),       # device copy without the host copy
    ([-1, 0], FAKE, (0, 0), b"position_offset"),    # negative
    ([0, 11], FAKE, (2, 3), b"rotary table"),       # 11 + 3 + 3 = 17 > 16 table rows
])
def test_position_offset_validation(g, host, dev, lens, msg):
    # (10 + 3 + 3 = 16 rows would fit; the oracle test below checks that
    # boundary, since a valid call here would launch on dummy pointers)
    o, keep = _with_offsets(g, host, dev)
    st = _call(g, "prefill", _shape(g, S=3), o, lens=lens, ws=FAKE)
    assert st == g.GQA_ERR_INVALID_ARG, g.lib.gqa_last_error()
    assert msg in g.lib.gqa_last_error()


def test_position_offset_rule_matches_oracle():
    c = gi.make_case("x", "fp16", 2, 3, 4, 2, 8, 16, [2, 3], 0, rotary=True, rotary_rows=16)
    c.position_offset = np.array([0, 10], np.int32)
    assert O.validate(c, "prefill") == O.OK
    c.position_offset = np.array([0, 11], np.int32)
    assert O.validate(c, "prefill") == O.INVALID


def test_stream_read_rejects_bad_arguments(g):
    """The read yardstick validates before any launch (no GPU needed)."""
    for ptr, nbytes in ((None, 1024), (16, 0), (16, 1000), (8, 1024)):
        st = g.lib.gqa_stream_read(ptr, nbytes, None)
        assert st == g.GQA_ERR_INVALID_ARG, (ptr, nbytes, st)
        assert b"gqa_stream_read" in g.lib.gqa_last_error()

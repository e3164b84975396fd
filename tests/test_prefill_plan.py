"""Host model of the MFMA prefill's key-split plan (CPU only).

When the 256-row blocks of a call fill less than three quarters of the chip,
the host cuts each row block's key tiles into up to 4 ranges, sized to the
lengths, and lists one workgroup per range in the kernel arguments; each
range writes a partial into a workspace slot and the last one to finish,
counted in a per-row-block counter, merges them. This model follows the same
integer arithmetic: the planner of launch_prefill_fast (tiles per row block,
the smallest range size T whose range count fits the budget, the order and
the packed entries) and the kernel's use of an entry (row block, key range
[t_begin, t_end), slot item * 4 + split, counter item). For many shapes it
checks that every slot and counter index lies inside the workspace regions
that workspace_layout reserves, that each row block's ranges cover its tiles
exactly once, and that every key a query row may see lies in its row block's
tiles. The model's workspace sizes are checked against the library's own
gqa_workspace_bytes, which ties the model to the code it mirrors. A mistake
here is an out-of-range store on the GPU, so it is checked on the host first.
"""
import ctypes
import functools

import numpy as np
import pytest

WG_ROWS, BK, MAX_SPLITS, PLAN_MAX, TARGET_WG = 256, 64, 4, 512, 256
SLOT_FLOATS = 512 * 32 + 2 * 512
DECODE_WG, DECODE_WAVES, DECODE_HG, DECODE_ARG_BATCH = 256, 8, 16, 64
EVICT_HALO_MAX, EVICT_CHUNK_ROWS = 4, 128


def cdiv(a, b):
    return -(-a // b)


def align256(x):
    return (x + 255) & ~255


def kept_rows(L, S, M, cap):
    if L + S <= M:
        return L
    return min(L, max(0, cap - S))


def may_split(B, S, G, Hkv, M):
    items = cdiv(S * G, WG_ROWS) * B * Hkv
    if items <= 0 or 4 * items >= 3 * TARGET_WG:
        return False
    return cdiv(M, 64) // 8 >= 2


def layout(B, S, H, Hkv, D, M, dt_bytes, window):
    """workspace_layout: (total, prefill partial region (offset, bytes),
    prefill counter region (offset, bytes))."""
    staged = window > 0 and S > 1
    M = M + (S if staged else 0)
    G = H // Hkv
    hg = cdiv(G, DECODE_HG)
    counters_bytes = align256(B * Hkv * hg * 4)
    fast = D in (128, 64) and dt_bytes == 2
    # decode partial slots are laid out for head size 128 (D = 64 uses half)
    partial = (DECODE_WG + B * Hkv * hg) * DECODE_HG * (128 + 2) * 4 if fast else 0
    row_bytes = D * dt_bytes
    halo = B * Hkv * 2 * cdiv(M, EVICT_CHUNK_ROWS) * EVICT_HALO_MAX * row_bytes
    dhalo = 2 * DECODE_WG * DECODE_WAVES * D * 2 if fast else 0
    pf_items = pf_partial = 0
    decode_only = S == 1
    if fast and S > 0 and not decode_only and may_split(B, S, G, Hkv, M):
        pf_items = cdiv(S * G, WG_ROWS) * B * Hkv
        pf_partial = pf_items * MAX_SPLITS * SLOT_FLOATS * 4
    scratch = counters_bytes
    scratch_bytes = align256(max(halo, align256(partial) + dhalo, pf_partial))
    pf_counters = scratch + scratch_bytes
    total = pf_counters + align256(pf_items * 4)
    if staged:
        total += 2 * align256(B * Hkv * M * row_bytes)
    return total, (scratch, scratch_bytes), (pf_counters, align256(pf_items * 4)), M


def row_block_keys(L, S, G, W, rb):
    r0 = rb * WG_ROWS
    ilo, ihi = r0 // G, min(S - 1, (r0 + WG_ROWS - 1) // G)
    kstart = max(0, L + ilo - W + 1) if W > 0 else 0
    return kstart, L + ihi + 1


def plan(B, S, G, Hkv, M, W, lens, cap, cus):
    """launch_prefill_fast's plan: None without a split, else packed entries."""
    n_rb = cdiv(S * G, WG_ROWS)
    units = B * Hkv
    n_items0 = n_rb * units
    if not may_split(B, S, G, Hkv, M):
        return None, n_items0
    budget = min(PLAN_MAX, max(cus, n_items0))
    tiles = []
    for k in range(n_items0):
        rb, b = n_rb - 1 - k // units, (k % units) // Hkv
        L = max(0, min(kept_rows(lens[b], S, M, cap), M - S))
        ks, ke = row_block_keys(L, S, G, W, rb)
        tiles.append(max(1, cdiv(ke, BK) - ks // BK))

    def ranges(k, T):
        return min(MAX_SPLITS, cdiv(tiles[k], T))

    lo, hi = 1, max(tiles)
    while lo < hi:
        mid = (lo + hi) // 2
        if sum(ranges(k, mid) for k in range(n_items0)) <= budget:
            hi = mid
        else:
            lo = mid + 1

    def before(x, y):
        return tiles[x] * ranges(y, lo) > tiles[y] * ranges(x, lo)

    order = sorted(range(n_items0),
                   key=functools.cmp_to_key(lambda x, y: -1 if before(x, y) else (1 if before(y, x) else 0)))
    entries = []
    for k in order:
        n = ranges(k, lo)
        entries += [k | (j << 16) | (n << 24) for j in range(n)]
    return entries, n_items0


def check_call(B, S, H, Hkv, M, W, lens, cap, cus=256, dt_bytes=2):
    G = H // Hkv
    total, (p_off, p_bytes), (c_off, c_bytes), Mk = layout(B, S, H, Hkv, 128, M, dt_bytes, W)
    # the kernel runs on the buffer as the call sees it (the staging frame of
    # M + S rows on the windowed-chunk path)
    staged = W > 0 and S > 1 and any(kept_rows(L, S, M, cap) < L for L in lens)
    Mrun = M + S if staged else M
    cap_run = Mrun if staged else cap
    entries, n_items0 = plan(B, S, G, Hkv, Mrun, W, lens, cap_run, cus)
    n_rb, units = cdiv(S * G, WG_ROWS), B * Hkv
    if entries is None:
        return 0
    assert len(entries) <= PLAN_MAX and len(entries) >= n_items0
    seen = {}
    for e in entries:
        item, split, nsplit = e & 0xFFFF, (e >> 16) & 0xFF, e >> 24
        assert 0 <= item < n_items0 and 1 <= nsplit <= MAX_SPLITS and 0 <= split < nsplit
        # the slot this range writes and the counter it bumps
        slot_end = ((item * MAX_SPLITS + split) + 1) * SLOT_FLOATS * 4
        assert p_off + slot_end <= p_off + p_bytes <= total
        assert c_off + (item + 1) * 4 <= c_off + c_bytes <= total
        # the kernel's key range for this entry
        b = (item % units) // Hkv
        rb = n_rb - 1 - item // units
        L = min(max(kept_rows(min(max(lens[b], 0), Mrun), S, Mrun, cap_run), 0), Mrun - S)
        ks, ke = row_block_keys(L, S, G, W, rb)
        t0, t1 = ks // BK, cdiv(ke, BK)
        tb = t0 + (t1 - t0) * split // nsplit
        te = t0 + (t1 - t0) * (split + 1) // nsplit
        assert tb < te, "empty key range"
        assert te * BK <= cdiv(L + S, BK) * BK                  # no tile past the valid length's tile
        seen.setdefault(item, []).append((split, nsplit, tb, te, t0, t1, L, rb))
    assert sorted(seen) == list(range(n_items0)), "a row block without a workgroup"
    for item, rs in seen.items():
        rs.sort()
        nsplit = rs[0][1]
        assert [r[0] for r in rs] == list(range(nsplit)) and all(r[1] == nsplit for r in rs)
        t0, t1, L, rb = rs[0][4], rs[0][5], rs[0][6], rs[0][7]
        # the ranges tile [t0, t1) exactly once, in order
        assert rs[0][2] == t0 and rs[-1][3] == t1
        assert all(rs[j][3] == rs[j + 1][2] for j in range(len(rs) - 1))
        # every key any row of the block may see lies in those tiles
        for r in range(rb * WG_ROWS, min((rb + 1) * WG_ROWS, S * G)):
            i = r // G
            lo = max(0, L + i - W + 1) if W > 0 else 0
            assert t0 * BK <= lo and L + i < t1 * BK
    return len(entries)


def lib_workspace(B, S, H, Hkv, M, W, dt, D=128):
    import grouped_query_kv_amd as gqa
    shape = gqa.Shape(B, S, H, Hkv, D, M, dt)
    opts = gqa.Options(0.0, W, None, None, 0, 0)
    return int(gqa.lib.gqa_workspace_bytes(ctypes.byref(shape), ctypes.byref(opts)))


def random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 7, 8, 16]))
        B = int(rng.integers(1, 12))
        M = int(rng.choice([512, 1024, 2048, 4096, 5000]))
        S = int(rng.choice([2, 7, 33, 64, 128, 200, 256, 500]))
        S = min(S, M)
        W = -1
        greedy = False
        if rng.random() < 0.4:
            W = int(rng.integers(max(1, S), M + 1))
            greedy = bool(rng.random() < 0.3 and W < M)
        if W > 0:
            lens = [int(rng.integers(0, M + 1)) for _ in range(B)]
        else:
            lens = [int(rng.integers(0, M - S + 1)) for _ in range(B)]
        yield B, S, G * Hkv, Hkv, M, W, lens, (W if greedy else M)


# the named workloads and the GPU tests' split cases
NAMED = [
    (8, 128, 28, 4, 4096, -1, "ragged"),                       # ragged continuation (lens below)
    (3, 40, 8, 2, 2048, -1, [0, 700, 1999]),
    (2, 33, 16, 2, 2048, 100, [1500, 0]),
    (2, 7, 8, 8, 1024, -1, [1017, 300]),
    (2, 40, 8, 2, 2048, 1024, [2040, 1000]),                   # windowed chunk, staging frame
    (4, 2048, 32, 8, 4096, -1, [0, 0, 0, 0]),                  # causal prefill: 1024 blocks, no split
    (8, 128, 32, 8, 4096, 4096, [4096] * 8),                   # windowed chunks into full caches
]


@pytest.mark.parametrize("spec", NAMED, ids=[str(i) for i in range(len(NAMED))])
@pytest.mark.parametrize("cus", [256, 80, 304])
def test_plan_bounds_on_named_shapes(spec, cus):
    B, S, H, Hkv, M, W, lens = spec
    if lens == "ragged":
        import gqa_inputs as gi
        lens = gi.workload("ragged-continuation-fp16").seqlens_k.tolist()
    check_call(B, S, H, Hkv, M, W, lens, M, cus)


def test_plan_bounds_on_random_shapes():
    n_split = 0
    for B, S, H, Hkv, M, W, lens, cap in random_shapes(400, 7):
        for cus in (256, 120):
            n_split += check_call(B, S, H, Hkv, M, W, lens, cap, cus) > 0
    assert n_split > 100            # the plan was exercised, not only the unsplit launch


def test_model_workspace_equals_the_library():
    """The model's layout is the library's: equal gqa_workspace_bytes for the
    named shapes, random shapes, head sizes 128, 64 and 8 and all three
    dtypes, with and without a window."""
    shapes = [(s[0], s[1], s[2], s[3], s[4], s[5]) for s in NAMED]
    shapes += [(B, S, H, Hkv, M, W) for B, S, H, Hkv, M, W, _, _ in random_shapes(150, 9)]
    shapes += [(16, 1, 32, 8, 4096, -1), (8, 1, 32, 8, 4096, 4096), (66, 1, 8, 2, 96, 64)]
    for B, S, H, Hkv, M, W in shapes:
        for D in (128, 64, 8):
            for dt in (0, 1, 2):
                want = layout(B, S, H, Hkv, D, M, 4 if dt == 0 else 2, W)[0]
                assert lib_workspace(B, S, H, Hkv, M, W, dt, D) == want, (B, S, H, Hkv, M, W, dt, D)


def test_ragged_continuation_is_split():
    """The ragged continuation's 128 row blocks fill half the chip: the plan
    splits them (the model would pass vacuously otherwise)."""
    import gqa_inputs as gi
    c = gi.workload("ragged-continuation-fp16")
    entries, n0 = plan(8, 128, 7, 4, 4096, -1, c.seqlens_k.tolist(), 4096, 256)
    assert n0 == 128 and entries is not None and 128 < len(entries) <= 256

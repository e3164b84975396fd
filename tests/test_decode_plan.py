"""Host model of the decode kernel's work plan (CPU only).

The split-KV decode kernel deals equal slices of all 16-key blocks to the
waves of the launch, keeps the partial of a unit cut by a slice boundary in
the workgroup's LDS, combines them per workgroup and merges across
workgroups. This model follows the same integer arithmetic (block list per
sequence and unit, slice bounds, locate / next-block walk, partial slots
`worker + unit` in LDS and `workgroup + unit` in the workspace) and checks,
for many shapes, that every block a wave loads exists, that no slot is
written twice, that the workspace bound holds and that each merge reads
exactly the partials that were written. A mistake here is an out-of-range
load on the GPU, so it is checked on the host first.
"""
import numpy as np
import pytest

KEYS, MAXHG, MERGEMAX, WAVES, MAXWG = 16, 16, 64, 8, 256
MAXWORKERS = MAXWG * WAVES


def seq_of(a, b):
    L = min(max(a["lens"][b], 0), a["M"])
    kend = min(L, a["M"] - 1) + 1
    kstart = max(kend - a["W"], 0) if a["W"] > 0 else 0
    return kstart, kend, -(-(kend - kstart) // KEYS)


def plan_launch(lens, B, H, Hkv, M, W):
    G = H // Hkv
    n_hg = -(-G // MAXHG)
    units = Hkv * n_hg
    a = dict(lens=lens, B=B, units=units, M=M, W=W)
    pb, total = [], 0
    for b in range(B):
        pb.append(total)
        total += seq_of(a, b)[2] * units
    pb.append(total)
    workers = min(MAXWORKERS, total)
    max_unit = max((pb[b + 1] - pb[b]) // units for b in range(B))
    while workers > 1 and max_unit * workers > (MERGEMAX - 1) * total:
        workers //= 2
    a.update(pb=pb, total=total, workers=workers)
    return a


def locate(a, x):
    b = 0
    for bb in range(a["B"]):
        if a["pb"][bb] <= x < a["pb"][bb + 1]:
            b = bb
    nb = seq_of(a, b)[2]
    off = x - a["pb"][b]
    ub = min(max(off // nb if nb else 0, 0), a["units"] - 1)
    i = min(max(off - ub * nb, 0), max(nb - 1, 0))
    return dict(b=b, ub=ub, i=i, nb=nb)


def next_block(a, c):
    k = dict(c)
    k["i"] += 1
    if k["i"] < k["nb"]:
        return k
    k["i"] = 0
    k["ub"] += 1
    if k["ub"] == a["units"]:
        k["ub"] = 0
        k["b"] += 1
    k["nb"] = seq_of(a, k["b"])[2] if k["b"] < a["B"] else -1
    return k


def valid(a, k):
    return 0 <= k["b"] < a["B"] and 0 <= k["ub"] < a["units"] and 0 <= k["i"] < seq_of(a, k["b"])[2]


def owner(a, x):
    return ((x + 1) * a["workers"] - 1) // a["total"]


def worker_range(a, b, ub):
    nb = seq_of(a, b)[2]
    x0 = a["pb"][b] + ub * nb
    return owner(a, x0), owner(a, x0 + nb - 1)


def check_owner(a):
    # owner(x) is the inverse of the slice bounds for every block
    if a["total"] == 0:
        return
    starts = np.array([w * a["total"] // a["workers"] for w in range(a["workers"] + 1)])
    assert starts[-1] == a["total"] and (np.diff(starts) > 0).all()
    xs = np.arange(a["total"])
    want = np.searchsorted(starts, xs, side="right") - 1
    assert (np.array([owner(a, int(x)) for x in xs]) == want).all()


def run_plan(a):
    check_owner(a)
    nunits = a["B"] * a["units"]
    gslots, gwrote = {}, {}
    for wg in range(-(-a["workers"] // WAVES)):
        tab = [[None, None] for _ in range(WAVES)]
        for wv in range(WAVES):
            w = wg * WAVES + wv
            if w >= a["workers"]:
                continue
            S, E = w * a["total"] // a["workers"], (w + 1) * a["total"] // a["workers"]
            if S >= E:
                continue
            cur = locate(a, S)
            assert valid(a, cur)
            # three blocks in flight: x, x + 1, x + 2 (clamped to the slice)
            nxt = next_block(a, cur) if S + 1 < E else cur
            ahead = next_block(a, nxt) if S + 2 < E else nxt
            assert valid(a, nxt) and valid(a, ahead)
            seg_shared, x = cur["i"] > 0, S
            while True:
                last = x + 1 >= E
                unit_end = cur["i"] + 1 >= cur["nb"]
                if unit_end or last:
                    shared = seg_shared or not unit_end
                    if shared:
                        slot = 1 if last else 0
                        assert tab[wv][slot] is None
                        tab[wv][slot] = (cur["b"], cur["ub"])
                    else:
                        assert worker_range(a, cur["b"], cur["ub"]) == (w, w)
                    if last:
                        break
                    seg_shared = False
                cur, nxt = nxt, ahead
                if x + 3 < E:
                    ahead = next_block(a, ahead)
                assert valid(a, ahead)
                x += 1
        entries = [tab[f >> 1][f & 1] for f in range(2 * WAVES)]
        seen, nglob, prev = set(), 0, None
        for e, ent in enumerate(entries):
            if ent is None or ent == prev:
                continue
            prev = ent
            u = ent[0] * a["units"] + ent[1]
            assert u not in seen
            seen.add(u)
            wf, wl = worker_range(a, *ent)
            mine = {wg * WAVES + (f >> 1) for f in range(2 * WAVES) if entries[f] == ent}
            assert mine == set(range(max(wf, wg * WAVES), min(wl, wg * WAVES + WAVES - 1) + 1))
            if not (wf >= wg * WAVES and wl < (wg + 1) * WAVES):
                slot = wg + u
                assert slot not in gslots and slot < MAXWG + nunits
                gslots[slot] = u
                gwrote.setdefault(u, set()).add(wg)
                nglob += 1
        assert nglob <= 2
    for u, wgs in gwrote.items():
        wf, wl = worker_range(a, *divmod(u, a["units"]))
        assert wgs == set(range(wf // WAVES, wl // WAVES + 1)) and len(wgs) <= MERGEMAX


FIXED = [
    ([0, 63, 257], 3, 8, 2, 300, -1), ([64, 511], 2, 32, 8, 600, -1),
    ([127, 128, 129, 1099], 4, 28, 4, 1100, -1), ([5, 199], 2, 8, 8, 200, -1),
    ([299, 17], 2, 16, 2, 300, 64), ([256, 256], 2, 16, 1, 256, 256),
    ([10, 99], 2, 4, 2, 100, -1), ([4095], 1, 32, 8, 4096, -1), ([0], 1, 4, 2, 64, -1),
    ([4096] * 8, 8, 32, 8, 4096, 4096),
]


@pytest.mark.parametrize("case", FIXED)
def test_plan_fixed(case):
    run_plan(plan_launch(*case))


def test_plan_decode_workload():
    import gqa_inputs as gi
    c = gi.workload("split-kv-decode-fp16")
    run_plan(plan_launch([int(x) for x in c.seqlens_k], 16, 32, 8, 4096, -1))


def test_plan_random():
    rng = np.random.default_rng(7)
    for _ in range(150):
        B = int(rng.integers(1, 65)); Hkv = int(rng.integers(1, 9)); G = int(rng.integers(1, 40))
        M = int(rng.integers(1, 5000)); W = int(rng.choice([-1, int(rng.integers(1, M + 1))]))
        lens = [int(x) for x in rng.integers(0, M, B)]
        run_plan(plan_launch(lens, B, G * Hkv, Hkv, M, W))

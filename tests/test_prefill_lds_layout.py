"""Host model of the prefill kernel's LDS tile layout (CPU only).

The MFMA prefill fills its 64-key K and V tiles straight from memory with
16-byte direct-to-LDS loads: lane i of a load instruction writes LDS slot i
of a 1 KB run, and its own memory offset picks which 16-byte chunk of which
key row lands there (chunk c of key row r goes to slot c ^ swizzle(r)). The
operand reads of the matrix products then find chunk c of key r at
r * row_bytes + 16 * (c ^ swizzle(r)). This model follows the kernel's
index arithmetic for head sizes 128 (256-byte rows, 16 chunks) and 64
(128-byte rows, 8 chunks) and checks that

- the loads of the eight waves fill every (key, chunk) of a tile exactly
  once and stay inside the tile;
- every operand read of the S = K Q^T and O^T = V^T P^T products addresses
  the chunk it means, inside the tile;
- the reads are free of LDS bank conflicts: 64 banks of 4 bytes, a 16-byte
  read serving 16 lanes per cycle and an 8-byte read 32 lanes per cycle,
  so the lanes of one cycle must cover disjoint bank sets.

A mistake in these formulas is a wrong result or an out-of-tile access on
the GPU, so they are checked on the host first.
"""
import pytest

KEYS, WAVES = 64, 8


def swz_k(D, key):
    return key & 15 if D == 128 else (key >> 1) & 7


def swz_v(D, key):
    return (key & 3) << 2 if D == 128 else ((key >> 1) & 1) << 2


def dma_writes(D, is_v):
    """(LDS byte offset, memory byte offset) of every lane of every wave's
    tile loads: the LDS address is the instruction's base plus 16 * lane,
    the memory offset the lane's own (plus the same immediate for V)."""
    row_bytes = 2 * D
    out = []
    for w in range(WAVES):
        for lane in range(64):
            if D == 128:
                lr, slot = lane >> 4, lane & 15
                for q in range(2):
                    if is_v:
                        # one offset pattern; the immediate 1024 q moves both
                        mem = (8 * w + lr) * 256 + 16 * (slot ^ swz_v(D, lr)) + 1024 * q
                        lds = 8 * w * 256 + 1024 * q + 16 * lane
                    else:
                        rrow = 8 * w + 4 * q + lr
                        mem = rrow * 256 + 16 * (slot ^ swz_k(D, rrow))
                        lds = (8 * w + 4 * q) * 256 + 16 * lane
                    out.append((lds, mem))
            else:
                rrow, slot = 8 * w + (lane >> 3), lane & 7
                sw = swz_v(D, rrow) if is_v else swz_k(D, rrow)
                mem = rrow * row_bytes + 16 * (slot ^ sw)
                lds = 8 * w * row_bytes + 16 * lane
                out.append((lds, mem))
    return out


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("is_v", [False, True], ids=["K", "V"])
def test_tile_loads_fill_every_chunk_once(D, is_v):
    row_bytes, tile = 2 * D, KEYS * 2 * D
    writes = dma_writes(D, is_v)
    assert len(writes) == tile // 16
    lds_slots = sorted(l for l, _ in writes)
    assert lds_slots == list(range(0, tile, 16))            # every slot once, inside the tile
    mems = sorted(m for _, m in writes)
    assert mems == list(range(0, tile, 16))                 # every memory chunk once
    # the slot of (key, chunk) is where the operand reads look for it
    sw = swz_v if is_v else swz_k
    for lds, mem in writes:
        key, chunk = divmod(mem, row_bytes)
        chunk //= 16
        assert lds == key * row_bytes + 16 * (chunk ^ sw(D, key))


def k_reads(D, kk, h):
    """Byte offsets of the 16-byte K operand reads of product kk, key half h:
    lane (col, c) reads chunk 2 kk + c of key 32 h + col."""
    row_bytes = 2 * D
    res = []
    for lane in range(64):
        col, c = lane & 31, lane >> 5
        key = 32 * h + col
        res.append((key, 2 * kk + c, key * row_bytes + 16 * ((2 * kk + c) ^ swz_k(D, col))))
    return res


def v_reads(D, u, dt, r):
    """Byte offsets of the transposing 8-byte V operand reads (key group u,
    output tile dt, half r): in each 16-lane group lane j points at key
    16 u + 8 r + 4 c + j / 4, dims 4 (j % 4) .. + 3 of the group's 16 dims."""
    row_bytes = 2 * D
    res = []
    for lane in range(64):
        j, c, g1 = lane & 15, lane >> 5, (lane >> 4) & 1
        key = 16 * u + 8 * r + 4 * c + (j >> 2)
        ch = 4 * dt + 2 * g1 + ((j & 3) >> 1)
        res.append((key, ch, 8 * (j & 1), key * row_bytes + 16 * (ch ^ swz_v(D, key)) + 8 * (j & 1)))
    return res


@pytest.mark.parametrize("D", [128, 64])
def test_k_operand_reads_hit_their_chunk_without_conflicts(D):
    row_bytes, tile = 2 * D, KEYS * 2 * D
    seen = set()
    for kk in range(D // 16):
        for h in range(2):
            reads = k_reads(D, kk, h)
            for key, chunk, addr in reads:
                assert 0 <= addr and addr + 16 <= tile
                assert addr == key * row_bytes + 16 * (chunk ^ swz_k(D, key))
                seen.add((key, chunk))
            for cyc in range(4):                             # 16 lanes per cycle
                banks = [set(range((a // 4) % 64, (a // 4) % 64 + 4)) for _, _, a in reads[16 * cyc:16 * cyc + 16]]
                assert sum(len(b) for b in banks) == len(set().union(*banks)) == 64
    assert seen == {(k, c) for k in range(KEYS) for c in range(D // 8)}


@pytest.mark.parametrize("D", [128, 64])
def test_v_operand_reads_hit_their_chunk_without_conflicts(D):
    row_bytes, tile = 2 * D, KEYS * 2 * D
    seen = set()
    for u in range(4):
        for dt in range(D // 32):
            for r in range(2):
                reads = v_reads(D, u, dt, r)
                for key, ch, half, addr in reads:
                    assert 0 <= addr and addr + 8 <= tile
                    assert addr == key * row_bytes + 16 * (ch ^ swz_v(D, key)) + half
                    seen.add((key, ch, half))
                for cyc in range(2):                         # 32 lanes per cycle
                    banks = [set(range((a // 4) % 64, (a // 4) % 64 + 2)) for *_, a in reads[32 * cyc:32 * cyc + 32]]
                    assert sum(len(b) for b in banks) == len(set().union(*banks)) == 64
    assert seen == {(k, c, h) for k in range(KEYS) for c in range(D // 8) for h in (0, 8)}


@pytest.mark.parametrize("D", [128, 64])
def test_output_staging_rows_round_trip(D):
    """Each wave stages its 32 output rows in 64 D bytes of LDS, chunk c of
    row r at r * 2 D + 16 * (c ^ swizzle_k(r)) (8-byte halves from the
    products' layout), then stores whole rows: every staged byte is read
    back exactly once, from where it was written."""
    row_bytes, chunks = 2 * D, D // 8
    written = {}
    for lane in range(64):
        col, c = lane & 31, lane >> 5
        for dt in range(D // 32):
            for v4 in range(4):
                a = col * row_bytes + (((4 * dt + v4) ^ swz_k(D, col)) << 4) + 8 * c
                assert a not in written and 0 <= a < 32 * row_bytes
                written[a] = (col, 4 * dt + v4, 8 * c)
    rows_per = 64 // chunks
    read = set()
    for k in range(32 // rows_per):
        for lane in range(64):
            rr, ch = rows_per * k + lane // chunks, lane % chunks
            a = rr * row_bytes + ((ch ^ swz_k(D, rr)) << 4)
            for half in (0, 8):
                assert written[a + half] == (rr, ch, half)
                read.add(a + half)
    assert read == set(written)

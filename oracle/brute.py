"""Scalar-loop twin of the oracle, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see gqa_oracle.py). It re-derives every value
element by element with Python floats (IEEE double) and `struct` decoding,
sharing no helper with gqa_oracle.py, so that a slip in either one (a wrong
head index, a transposed operand, an off-by-one in the mask, a dropped scale)
shows up as a disagreement between the two.

Definitions followed (page titles as in gqa_oracle.py):
  * causal visibility j <= past + i: "[TorchOnnxToTorch] Add pad+scatter KV
    cache and mask to GQA", paragraph 2;
  * new rows land at seqlens_k[b] + i: same page, paragraph 2;
  * softmax(Q x K) x V per head: "KV Cache", worked example.
"""
from __future__ import annotations

import math
import struct


def _val(bits: int, dtype: str) -> float:
    if dtype == "fp32":
        return struct.unpack("<f", struct.pack("<I", bits))[0]
    if dtype == "fp16":
        return struct.unpack("<e", struct.pack("<H", bits))[0]
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]      # bf16


def _bits(x: float, dtype: str) -> int:
    """double -> float (nearest-even) -> dtype (nearest-even)."""
    f32 = struct.unpack("<I", struct.pack("<f", x))[0]     # pack('<f') rounds to nearest-even
    if dtype == "fp32":
        return f32
    f = struct.unpack("<f", struct.pack("<I", f32))[0]
    if dtype == "fp16":
        return struct.unpack("<H", struct.pack("<e", f))[0]
    keep, rest = f32 >> 16, f32 & 0xFFFF
    if rest > 0x8000 or (rest == 0x8000 and keep & 1):
        keep += 1
    return keep & 0xFFFF


def brute_attention(case, window_before_evict: bool = True):
    """Returns (out[b][i][h*D+d] as nested lists, k_cache list, v_cache list).

    Handles rotary, window eviction and append by plain loops.
    """
    B, S, H, Hkv, D, M = (case.batch, case.new_tokens, case.num_heads,
                          case.kv_num_heads, case.head_size, case.max_seq_len)
    W, dt = case.local_window_size, case.dtype
    bias = getattr(case, "attention_bias", None)
    G = H // Hkv
    sc = case.scale if case.scale != 0.0 else 1.0 / math.sqrt(D)
    kc = [[[[int(case.k_cache[b, g, t, d]) for d in range(D)] for t in range(M)]
           for g in range(Hkv)] for b in range(B)]
    vc = [[[[int(case.v_cache[b, g, t, d]) for d in range(D)] for t in range(M)]
           for g in range(Hkv)] for b in range(B)]

    def rot(bits_row, pos):
        x = [_val(int(v), dt) for v in bits_row]
        if case.cos is None:
            return [int(v) for v in bits_row]
        y = [0.0] * D
        for j in range(D // 2):
            c = float(case.cos[pos, j])
            s = float(case.sin[pos, j])
            a, bb = (2 * j, 2 * j + 1) if case.rotary_interleaved else (j, j + D // 2)
            y[a] = x[a] * c - x[bb] * s
            y[bb] = x[bb] * c + x[a] * s
        return [_bits(v, dt) for v in y]

    out = [[[0.0] * (H * D) for _ in range(S)] for _ in range(B)]
    for b in range(B):
        L = int(case.seqlens_k[b])
        qrow = [[rot(case.q[b, i, h * D:(h + 1) * D], L + i) for h in range(H)] for i in range(S)]
        krow = [[rot(case.k_new[b, i, g * D:(g + 1) * D], L + i) for g in range(Hkv)] for i in range(S)]
        vrow = [[[int(x) for x in case.v_new[b, i, g * D:(g + 1) * D]] for g in range(Hkv)] for i in range(S)]
        # logical key list (past then new), by KV head
        logical_k = [[kc[b][g][t] for t in range(L)] + [krow[i][g] for i in range(S)] for g in range(Hkv)]
        logical_v = [[vc[b][g][t] for t in range(L)] + [vrow[i][g] for i in range(S)] for g in range(Hkv)]
        for i in range(S):
            p = L + i
            for h in range(H):
                g = h // G
                scores = []
                for j in range(L + S):
                    if j > p or (W > 0 and j < p - W + 1):
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += _val(qrow[i][h][d], dt) * _val(logical_k[g][j][d], dt)
                    extra = 0.0
                    if bias is not None:   # column j: position j of past ++ new
                        bb_ = b if bias.shape[0] > 1 else 0
                        hh_ = h if bias.shape[1] > 1 else 0
                        extra = _val(int(bias[bb_, hh_, i, j]), dt)
                    scores.append((j, dot * sc + extra))
                mx = max(s for _, s in scores)
                den = sum(math.exp(s - mx) for _, s in scores)
                for d in range(D):
                    acc = 0.0
                    for j, s in scores:
                        acc += math.exp(s - mx) / den * _val(logical_v[g][j][d], dt)
                    out[b][i][h * D + d] = acc
        # cache edits: drop the oldest rows on overflow (window), then append
        start = L
        if W > 0 and L + S > M:
            drop = L + S - M
            for g in range(Hkv):
                kc[b][g][0:L - drop] = [list(r) for r in kc[b][g][drop:L]]
                vc[b][g][0:L - drop] = [list(r) for r in vc[b][g][drop:L]]
            start = L - drop
        for i in range(S):
            for g in range(Hkv):
                kc[b][g][start + i] = list(krow[i][g])
                vc[b][g][start + i] = list(vrow[i][g])
    return out, kc, vc

"""fp64 CPU oracle for GroupQueryAttention over a shared-buffer KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do. It shares no code with the HIP library and imports
nothing from it; its only inputs are numpy arrays (raw bit patterns for
tensors in the storage dtype).

Sources (the pages, by title and section):
  [P1] "Clarification about GroupQueryAttention behavior" (onnxruntime
       discussion): the question quoting the op doc on past_key (shared
       buffer of length max_sequence_length), the answer by Tianlei Wu
       (runtime check that past and present share one address; the operator
       fails when there is no room to append), and the sliding-window
       follow-up (keep the min(total, capacity) most recent tokens,
       contiguously).
  [P2] "[TorchOnnxToTorch] Add pad+scatter KV cache and mask to GQA"
       (torch-mlir pull request): paragraph 1 (Q/K/V reshape to
       [batch, seq, heads, head] then transpose; rotary positions are
       arange + past seqlens; key rotary uses kv_num_heads; seqlens_k is 0
       for an empty past; output transposed back to [batch, seq, hidden]) and
       paragraph 2 (new K/V scattered at the seqlens_k positions along the
       sequence axis; causal mask k_pos <= past_len + q_pos; seqlens_k int32).
  [P3] "KV Cache" (rocMLIR discussion): the worked prefill/decode example
       (gemm0 = Q x K, softmax, gemm1 = P x V) and the notes that the key axis
       grows, is capped at max_seq_len and is a reduction axis, so work past
       the current length is skipped rather than computed and masked.

Because skipping fully masked work, online softmax and log-sum-exp merging
are exact rewrites, the oracle is the plain definition: explicit buffer
writes and a naive per-head softmax(scale * Q K^T + mask) V over a
materialised mask, in float64.

Readings where the pages are silent (each also listed in the design notes):
  * seqlens_k[b] counts the valid tokens already in the buffer ([P2] para 1).
  * query head h reads KV head h // G with G = num_heads / kv_num_heads.
  * causal alignment is bottom-right: key j is visible to query i of
    sequence b iff j <= L_b + i ([P2] para 2).
  * a window of W keeps W keys including the query itself: j >= p - W + 1.
  * the window's cache capacity is the buffer length M; when L_b + S > M the
    oldest L_b + S - M tokens are dropped and the rest shifted to slot 0.
  * rotary is rotate-half (or interleaved pairs) over the full head, angle
    table given as fp32 inputs; each output is computed as one rounded fp64
    expression x1*c - x2*s / x2*c + x1*s (both products exact in fp64), then
    rounded to fp32 and to the storage dtype, both nearest-even.
  * rotated Q is rounded to the storage dtype before use, like rotated K.
  * rotary positions are offset_b + L_b + i, where L_b is the length before
    any eviction of the call and offset_b (0 unless given) is the absolute
    position of buffer row 0: [P2] para 1 puts the positions at arange plus
    the past length, and once a window has dropped old tokens ([P1]
    follow-up) the past length alone no longer counts them, so a caller
    keeping a rolling window passes the dropped count as the offset.
  * with a window, S > 1 and eviction, attention runs over the logical
    sequence before eviction (past ++ new), then the cache is compacted.

Status strings: "ok", "no_room", "invalid_arg".
"""
from __future__ import annotations

import copy
import math
from typing import Optional

import numpy as np

OK, NO_ROOM, INVALID = "ok", "no_room", "invalid_arg"


# ---------------------------------------------------------------------------
# storage dtypes (bit patterns <-> exact float64)
# ---------------------------------------------------------------------------

def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of each stored element (NaN poison stays NaN)."""
    if dtype == "fp32":
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_f64_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> fp32 (nearest-even) -> storage dtype (nearest-even); returns bits."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "fp32":
        return f.view(np.uint32)
    if dtype == "fp16":
        return f.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = f.view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# validation ([P1] answer: fail when there is no room; check every sequence
# before touching the buffer so a failure leaves it as it was)
# ---------------------------------------------------------------------------

def validate(case, entry: str) -> str:
    """entry in {"append", "prefill", "decode"}."""
    B, S, H, Hkv, D, M = (case.batch, case.new_tokens, case.num_heads,
                          case.kv_num_heads, case.head_size, case.max_seq_len)
    W = case.local_window_size
    if case.dtype not in ("fp32", "fp16", "bf16"):
        return INVALID
    if B < 0 or S < 0 or H < 1 or Hkv < 1 or D < 1 or M < 1 or H % Hkv:
        return INVALID
    if D > 256:
        return INVALID
    if entry in ("prefill", "decode") and S < 1:
        return INVALID
    if entry == "decode" and S != 1:
        return INVALID
    if not (W == -1 or 1 <= W <= M):
        return INVALID
    if not math.isfinite(case.scale):
        return INVALID
    lens = np.asarray(case.seqlens_k, dtype=np.int64)
    if lens.shape != (B,) or (B and (lens.min() < 0 or lens.max() > M)):
        return INVALID
    off = position_offsets(case)
    if off.shape != (B,) or (B and off.min() < 0):
        return INVALID
    rot = case.cos is not None
    if rot:
        if D % 2 or case.sin is None or case.cos.shape != case.sin.shape:
            return INVALID
        if case.cos.shape[1] != D // 2:
            return INVALID
        if B and S and int((off + lens).max()) + S > case.cos.shape[0]:
            return INVALID
    bias = getattr(case, "attention_bias", None)
    if bias is not None and entry != "append":
        if bias.ndim != 4 or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H):
            return INVALID
        if bias.shape[2] != S or (B and bias.shape[3] < int((lens + S).max())) or bias.shape[3] < 1:
            return INVALID
    windowed = W > 0 and entry != "append"
    if getattr(case, "greedy_eviction", 0) and entry != "append" and not windowed:
        return INVALID                      # greedy eviction keeps the latest W: needs a window
    if windowed:
        if S > M:
            return INVALID
    elif B and S and int((lens + S).max()) > M:
        return NO_ROOM
    return OK


# ---------------------------------------------------------------------------
# rotary ([P2] para 1: positions arange + past seqlens; K uses kv_num_heads)
# ---------------------------------------------------------------------------

def rotary_f64(x: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray,
               interleaved: int) -> np.ndarray:
    """Unrounded rotation of x[..., n, D] at integer positions pos[n].

    Pairs are (j, j + D/2) (rotate-half) or (2j, 2j+1) (interleaved).
    """
    D = x.shape[-1]
    c = cos[pos].astype(np.float64)       # [n, D/2]
    s = sin[pos].astype(np.float64)
    if interleaved:
        x1, x2 = x[..., 0::2], x[..., 1::2]
    else:
        x1, x2 = x[..., : D // 2], x[..., D // 2:]
    y1 = x1 * c - x2 * s
    y2 = x2 * c + x1 * s
    y = np.empty_like(x)
    if interleaved:
        y[..., 0::2], y[..., 1::2] = y1, y2
    else:
        y[..., : D // 2], y[..., D // 2:] = y1, y2
    return y


def _heads_first(bits: np.ndarray, B: int, S: int, nh: int, D: int) -> np.ndarray:
    """[B, S, nh*D] -> [B, nh, S, D] ([P2] para 1: reshape then transpose)."""
    return bits.reshape(B, S, nh, D).transpose(0, 2, 1, 3)


def position_offsets(case) -> np.ndarray:
    """Absolute position of buffer row 0 per sequence (zeros when not given)."""
    off = getattr(case, "position_offset", None)
    if off is None:
        return np.zeros(case.batch, dtype=np.int64)
    return np.asarray(off, dtype=np.int64)


def rotated_bits(case, bits: np.ndarray, nh: int) -> np.ndarray:
    """Q or K_new in [B, nh, S, D] bits, rotated when the case has tables.

    Token i of sequence b sits at position offset_b + L_b + i ([P2] para 1,
    with the offset of a rolling window; L_b before any eviction)."""
    B, S, D = case.batch, case.new_tokens, case.head_size
    x = _heads_first(bits, B, S, nh, D)
    if case.cos is None:
        return np.ascontiguousarray(x)
    off = position_offsets(case)
    out = np.empty(x.shape, dtype=bits.dtype)
    for b in range(B):
        pos = int(off[b]) + int(case.seqlens_k[b]) + np.arange(S)
        y = rotary_f64(to_f64(x[b], case.dtype), pos, case.cos, case.sin, case.rotary_interleaved)
        out[b] = round_f64_to_dtype(y, case.dtype)
    return out


# ---------------------------------------------------------------------------
# cache edits: eviction ([P1] follow-up) and append ([P2] para 2)
# ---------------------------------------------------------------------------

def evict(k_cache: np.ndarray, v_cache: np.ndarray, lens: np.ndarray, incoming: int,
          cap: Optional[int] = None):
    """Make room for `incoming` tokens by dropping the oldest ones.

    Only a sequence with L + incoming > M evicts. By default ([P1] follow-up:
    keep the min(total, capacity) most recent tokens) it drops
    d = L + incoming - M rows. With cap = W < M (the follow-up's "conditional
    and greedy" eviction: on overflow keep only the latest W) it keeps the
    min(L, max(0, W - incoming)) most recent past rows, so that after the
    append the buffer holds the W most recent tokens (all `incoming` of them
    when incoming > W). Rows [d, L) move to [0, L - d), in place; rows past
    L - d keep their old bytes. Returns the new lengths.
    """
    M = k_cache.shape[2]
    cap = M if cap is None else cap
    new = np.array(lens, dtype=np.int32, copy=True)
    for b in range(len(lens)):
        L = int(lens[b])
        if L + incoming <= M:
            continue
        d = L - min(L, max(0, cap - incoming))
        if d <= 0:
            continue
        for cache in (k_cache, v_cache):
            kept = cache[b, :, d:L].copy()          # copy first: no aliasing
            cache[b, :, 0:L - d] = kept
        new[b] = L - d
    return new


def append(k_cache, v_cache, lens, k_rows, v_rows):
    """cache[b, g, L_b + i] = new[b, g, i] for i < S; nothing else written."""
    S = k_rows.shape[2]
    for b in range(len(lens)):
        L = int(lens[b])
        k_cache[b, :, L:L + S] = k_rows[b]
        v_cache[b, :, L:L + S] = v_rows[b]


# ---------------------------------------------------------------------------
# attention ([P3] worked example: gemm0, softmax, gemm1; [P2] para 2: mask)
# ---------------------------------------------------------------------------

def allowed_mask(S: int, T: int, past: int, W: int) -> np.ndarray:
    """allowed[i, j] for queries at positions past + i and keys 0..T-1."""
    p = past + np.arange(S)[:, None]
    j = np.arange(T)[None, :]
    ok = j <= p
    if W > 0:
        ok &= j >= p - W + 1
    return ok


def attend_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray,
               scale: float, return_weights: bool = False, bias: Optional[np.ndarray] = None):
    """softmax(scale * q k^T + bias, masked) v for one head; q [S,D], k/v [T,D]
    fp64, bias [S,T] fp64 or None."""
    s = (q @ k.T) * scale
    if bias is not None:
        s = s + bias
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(allowed, np.exp(s - m), 0.0)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ v
    return (o, p) if return_weights else o


def scale_of(case) -> float:
    return case.scale if case.scale != 0.0 else 1.0 / math.sqrt(case.head_size)


def _attention(case, qr_bits, keys_f64, vals_f64, past, out, b):
    """Fill out[b] ([H, S, D] view) for sequence b over the given keys."""
    H, Hkv = case.num_heads, case.kv_num_heads
    G = H // Hkv
    S = case.new_tokens
    T = keys_f64.shape[1]
    allowed = allowed_mask(S, T, past, case.local_window_size)
    qf = to_f64(qr_bits[b], case.dtype)           # [H, S, D]
    sc = scale_of(case)
    bias = getattr(case, "attention_bias", None)
    for h in range(H):
        g = h // G
        # the bias column of a key is its position in past ++ new, which is
        # its index in `keys_f64` here (both branches of the whole op)
        bh = None
        if bias is not None:
            bh = to_f64(bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0, :, :T],
                        case.dtype)
        out[b, h] = attend_one(qf[h], keys_f64[g], vals_f64[g], allowed, sc, bias=bh)


def gqa_attention(case, entry: str = "prefill"):
    """The whole op: rotary -> (window) eviction -> append -> attention.

    Returns (status, out, k_cache, v_cache, lens_after) where out is fp64
    [B, S, H*D] ([P2] para 1 output layout) and the caches are new arrays
    (the inputs are not modified). On error the caches are unchanged copies.
    """
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    st = validate(case, entry)
    if st != OK:
        return st, None, kc, vc, np.array(case.seqlens_k, copy=True)
    B, S, H, Hkv, D, M = (case.batch, case.new_tokens, case.num_heads,
                          case.kv_num_heads, case.head_size, case.max_seq_len)
    W = case.local_window_size
    lens = np.asarray(case.seqlens_k, dtype=np.int32)
    qr = rotated_bits(case, case.q, H)             # [B, H, S, D]
    kr = rotated_bits(case, case.k_new, Hkv)       # [B, Hkv, S, D]
    vr = np.ascontiguousarray(_heads_first(case.v_new, B, S, Hkv, D))
    out = np.zeros((B, H, S, D), dtype=np.float64)
    needs_evict = W > 0 and B > 0 and int((lens + S).max()) > M

    if needs_evict:
        # attention first over the logical sequence past ++ new (then compact)
        for b in range(B):
            L = int(lens[b])
            keys = np.concatenate([to_f64(kc[b, :, :L], case.dtype), to_f64(kr[b], case.dtype)], axis=1)
            vals = np.concatenate([to_f64(vc[b, :, :L], case.dtype), to_f64(vr[b], case.dtype)], axis=1)
            _attention(case, qr, keys, vals, L, out, b)
        cap = W if getattr(case, "greedy_eviction", 0) else M
        lens2 = evict(kc, vc, lens, S, cap)
        append(kc, vc, lens2, kr, vr)
    else:
        append(kc, vc, lens, kr, vr)
        lens2 = lens.copy()
        for b in range(B):
            L = int(lens[b])
            keys = to_f64(kc[b, :, :L + S], case.dtype)
            vals = to_f64(vc[b, :, :L + S], case.dtype)
            _attention(case, qr, keys, vals, L, out, b)
    out = out.transpose(0, 2, 1, 3).reshape(B, S, H * D)
    return OK, out, kc, vc, lens2 + S


def gqa_attention_present(case, past_k: np.ndarray, past_v: np.ndarray):
    """The whole op with separate past and present buffers ([P1] question:
    past is of length past_sequence_length unless it is the present tensor;
    the asker's summary: with different shapes, present is past + new in a
    different tensor).

    case.k_cache / case.v_cache are the present buffers [B, Hkv, M, D] as they
    stand before the call; past_k / past_v [B, Hkv, past_rows, D] hold rows
    [0, L_b) of each sequence. Present rows [0, L_b) take the past rows, then
    the op runs on present exactly as in shared mode. Returns what
    gqa_attention returns; past is never modified.
    """
    st = validate(case, "prefill")
    lens = np.asarray(case.seqlens_k, dtype=np.int64)
    past_rows = past_k.shape[2]
    if st == OK and case.batch and int(lens.max()) > past_rows:
        st = INVALID
    if st != OK:
        return st, None, case.k_cache.copy(), case.v_cache.copy(), np.array(case.seqlens_k, copy=True)
    present = copy.copy(case)               # same inputs, own present arrays
    present.k_cache, present.v_cache = case.k_cache.copy(), case.v_cache.copy()
    for b in range(case.batch):
        L = int(lens[b])
        present.k_cache[b, :, :L] = past_k[b, :, :L]
        present.v_cache[b, :, :L] = past_v[b, :, :L]
    return gqa_attention(present, "prefill")


def gqa_append_kv(case):
    """Append half: rotary on K (if tables are given), then the scatter.

    No eviction: with L_b + S > M it fails with no_room, window or not.
    """
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    st = validate(case, "append")
    if st != OK:
        return st, kc, vc
    B, S, Hkv, D = case.batch, case.new_tokens, case.kv_num_heads, case.head_size
    kr = rotated_bits(case, case.k_new, Hkv)
    vr = np.ascontiguousarray(_heads_first(case.v_new, B, S, Hkv, D))
    append(kc, vc, np.asarray(case.seqlens_k), kr, vr)
    return OK, kc, vc


def gqa_evict_window(case, incoming: int):
    """Eviction half: compact each sequence so `incoming` tokens fit.

    Returns (status, k_cache, v_cache, lens_after) with
    lens_after[b] = min(L_b, M - incoming).
    """
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    lens = np.asarray(case.seqlens_k, dtype=np.int64)
    M = case.max_seq_len
    bad = (incoming < 0 or incoming > M or case.kv_num_heads < 1 or case.head_size < 1
           or case.head_size > 256 or lens.shape != (case.batch,)
           or (case.batch and (lens.min() < 0 or lens.max() > M)))
    if bad:
        return INVALID, kc, vc, np.array(case.seqlens_k, copy=True)
    new = evict(kc, vc, np.asarray(case.seqlens_k, dtype=np.int32), incoming)
    return OK, kc, vc, new


# ---------------------------------------------------------------------------
# split-KV partials and their log-sum-exp merge (exact rewrite of one softmax)
# ---------------------------------------------------------------------------

def partial_attention(q, k, v, allowed, scale):
    """(o_unnormalised / l, m, l) of one query row over a subset of keys.

    q [D], k/v [T, D], allowed [T]. Returns (o [D], m, l) with
    o = sum_j e^{s_j - m} v_j / l, l = sum_j e^{s_j - m}, m = max_j s_j.
    """
    s = (k @ q) * scale
    if not allowed.any():
        return np.zeros(q.shape[0]), -np.inf, 0.0
    m = s[allowed].max()
    e = np.where(allowed, np.exp(np.where(allowed, s, m) - m), 0.0)
    l = e.sum()
    return (e @ v) / l, m, l


def lse_merge(parts):
    """Merge partials (o_s, m_s, l_s): m = max m_s, l = sum l_s e^{m_s - m},
    o = sum (l_s e^{m_s - m} / l) o_s."""
    m = max(p[1] for p in parts)
    w = [p[2] * math.exp(p[1] - m) if p[2] > 0 else 0.0 for p in parts]
    l = sum(w)
    return sum(wi / l * p[0] for wi, p in zip(w, parts))

"""The decode entry point that allocates nothing (its workspace is the
library's static device scratch), through the C ABI, against
gqa_attention_decode on the same inputs: both caches bit for bit and the
outputs within the tolerance of the fp64 comparison (1e-4 fp32, 2e-2
fp16/bf16), and both against the oracle. Two calls in a row on the shared
scratch, the second with a smaller input, so that counters left by the first
call and stale partials cannot leak into the second."""
import numpy as np
import pytest

import gqa_inputs as gi
from oracle import gqa_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_query_kv_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch


def _compare(case, what):
    import torch
    import grouped_query_kv_amd as gqa
    from gpu_helpers import DevCase, assert_bits_equal, assert_close, out_f64
    print(f"[gpu] no-alloc {what}: B={case.batch} H={case.num_heads} Hkv={case.kv_num_heads} "
          f"M={case.max_seq_len} dt={case.dtype} W={case.local_window_size} "
          f"lens={list(case.seqlens_k)[:8]}", flush=True)
    st, want, kc, vc, _ = O.gqa_attention(case, "decode")
    assert st == O.OK
    ref, mine = DevCase(case), DevCase(case)
    out_ref = ref.run("decode")
    out = torch.empty_like(mine.q)
    gqa.gqa_attention_decode_noalloc(mine.q, mine.k_new, mine.v_new, mine.k_cache, mine.v_cache,
                                     mine.lens_host, mine.lens_dev, out, scale=case.scale,
                                     local_window_size=case.local_window_size, cos_cache=mine.cos,
                                     sin_cache=mine.sin,
                                     rotary_interleaved=case.rotary_interleaved,
                                     greedy_eviction=bool(case.greedy_eviction),
                                     attention_bias=mine.bias)
    torch.cuda.synchronize()
    rk, rv = ref.caches()
    gk, gv = mine.caches()
    assert_bits_equal(gk, rk, f"{what}: k_cache vs gqa_attention_decode")
    assert_bits_equal(gv, rv, f"{what}: v_cache vs gqa_attention_decode")
    assert_bits_equal(gk, kc, f"{what}: k_cache vs oracle")
    assert_bits_equal(gv, vc, f"{what}: v_cache vs oracle")
    got, exp = out_f64(out, case.dtype), out_f64(out_ref, case.dtype)
    assert_close(got, exp, case.dtype, f"{what}: out vs gqa_attention_decode")
    err = assert_close(got, want, case.dtype, f"{what}: out vs oracle")
    print(f"[gpu]   max abs error {err:.3e}; max difference to gqa_attention_decode "
          f"{float(np.abs(got - exp).max()):.3e}", flush=True)


def test_noalloc_equals_decode_on_two_calls_in_a_row():
    # the split-KV decode workload (16 sequences, 8 kv heads, many units cut
    # between workgroups), then a smaller call with fewer units: a full
    # window cache (fused eviction), rotary and a bias
    _compare(gi.workload("split-kv-decode-fp16"), "call 1")
    small = gi.make_case("noalloc-small", "bf16", 3, 1, 16, 4, 128, 512, [512, 300, 7], 21,
                         window=512, rotary=True, rotary_rows=600)
    rng = np.random.default_rng(21)
    small.attention_bias = gi.to_bits(rng.standard_normal((3, 16, 1, 515)), "bf16")
    _compare(small, "call 2")

"""The entry point that allocates nothing (attn_bias_gqa_fwd_noalloc: the
library's own per-GPU scratch array) against attn_bias_gqa_fwd with a
workspace, through the C ABI: bit-identical outputs, on calls in a row whose
later inputs are smaller than the earlier ones (decode with split records and
arrival counts, then prefill with a live-tile map), both mask variants."""
import numpy as np
import pytest
import torch

import additive_bias_gqa_amd as ab
import oracle
from additive_bias_gqa_amd import workloads as wl
from pipeline import announce, check_parity, dead_rows, dev, fwd, poisoned, to_f64

pytestmark = pytest.mark.gpu


def _cases():
    return [
        wl.decode_full(B=8, Hq=16, Hkv=4, D=512, max_seq=2048, nonpad_lo=100),
        wl.decode_sliding(B=3, Hq=8, Hkv=4, D=256, max_seq=600, window=100, nonpad_lo=1),
        wl.prefill_vision(B=2, Hq=8, Hkv=4, D=256, S_q=200, max_seq=1024, window=256,
                          start_hi=600, block=64),
        wl.prefill_vision(B=1, Hq=4, Hkv=2, D=256, S_q=40, max_seq=256, window=64,
                          start_hi=100, block=16),
    ]


@pytest.mark.parametrize("variant", ["bias", "rules"])
def test_noalloc_matches_workspace_entry(variant):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    for w in _cases():
        st = w.steps[0]
        announce(f"no-alloc {variant} {w.name}")
        k, v = dev(w.k_cache), dev(w.v_cache)
        ab.kv_tensor_scatter(k, dev(st.k_new), dev(st.write_indices))
        ab.kv_tensor_scatter(v, dev(st.v_new), dev(st.write_indices))
        q, npd, qs, kind = dev(st.q), dev(st.nonpad), dev(st.q_start), dev(st.slot_kind)
        bias = None
        if variant == "bias":
            bias = ab.build_static_cache_bias(npd, qs, kind, st.S_q, w.max_seq, w.window, dtype=w.dtype)
        rules = dict(q_start=qs, slot_kind=kind, window=w.window) if variant == "rules" else {}
        ref = fwd(q, k, v, bias, npd, w.scale, **rules)
        for rep in range(2):
            got = ab.attn_bias_gqa_fwd_noalloc(q, k, v, bias, npd, w.scale,
                                               out=poisoned((w.B, w.Hq, st.S_q, w.Dv), w.dtype), **rules)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{w.name} call {rep}"
        # and the oracle's result, to the stated tolerance
        k_h = oracle.scatter(w.k_cache, st.k_new, st.write_indices)
        v_h = oracle.scatter(w.v_cache, st.v_new, st.write_indices)
        b_ref = oracle.bias(st.nonpad, st.q_start, st.slot_kind, st.S_q, w.max_seq, w.window)
        y_ref = oracle.attention(st.q, k_h, v_h, b_ref, st.nonpad, w.scale)
        check_parity(to_f64(got), y_ref, w.dtype, dead_rows(b_ref, st.nonpad, w.Hq), f"noalloc/{w.name}")


def test_noalloc_refuses_large_scratch():
    B, Hq, Hkv, T, D = 2048, 16, 8, 16, 512
    assert ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, 1, T, D) > 8 << 20
    q = torch.zeros((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, T, D), dtype=torch.bfloat16, device="cuda")
    n = torch.full((B,), T, dtype=torch.int64, device="cuda")
    with pytest.raises(RuntimeError, match="holds 8388608"):
        ab.attn_bias_gqa_fwd_noalloc(q, k, k, None, n, 0.05, out=torch.empty_like(q))

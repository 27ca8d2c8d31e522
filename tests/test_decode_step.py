"""The fused decode step (attn_bias_gqa_decode_step and its circular form)
against the separate calls it replaces and against the oracle.

The step does a decode step's TensorScatter of K and V, its bias build and its
attention in one launch. Its results must be those of kv_tensor_scatter (K, V),
build_static_cache_bias and attn_bias_gqa_fwd with that bias, bit for bit
(caches, bias and output), and the output must match the fp64 oracle within the
bf16 tolerance. Every output, bias and workspace starts poisoned."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import additive_bias_gqa_amd as ab
from additive_bias_gqa_amd import workloads as wl
from pipeline import (announce, check_parity, dead_rows, dev, fused_step, gpu_step, oracle_step,
                      poisoned, poisoned_workspace, same_bits)

pytestmark = pytest.mark.gpu


def check_step(w: wl.Workload, step: wl.Step, bias_dtype=torch.bfloat16, with_bias=True,
               softcap=0.0, default_q_start=False, oracle_check=True):
    k1, v1 = dev(w.k_cache.clone()), dev(w.v_cache.clone())
    k2, v2 = dev(w.k_cache.clone()), dev(w.v_cache.clone())
    bias1, out1 = gpu_step(w, step, k1, v1, bias_dtype=bias_dtype, softcap=softcap,
                           default_q_start=default_q_start)
    bias2, out2 = fused_step(w, step, k2, v2, bias_dtype=bias_dtype, with_bias=with_bias,
                             softcap=softcap, default_q_start=default_q_start)
    torch.cuda.synchronize()
    assert same_bits(k1, k2), "K cache after the step"
    assert same_bits(v1, v2), "V cache after the step"
    if with_bias:
        assert same_bits(bias1, bias2), "bias"
    assert same_bits(out1, out2), "output differs from the separate calls"
    if oracle_check:
        k_ref, v_ref, bias_ref, ref = oracle_step(w, step, w.k_cache.clone(), w.v_cache.clone(),
                                                  default_q_start=default_q_start, softcap=softcap)
        assert same_bits(k2.cpu(), k_ref), "K cache against the oracle"
        assert same_bits(v2.cpu(), v_ref), "V cache against the oracle"
        valid = step.nonpad.clamp(0, w.max_seq) if w.circular else step.nonpad
        got = out2.float().cpu().numpy().astype(np.float64)
        check_parity(got, ref, w.dtype, dead_rows(bias_ref, valid, w.Hq), w.name)


CASES = {
    "sliding_d256": lambda: wl.decode_sliding(B=3, Hq=4, Hkv=2, D=256, max_seq=1001, window=300,
                                              nonpad_lo=1),
    "full_d512": lambda: wl.decode_full(B=3, Hq=8, Hkv=2, D=512, max_seq=777, nonpad_lo=1),
    "full_kvshared": lambda: wl.decode_full(B=3, Hq=8, Hkv=2, D=512, max_seq=777, nonpad_lo=1,
                                            kv_shared=True),
    "d64_g8": lambda: wl.decode_sliding(B=2, Hq=16, Hkv=2, D=64, max_seq=300, window=50, nonpad_lo=1),
    "d128_g1": lambda: wl.decode_full(B=2, Hq=4, Hkv=4, D=128, max_seq=512, nonpad_lo=1),
    "g3": lambda: wl.decode_full(B=2, Hq=6, Hkv=2, D=256, max_seq=200, nonpad_lo=1),
    "g16": lambda: wl.decode_sliding(B=2, Hq=32, Hkv=2, D=128, max_seq=400, window=0, nonpad_lo=1),
    "b64": lambda: wl.decode_full(B=64, Hq=8, Hkv=4, D=128, max_seq=300, nonpad_lo=1),
    "dv256": lambda: wl.decode_full(B=3, Hq=8, Hkv=2, D=512, Dv=256, max_seq=640, nonpad_lo=1),
    "dv512": lambda: wl.decode_full(B=3, Hq=8, Hkv=2, D=256, Dv=512, max_seq=640, nonpad_lo=1),
    "circ_d256": lambda: wl.decode_sliding_circular(B=5, Hq=8, Hkv=4, D=256, capacity=300, window=200,
                                                    len_lo=1, len_hi=1000),
    "circ_d512": lambda: wl.decode_sliding_circular(B=4, Hq=16, Hkv=4, D=512, capacity=256, window=256,
                                                    len_lo=100, len_hi=900),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_equals_separate_calls(name):
    w = CASES[name]()
    announce(f"decode step {name} {w.name}")
    check_step(w, w.steps[0])


@pytest.mark.parametrize("bias_dtype,with_bias", [(torch.float32, True), (torch.bfloat16, False)])
def test_step_bias_output(bias_dtype, with_bias):
    w = CASES["sliding_d256"]()
    announce(f"decode step bias {bias_dtype} written={with_bias}")
    check_step(w, w.steps[0], bias_dtype=bias_dtype, with_bias=with_bias)


def test_step_softcap_and_default_q_start():
    w = CASES["full_d512"]()
    announce("decode step softcap 50, default q_start")
    check_step(w, w.steps[0], softcap=50.0, default_q_start=True)


def test_step_edges():
    """Two new tokens per row (S_q = S_new = 2) with write slots that drop a
    token (the last slot of the cache, a negative first position), a new token
    past nonpad, a batch row with nonpad = 0, slots of an image block and pads."""
    B, Hq, Hkv, D, T, S = 5, 8, 4, 256, 96, 2
    dt = torch.bfloat16
    rng = np.random.Generator(np.random.PCG64(4242))
    kc = wl.normal(rng, (B, Hkv, T, D), dt)   # every slot finite: nonpad reaches T in row 0
    vc = wl.normal(rng, (B, Hkv, T, D), dt)
    q = wl.normal(rng, (B, Hq, S, D), dt)
    kn = wl.normal(rng, (B, Hkv, S, D), dt)
    vn = wl.normal(rng, (B, Hkv, S, D), dt)
    wi = torch.tensor([T - 1, -1, 40, 10, 60], dtype=torch.int64)   # row 0: 2nd token dropped; row 1: 1st
    nonpad = torch.tensor([T, 1, 30, 0, 62], dtype=torch.int64)    # row 2: tokens past nonpad
    q_start = torch.tensor([T - 2, 0, 40, 0, 60], dtype=torch.int64)
    kind = torch.zeros((B, T), dtype=torch.int32)
    kind[4, 50:62] = 1            # an image block holding both queries of row 4
    kind[2, 0:5] = wl.PAD
    step = wl.Step(q, kn, vn, wi, nonpad, q_start, kind)
    w = wl.Workload("step_edges", dt, B, Hq, Hkv, D, T, 20, D ** -0.5, kc, vc, [step])
    announce("decode step edges")
    check_step(w, step)


def _with_pads(w: wl.Workload) -> wl.Step:
    """The workload's step with pad slots placed at the ends of the batch rows'
    causal/window intervals (and elsewhere), one pattern per row."""
    st = w.steps[0]
    kind = torch.zeros((w.B, w.max_seq), dtype=torch.int32)
    for b in range(w.B):
        n = int(st.nonpad[b])
        q = n - 1
        lo = max(q - w.window + 1, 0) if w.window > 0 else 0
        pattern = b % 8
        if pattern == 1:
            kind[b, :min(75, n)] = wl.PAD                 # leading pads
        elif pattern == 2:
            kind[b, :max(n - 200, 1)] = wl.PAD            # all but the last 200 keys
        elif pattern == 3:
            kind[b, max(n - 3, 0):n] = wl.PAD             # trailing pads, the query slot among them
        elif pattern == 4:
            kind[b, lo + 20:lo + 50] = wl.PAD             # inside the interval only: ends exact
        elif pattern == 5:
            kind[b, :n] = wl.PAD                          # every valid slot: no live key
        elif pattern == 6:
            kind[b, lo:lo + 9] = wl.PAD                   # the interval's first keys
        elif pattern == 7:
            kind[b, lo] = wl.PAD                          # exactly the first key
            kind[b, q] = wl.PAD                           # and the last
    return wl.Step(st.q, st.k_new, st.v_new, st.write_indices, st.nonpad, st.q_start, kind)


PAD_CASES = {
    # 2 and 4 rows per lane group at head 256 (eight wavefronts), head 512, head 128
    "sliding_g2": lambda: wl.decode_sliding(B=8, Hq=16, Hkv=8, D=256, max_seq=2048, window=700,
                                            nonpad_lo=400),
    "sliding_g4": lambda: wl.decode_sliding(B=8, Hq=32, Hkv=8, D=256, max_seq=2048, window=700,
                                            nonpad_lo=400),
    "full_d512": lambda: wl.decode_full(B=8, Hq=16, Hkv=4, D=512, max_seq=2048, nonpad_lo=400),
    "full_d128": lambda: wl.decode_full(B=16, Hq=32, Hkv=8, D=128, max_seq=1500, nonpad_lo=300),
}


@pytest.mark.parametrize("name", list(PAD_CASES))
def test_step_pad_ends(name):
    """Pad slots at the ends of the causal/window interval: the rules form (the
    fused step's and attn_bias_gqa_fwd's without a bias) must find the same live
    key range as a scan of the bias, or its splits would sum in another order.
    Outputs of many rows and heads, so that a changed order shows through the
    bf16 rounding of the output."""
    w = PAD_CASES[name]()
    step = _with_pads(w)
    announce(f"decode step pad ends {w.name}")
    check_step(w, step)
    _, o_bias = gpu_step(w, step, dev(w.k_cache.clone()), dev(w.v_cache.clone()), rules=False)
    _, o_rules = gpu_step(w, step, dev(w.k_cache.clone()), dev(w.v_cache.clone()), rules=True)
    torch.cuda.synchronize()
    assert same_bits(o_bias, o_rules), "rules form differs from the bias form"


FULL_STEP = {
    "decode_sliding": wl.decode_sliding,
    "decode_full": wl.decode_full,
    "decode_sliding_circular": wl.decode_sliding_circular,
    # batches that do not divide the 256 CUs (5 splits of 96 pairs; 1 split of 320)
    "decode_sliding_b12": lambda: wl.decode_sliding(B=12),
    "decode_sliding_b40": lambda: wl.decode_sliding(B=40),
    "decode_full_b24": lambda: wl.decode_full(B=24),
}


@pytest.mark.parametrize("name", list(FULL_STEP))
def test_step_full_size(name):
    """The full-size workloads, bit for bit against the separate calls (whose
    output the full-size parity tests compare with the oracle)."""
    w = FULL_STEP[name]()
    announce(f"decode step full size {w.name}")
    check_step(w, w.steps[0], oracle_check=False)


def test_step_graph_replay():
    """The step captured in a HIP graph and replayed three times, eager work
    and synchronisations between the replays: every replay gives the eager
    result (the step rewrites the same cache rows each time)."""
    w = CASES["sliding_d256"]()
    step = w.steps[0]
    announce("decode step graph replay")
    k, v = dev(w.k_cache.clone()), dev(w.v_cache.clone())
    bias_e, out_e = fused_step(w, step, k, v)
    B, Hq, S_q, D = step.q.shape
    q, kn, vn = dev(step.q), dev(step.k_new), dev(step.v_new)
    wi, npd, qs, kind = dev(step.write_indices), dev(step.nonpad), dev(step.q_start), dev(step.slot_kind)
    bias = poisoned((w.B, 1, S_q, w.max_seq), torch.bfloat16)
    out = poisoned((B, Hq, S_q, D), w.dtype)
    ws = poisoned_workspace(ab.attn_bias_gqa_workspace_bytes(B, Hq, w.Hkv, S_q, w.max_seq, D, D))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ab.attn_bias_gqa_decode_step(q, k, v, kn, vn, wi, npd, w.scale, q_start=qs, slot_kind=kind,
                                     window=w.window, bias=bias, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ab.attn_bias_gqa_decode_step(q, k, v, kn, vn, wi, npd, w.scale, q_start=qs, slot_kind=kind,
                                     window=w.window, bias=bias, out=out, workspace=ws)
    for rep in range(3):
        out.view(torch.int16).fill_(0x7FC1)
        bias.view(torch.int16).fill_(0x7FC1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(out, out_e), f"replay {rep}: output"
        assert same_bits(bias, bias_e), f"replay {rep}: bias"
        _ = (q.float() * 2).sum().item()   # eager work between replays


def test_step_check_mode(monkeypatch):
    """ABGQA_CHECK=1 on the fused step: write indices, nonpad and q_start are
    validated on the host before anything is enqueued, a workspace with a
    nonzero arrival count is refused, and a valid step under the check still
    matches the separate calls bit for bit."""
    monkeypatch.setenv("ABGQA_CHECK", "1")
    w = CASES["sliding_d256"]()
    step = w.steps[0]
    B = w.B
    k, v = dev(w.k_cache.clone()), dev(w.v_cache.clone())
    q, kn, vn = dev(step.q), dev(step.k_new), dev(step.v_new)
    npd, qs = dev(step.nonpad), dev(step.q_start)
    bad_w = step.write_indices.clone()
    bad_w[1] = w.max_seq            # the new token's slot past the cache
    announce("decode step check mode: bad device values refused")
    with pytest.raises(RuntimeError, match=r"ABGQA_CHECK: write_indices\[1\]"):
        ab.attn_bias_gqa_decode_step(q, k, v, kn, vn, dev(bad_w), npd, w.scale, q_start=qs,
                                     window=w.window)
    bad_np = step.nonpad.clone()
    bad_np[0] = -2
    with pytest.raises(RuntimeError, match=r"ABGQA_CHECK: nonpad_kv_seqlen\[0\] = -2"):
        ab.attn_bias_gqa_decode_step(q, k, v, kn, vn, dev(step.write_indices), dev(bad_np), w.scale,
                                     q_start=qs, window=w.window)
    bad_qs = step.q_start.clone()
    bad_qs[2] = -5
    with pytest.raises(RuntimeError, match=r"ABGQA_CHECK: q_start\[2\] = -5"):
        ab.attn_bias_gqa_decode_step(q, k, v, kn, vn, dev(step.write_indices), npd, w.scale,
                                     q_start=dev(bad_qs), window=w.window)
    D = step.q.shape[3]
    ws = poisoned_workspace(ab.attn_bias_gqa_workspace_bytes(B, w.Hq, w.Hkv, 1, w.max_seq, D, D))
    ws[4:8] = torch.tensor([3, 0, 0, 0], dtype=torch.uint8)    # arrival count 1 left at 3
    with pytest.raises(RuntimeError, match="ABGQA_CHECK: decode arrival count 1"):
        ab.attn_bias_gqa_decode_step(q, k, v, kn, vn, dev(step.write_indices), npd, w.scale,
                                     q_start=qs, window=w.window, workspace=ws)
    assert same_bits(k, dev(w.k_cache)), "a refused call must not have touched the cache"
    announce("decode step check mode: valid step")
    check_step(w, step, oracle_check=False)

"""Seeded random shapes through the whole hot path, GPU against the oracle.

Each case draws a shape from the ranges the library takes (head sizes 64 to
512 and the two mixed pairs, 1 to 8 query heads per KV head, static or
circular cache, decode or prefill chunk, aligned or ragged cache length,
window or none, image blocks, left padding, softcap, bf16 or fp32, bias
variant with a bf16 or fp32 bias, or the in-kernel rules) and runs TensorScatter
of K and V, the bias build and the attention on both sides: the caches and the
bias must match bit for bit, the output within the stated tolerance, and rows
with no allowed key must be exact zeros. A decode-sized shape (S_q * G <= 16)
also runs the attention's other form (bias <-> rules), which must give the
same bits, and in bf16 the fused decode step (scatters, bias and attention in
one launch), which must give the separate calls' caches, bias and output bit
for bit. Outputs, biases and
workspaces start poisoned, so an unwritten element fails. Sizes keep the fp64
oracle to well under a second per case.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from additive_bias_gqa_amd import workloads as wl
from pipeline import announce, check_parity, dead_rows, dev, fused_step, gpu_step, oracle_step, same_bits

pytestmark = pytest.mark.gpu

N_CASES = 240
PAIRS_BF16 = [(64, 64), (128, 128), (256, 256), (512, 512), (256, 512), (512, 256)]
PAIRS_F32 = [(64, 64), (128, 128), (64, 128)]


def draw_case(i: int):
    rng = np.random.Generator(np.random.PCG64(9000 + i))
    dtype = torch.float32 if rng.random() < 0.2 else torch.bfloat16
    pairs = PAIRS_F32 if dtype == torch.float32 else PAIRS_BF16
    D, Dv = pairs[int(rng.integers(len(pairs)))]
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 4))
    circular = bool(rng.random() < 0.2)
    T = int(rng.integers(8, 129)) * 8 if rng.random() < 0.8 else int(rng.integers(40, 800))
    kind_r = rng.random()
    S_q = 1 if kind_r < 0.4 else (int(rng.integers(2, 5)) if kind_r < 0.55 else int(rng.integers(5, 161)))
    S_q = min(S_q, T)
    if S_q > 16:           # keep the oracle's work bounded
        T = min(T, 640)
        S_q = min(S_q, T)
    window = 0 if rng.random() < 0.4 else int(rng.integers(1, T + 1))
    blocks = bool(rng.random() < 0.3) and S_q >= 4
    pads = bool(rng.random() < 0.2) and not circular
    softcap = 0.0 if rng.random() < 0.8 else float(rng.choice([20.0, 50.0]))
    variant = str(rng.choice(["bias_bf16", "bias_f32", "rules"]))
    if dtype == torch.float32 and variant == "bias_bf16":
        variant = "bias_f32"
    default_q_start = bool(rng.random() < 0.3)

    Hq = G * Hkv
    if circular:
        # tokens written after the step; the S_q new ones go to positions L - S_q ..
        L = rng.integers(S_q, 3 * T + 1, size=B).astype(np.int64)
        before = L - S_q
        kc = wl._fill_circular(rng, B, Hkv, T, D, before, dtype)
        vc = wl._fill_circular(rng, B, Hkv, T, Dv, before, dtype)
        nonpad = L
    else:
        nonpad = rng.integers(S_q, T + 1, size=B).astype(np.int64)
        nonpad[rng.random(B) < 0.15] = S_q
        before = nonpad - S_q
        kc = wl._fill_cache(rng, B, Hkv, T, D, before, dtype)
        vc = wl._fill_cache(rng, B, Hkv, T, Dv, before, dtype)
    q = wl.normal(rng, (B, Hq, S_q, D), dtype)
    kn = wl.normal(rng, (B, Hkv, S_q, D), dtype)
    vn = wl.normal(rng, (B, Hkv, S_q, Dv), dtype)
    kind = torch.zeros((B, T), dtype=torch.int32)
    for b in range(B):
        start = int(before[b])
        if blocks:
            for blk in range(int(rng.integers(1, 3))):
                size = int(rng.integers(2, S_q + 1))
                off = int(rng.integers(0, S_q - size + 1))
                for t in range(off, off + size):
                    kind[b, (start + t) % T] = blk + 1
        if pads and start > 0:
            kind[b, :int(rng.integers(0, start + 1))] = wl.PAD
    wi = torch.from_numpy(before.copy())
    npt = torch.from_numpy(nonpad.copy())
    step = wl.Step(q, kn, vn, wi, npt, wi.clone(), kind if (blocks or pads or rng.random() < 0.5) else None)
    w = wl.Workload(f"fuzz{i}", dtype, B, Hq, Hkv, D, T, window, 1.0 / math.sqrt(D), kc, vc, [step],
                    circular=circular)
    desc = dict(dtype=str(dtype).replace("torch.", ""), B=B, Hq=Hq, Hkv=Hkv, D=D, Dv=Dv, T=T, S_q=S_q,
                window=window, circular=circular, blocks=blocks, pads=pads, softcap=softcap,
                variant=variant, default_q_start=default_q_start, nonpad=nonpad.tolist())
    return w, step, variant, softcap, default_q_start, desc


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_case(i):
    w, step, variant, softcap, default_q_start, desc = draw_case(i)
    announce(f"fuzz {i} {desc}")
    k_dev, v_dev = dev(w.k_cache.clone()), dev(w.v_cache.clone())
    rules = variant == "rules"
    bias_dtype = torch.float32 if variant == "bias_f32" else torch.bfloat16
    bias, out = gpu_step(w, step, k_dev, v_dev, rules=rules, bias_dtype=bias_dtype,
                         default_q_start=default_q_start, softcap=softcap)
    k_ref, v_ref, bias_ref, ref = oracle_step(w, step, w.k_cache.clone(), w.v_cache.clone(),
                                              default_q_start=default_q_start, softcap=softcap)
    assert torch.equal(k_dev.cpu().view(torch.uint8), k_ref.view(torch.uint8)), "K cache after TensorScatter"
    assert torch.equal(v_dev.cpu().view(torch.uint8), v_ref.view(torch.uint8)), "V cache after TensorScatter"
    if bias is not None:
        ref_bits = torch.from_numpy(np.ascontiguousarray(bias_ref)).to(bias_dtype)
        assert torch.equal(bias.cpu().view(torch.uint8), ref_bits.view(torch.uint8)), "bias"
    valid = step.nonpad.clamp(0, w.max_seq) if w.circular else step.nonpad
    got = out.float().cpu().numpy().astype(np.float64)
    check_parity(got, ref, w.dtype, dead_rows(bias_ref, valid, w.Hq), f"fuzz{i}")
    # a decode shape (S_q * Hq / Hkv <= 16): the bias and the rules forms of
    # the attention take the same kernel and must give the same bits (the
    # rules form finds the same live key range as a scan of the bias)
    if step.S_q * (w.Hq // w.Hkv) <= 16:
        k3, v3 = dev(w.k_cache.clone()), dev(w.v_cache.clone())
        _, out3 = gpu_step(w, step, k3, v3, rules=not rules, bias_dtype=bias_dtype,
                           default_q_start=default_q_start, softcap=softcap)
        assert same_bits(out3, out), "bias and rules forms differ"
    # a bf16 decode shape (S_q * Hq / Hkv <= 16, head sizes of the split-KV
    # kernel): the fused decode step must reproduce the separate calls bit for
    # bit (caches, the bias when built, output)
    Dv = w.v_cache.shape[3]
    decode_pair = (w.D == Dv and w.D in (64, 128, 256, 512)) or (w.D, Dv) in ((256, 512), (512, 256))
    if w.dtype == torch.bfloat16 and step.S_q * (w.Hq // w.Hkv) <= 16 and decode_pair:
        k2, v2 = dev(w.k_cache.clone()), dev(w.v_cache.clone())
        bias2, out2 = fused_step(w, step, k2, v2, bias_dtype=bias_dtype, with_bias=not rules,
                                 softcap=softcap, default_q_start=default_q_start)
        assert same_bits(k2, k_dev) and same_bits(v2, v_dev), "fused step: caches"
        if not rules:
            assert same_bits(bias2, bias), "fused step: bias"
        assert same_bits(out2, out), "fused step: output differs from the separate calls"

"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

TensorScatter and the bias are compared bit for bit; attention within fp32
max-abs 1e-5, or bf16 max-abs 2e-2 and mean-rel 1e-2, with fully-masked rows
required to be exact zeros. Small shapes compare every output element (several
tiles, ragged tails); the five full-size workloads compare sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import additive_bias_gqa_amd as ab
import oracle
from additive_bias_gqa_amd import workloads as wl
from pipeline import (announce, check_parity, dead_rows, dev, fwd, gpu_step, oracle_step, poison_,
                      poisoned, poisoned_workspace, tile_rows, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run them with -m gpu on an MI355X)")
    ab.load()
    torch.cuda.synchronize()


# --------------------------------------------------------------------------- #
# TensorScatter: bit-exact
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 256, 512])
def test_scatter_bit_exact(dtype, D):
    announce(f"scatter dtype={dtype} D={D}")
    rng = wl.rng_for(200 + D)
    B, H, T, S_new = 4, 3, 37, 9
    cache = wl.garbage(rng, (B, H, T, D), dtype)
    upd = wl.garbage(rng, (B, H, S_new, D), dtype)
    w = torch.tensor([0, 5, T - S_new, T - 3], dtype=torch.int64)  # last runs off the end
    ref = oracle.scatter(cache, upd, w)
    c = dev(cache)
    ab.kv_tensor_scatter(c, dev(upd), dev(w))
    ibits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(c.cpu().view(ibits), ref.view(ibits))


def test_scatter_null_indices_and_noop():
    announce("scatter null indices / S_new=0")
    rng = wl.rng_for(210)
    cache = wl.garbage(rng, (2, 2, 16, 256), torch.bfloat16)
    upd = wl.garbage(rng, (2, 2, 3, 256), torch.bfloat16)
    c = dev(cache)
    ab.kv_tensor_scatter(c, dev(upd), None)
    ref = oracle.scatter(cache, upd, None)
    assert torch.equal(c.cpu().view(torch.int16), ref.view(torch.int16))
    empty = torch.empty((2, 2, 0, 256), dtype=torch.bfloat16)
    ab.kv_tensor_scatter(c, dev(empty), None)
    assert torch.equal(c.cpu().view(torch.int16), ref.view(torch.int16))


# --------------------------------------------------------------------------- #
# bias builder: bit-exact
# --------------------------------------------------------------------------- #
def _rand_kinds(rng, B, T):
    kind = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        kind[b, rng.random(T) < 0.1] = wl.PAD
        for blk in (1, 2):
            lo = int(rng.integers(0, T))
            kind[b, lo:lo + int(rng.integers(1, max(2, T // 4)))] = blk
    return torch.from_numpy(kind)


@pytest.mark.parametrize("bias_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,S_q,W", [(64, 16, 8), (1001, 33, 100), (4096, 1, 1024),
                                     (777, 200, 0), (40, 40, 1000)])
def test_bias_bit_exact(bias_dtype, T, S_q, W):
    announce(f"bias dtype={bias_dtype} T={T} S_q={S_q} W={W}")
    rng = wl.rng_for(300 + T + S_q)
    B = 3
    nonpad = torch.from_numpy(rng.integers(0, T, size=B, endpoint=True).astype(np.int64))
    kind = _rand_kinds(rng, B, T)
    q_start = torch.from_numpy(rng.integers(-5, T, size=B).astype(np.int64))
    for qs in (q_start, None):
        for kd in (kind, None):
            ref = oracle.bias(nonpad, qs, kd, S_q, T, W)
            got = ab.build_static_cache_bias(dev(nonpad), dev(qs), dev(kd), S_q, T, W,
                                             dtype=bias_dtype)
            g = got.cpu().to(torch.float32)
            r = torch.from_numpy(ref).to(torch.float32)
            assert torch.equal(g.view(torch.int32), r.view(torch.int32)), (qs is None, kd is None)


# --------------------------------------------------------------------------- #
# the fused preparation (K scatter + V scatter + bias, one launch): bit-exact
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("dtype,bias_dtype", [(torch.bfloat16, torch.bfloat16),
                                              (torch.float32, torch.float32),
                                              (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("B,H,T,D,S_new,S_q,W", [(4, 3, 37, 64, 9, 9, 8),      # ragged, off the end
                                                (8, 8, 4096, 256, 1, 1, 1024), # decode_sliding-like
                                                (2, 4, 300, 512, 0, 1, 0),     # KV-shared: bias only
                                                (2, 2, 520, 128, 130, 130, 64)])
def test_fused_prepare_bit_exact(dtype, bias_dtype, B, H, T, D, S_new, S_q, W):
    announce(f"fused prepare dtype={dtype} bias={bias_dtype} B={B} H={H} T={T} D={D} "
             f"S_new={S_new} S_q={S_q} W={W}")
    rng = wl.rng_for(400 + T + D + S_new)
    kc, vc = wl.garbage(rng, (B, H, T, D), dtype), wl.garbage(rng, (B, H, T, D), dtype)
    ku, vu = wl.garbage(rng, (B, H, S_new, D), dtype), wl.garbage(rng, (B, H, S_new, D), dtype)
    w = torch.from_numpy(rng.integers(-2, T, size=B).astype(np.int64))   # some off either end
    nonpad = torch.from_numpy(rng.integers(0, T, size=B, endpoint=True).astype(np.int64))
    kind = _rand_kinds(rng, B, T)
    ibits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    for with_bias in (True, False):
        k_d, v_d = dev(kc), dev(vc)
        bias = torch.empty((B, 1, S_q, T), dtype=bias_dtype, device="cuda") if with_bias else None
        ab.kv_scatter_and_bias(k_d, v_d, dev(ku), dev(vu), dev(w), dev(nonpad), None, dev(kind),
                               S_q, W, bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(k_d.cpu().view(ibits), oracle.scatter(kc, ku, w).view(ibits))
        assert torch.equal(v_d.cpu().view(ibits), oracle.scatter(vc, vu, w).view(ibits))
        if with_bias:
            ref = torch.from_numpy(oracle.bias(nonpad, None, kind, S_q, T, W)).to(torch.float32)
            assert torch.equal(bias.cpu().to(torch.float32).view(torch.int32), ref.view(torch.int32))


# --------------------------------------------------------------------------- #
# attention: small shapes, every element
# --------------------------------------------------------------------------- #
SMALL = {
    "decode_sliding": lambda: wl.decode_sliding(B=3, Hq=4, Hkv=2, D=256, max_seq=1001,
                                                window=100, nonpad_lo=50),
    "decode_full": lambda: wl.decode_full(B=3, Hq=8, Hkv=2, D=512, max_seq=777, nonpad_lo=1),
    "decode_full_kvshared": lambda: wl.decode_full(B=3, Hq=8, Hkv=2, D=512, max_seq=777,
                                                   nonpad_lo=1, kv_shared=True),
    "decode_d64_g8": lambda: wl.decode_sliding(B=2, Hq=16, Hkv=2, D=64, max_seq=300,
                                               window=0, nonpad_lo=1),
    "decode_d128_g1": lambda: wl.decode_full(B=2, Hq=4, Hkv=4, D=128, max_seq=512, nonpad_lo=1),
    "decode_g3": lambda: wl.decode_full(B=2, Hq=6, Hkv=2, D=256, max_seq=200, nonpad_lo=1),
    # 256 (b, kv head) pairs: one split per row, written without the merge
    "decode_b64": lambda: wl.decode_full(B=64, Hq=8, Hkv=4, D=128, max_seq=300, nonpad_lo=1),
    # 16 rows per KV head: the largest row block of the decode kernel
    "decode_g16": lambda: wl.decode_sliding(B=2, Hq=32, Hkv=2, D=128, max_seq=400, window=0,
                                            nonpad_lo=1),
    "prefill_vision": lambda: wl.prefill_vision(B=2, Hq=4, Hkv=2, D=256, S_q=100, max_seq=512,
                                                window=64, start_hi=300, block=40),
    # max_seq 300: bf16 bias rows not 16-byte multiples (register-staged kernel
    # for the bias, direct-to-LDS for the rules); 320: direct-to-LDS for both
    "prefill_long": lambda: wl.prefill_long(B=2, Hq=8, Hkv=2, D=512, S_q=200, max_seq=300,
                                            pad_hi=30, block=50),
    "prefill_long_a": lambda: wl.prefill_long(B=2, Hq=8, Hkv=2, D=512, S_q=200, max_seq=320,
                                              pad_hi=30, block=50),
    "prefill_d64_g8": lambda: wl.prefill_vision(B=1, Hq=8, Hkv=1, D=64, S_q=70, max_seq=200,
                                                window=30, start_hi=100, block=20),
    "prefill_d128_g3": lambda: wl.prefill_long(B=2, Hq=6, Hkv=2, D=128, S_q=90, max_seq=130,
                                               pad_hi=20, block=30),
}


@pytest.mark.parametrize("variant", ["bias", "rules"])
@pytest.mark.parametrize("name", list(SMALL))
def test_attention_small(name, variant):
    w = SMALL[name]()
    step = w.steps[0]
    announce(f"attention small {name} variant={variant} {w.describe()}")
    _, _, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache)
    _, out = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), rules=(variant == "rules"))
    check_parity(to_f64(out), ref, w.dtype, dead_rows(bias_ref, step.nonpad, w.Hq),
                 f"{name}/{variant}")


@pytest.mark.parametrize("variant", ["bias", "rules"])
@pytest.mark.parametrize("name", ["decode_sliding", "decode_full", "decode_d64_g8", "prefill_vision",
                                  "prefill_long", "prefill_d64_g8", "prefill_d128_g3"])
@pytest.mark.parametrize("cap", [0.5, 20.0])
def test_attention_softcap(name, variant, cap):
    """softcap * tanh(scale * q.k / softcap) before the bias (skill page,
    section 4), every kernel path: decode, direct-to-LDS prefill (D 64/256/512),
    register-staged prefill (unaligned max_seq)."""
    w = SMALL[name]()
    step = w.steps[0]
    announce(f"softcap={cap} {name} variant={variant} {w.describe()}")
    _, _, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache, softcap=cap)
    _, out = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), rules=(variant == "rules"), softcap=cap)
    check_parity(to_f64(out), ref, w.dtype, dead_rows(bias_ref, step.nonpad, w.Hq),
                 f"softcap{cap}/{name}/{variant}")


def test_softcap_fp32_and_masked_poison():
    """fp32 path with softcap, and the ordering property: a small cap with a -inf
    bias entry and huge V at that key leaves the output as without the key."""
    w = wl.tiny_fp32()
    step = w.steps[0]
    cap = 0.3
    announce("softcap fp32 tiny")
    _, _, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache, softcap=cap)
    k_d, v_d = dev(w.k_cache), dev(w.v_cache)
    _, out = gpu_step(w, step, k_d, v_d, softcap=cap)
    check_parity(to_f64(out), ref, w.dtype, dead_rows(bias_ref, step.nonpad, w.Hq), "softcap/fp32")
    # bf16 decode: mask one valid key of every row with -inf, poison its V
    rng = wl.rng_for(610)
    B, Hq, Hkv, T, D = 2, 8, 2, 96, 256
    q = wl.normal(rng, (B, Hq, 1, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.tensor([T, 70], dtype=torch.int64)
    bias = torch.zeros((B, 1, 1, T), dtype=torch.bfloat16)
    bias[:, 0, 0, 10] = float("-inf")
    v_poison = v.clone()
    v_poison[:, :, 10] = 1e30
    got = fwd(dev(q), dev(k), dev(v_poison), dev(bias), dev(nonpad), 0.0625, softcap=cap)
    ref2 = oracle.attention(q, k, v, bias, nonpad, 0.0625, softcap=cap)
    check_parity(to_f64(got), ref2, torch.bfloat16, what="softcap/poison")


def test_attention_rules_equal_bias_bitwise():
    # shapes where both variants take the same kernel (prefill_long at
    # max_seq 300 does not: see SMALL)
    for name in ("decode_sliding", "decode_full", "prefill_vision", "prefill_long_a"):
        w = SMALL[name]()
        step = w.steps[0]
        announce(f"rules == bias {name}")
        _, o_bias = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), rules=False)
        _, o_rules = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), rules=True)
        assert torch.equal(o_bias.view(torch.int16), o_rules.view(torch.int16)), name


@pytest.mark.parametrize("D", [64, 256, 512])
@pytest.mark.parametrize("bias_dtype", [torch.bfloat16, torch.float32])
def test_prefill_live_tile_map(D, bias_dtype):
    """The live-tile map built by a pass over the bias (used when the caller's
    workspace holds it) and each workgroup's own bias scan (no workspace) give
    bit-identical outputs, on a bias whose -inf blocks leave dead 32-key tiles
    at arbitrary places; both match the oracle."""
    rng = wl.rng_for(620 + D)
    B, Hq, Hkv, S_q, T = 2, 8, 2, 100, 512
    q = wl.normal(rng, (B, Hq, S_q, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.tensor([T, 300], dtype=torch.int64)
    # -inf over random (8-row, 32-key) blocks, plus scattered single entries
    dead_blk = torch.from_numpy(rng.random((B, (S_q + 7) // 8, T // 32)) < 0.45)
    mask = dead_blk.repeat_interleave(8, dim=1)[:, :S_q].repeat_interleave(32, dim=2)
    mask |= torch.from_numpy(rng.random((B, S_q, T)) < 0.05)
    bias = torch.where(mask, float("-inf"), 0.25 * torch.from_numpy(rng.standard_normal((B, S_q, T))))
    bias = bias.to(bias_dtype).reshape(B, 1, S_q, T)
    announce(f"live-tile map D={D} bias={bias_dtype}")
    ref = oracle.attention(q, k, v, bias, nonpad, 1.0 / math.sqrt(D))
    args = (dev(q), dev(k), dev(v), dev(bias), dev(nonpad), 1.0 / math.sqrt(D))
    assert ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, T, D) > 0
    o_map = fwd(*args)
    o_scan = fwd(*args, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert torch.equal(o_map.view(torch.int16), o_scan.view(torch.int16))
    check_parity(to_f64(o_map), ref, torch.bfloat16,
                 dead_rows(bias.float().numpy(), nonpad, Hq), f"tilemap/D{D}")


@pytest.mark.parametrize("variant", ["bias", "rules"])
@pytest.mark.parametrize("D,Hq,Hkv", [(512, 4, 1), (256, 8, 2)])
def test_decode_uneven_rows(D, Hq, Hkv, variant):
    """Decode with batch rows of very different live length (an empty row, a
    one-key row, full rows): the split workgroups share the rows' work in
    proportion to their live keys, and ranks past the last split do nothing."""
    rng = wl.rng_for(640 + D)
    B, T = 6, 1024
    q = wl.normal(rng, (B, Hq, 1, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.tensor([0, 1, T, 37, T - 5, 300], dtype=torch.int64)
    q_start = (nonpad - 1).clamp(min=0)
    bias = torch.from_numpy(oracle.bias(nonpad, q_start, None, 1, T, 0)).to(torch.bfloat16)
    announce(f"decode uneven rows D={D} Hq={Hq} Hkv={Hkv} {variant}")
    ref = oracle.attention(q, k, v, bias, nonpad, 1.0 / math.sqrt(D))
    if variant == "bias":
        got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), 1.0 / math.sqrt(D))
    else:
        got = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), 1.0 / math.sqrt(D),
                                   q_start=dev(q_start), window=0)
    check_parity(to_f64(got), ref, torch.bfloat16,
                 dead_rows(bias.float().numpy(), nonpad, Hq), f"uneven/{variant}")


def test_shared_workspace_counts():
    """One zero-filled workspace serves decode calls of two shapes and a
    prefill call with a live-tile map in between: every decode result matches
    the oracle, and the decode arrival counts (the first 64 KiB) are zero
    again after every call, ready for the next."""
    rng = wl.rng_for(700)
    ws = torch.zeros(4 << 20, dtype=torch.uint8, device="cuda")

    def decode(B, Hq, Hkv, T, D, seed):
        r = wl.rng_for(seed)
        q = wl.normal(r, (B, Hq, 1, D), torch.bfloat16)
        k = wl.normal(r, (B, Hkv, T, D), torch.bfloat16)
        v = wl.normal(r, (B, Hkv, T, D), torch.bfloat16)
        nonpad = torch.from_numpy(r.integers(1, T, size=B, endpoint=True).astype(np.int64))
        q_start = nonpad - 1
        bias = torch.from_numpy(oracle.bias(nonpad, q_start, None, 1, T, 128)).to(torch.bfloat16)
        assert ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, 1, T, D) <= ws.numel()
        got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), 1.0 / math.sqrt(D),
                                   workspace=ws)
        ref = oracle.attention(q, k, v, bias, nonpad, 1.0 / math.sqrt(D))
        check_parity(to_f64(got), ref, torch.bfloat16, dead_rows(bias.float().numpy(), nonpad, Hq),
                     f"shared ws decode B={B} Hkv={Hkv} D={D}")

    def counts_zero():
        torch.cuda.synchronize()
        assert int(ws[:65536].view(torch.int32).abs().sum()) == 0

    announce("shared workspace: decode, prefill with map, decode")
    for rep in range(3):
        decode(8, 16, 8, 700, 256, 701 + rep)
        counts_zero()
    # prefill with a live-tile map in the same workspace
    B, Hq, Hkv, S_q, T, D = 2, 8, 2, 96, 320, 128
    q = wl.normal(rng, (B, Hq, S_q, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.tensor([T, 200], dtype=torch.int64)
    q_start = (nonpad - S_q).clamp(min=0)
    bias = torch.from_numpy(oracle.bias(nonpad, q_start, None, S_q, T, 64)).to(torch.bfloat16)
    assert ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, T, D) > 65536
    got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), 1.0 / math.sqrt(D), workspace=ws)
    ref = oracle.attention(q, k, v, bias, nonpad, 1.0 / math.sqrt(D))
    check_parity(to_f64(got), ref, torch.bfloat16, dead_rows(bias.float().numpy(), nonpad, Hq), "shared ws prefill")
    counts_zero()
    for rep in range(2):
        decode(5, 8, 2, 1000, 512, 711 + rep)
        counts_zero()


@pytest.mark.parametrize("variant", ["bias", "rules"])
@pytest.mark.parametrize("D,Dv,S_q,dtype", [
    (256, 512, 1, torch.bfloat16),    # decode on the matrix cores
    (512, 256, 1, torch.bfloat16),
    (512, 256, 2, torch.bfloat16),    # two query tokens per step
    (64, 512, 1, torch.bfloat16),     # decode, a pair without matrix-core kernels
    (256, 512, 40, torch.bfloat16),   # prefill chunk (bias rows of 600 bytes: bias on the vector path)
    (64, 128, 9, torch.float32),      # fp32 path
])
def test_value_head_size(D, Dv, S_q, dtype, variant):
    """V with another head size than Q and K (head_size != v_head_size): the
    scores use D, the output has V's Dv columns."""
    rng = wl.rng_for(660 + D + Dv + S_q)
    B, Hq, Hkv, T = 3, 8, 2, 300
    q = wl.normal(rng, (B, Hq, S_q, D), dtype)
    k = wl.normal(rng, (B, Hkv, T, D), dtype)
    v = wl.normal(rng, (B, Hkv, T, Dv), dtype)
    nonpad = torch.tensor([T, 77, 150], dtype=torch.int64)
    q_start = (nonpad - S_q).clamp(min=0)
    kind = torch.zeros((B, T), dtype=torch.int32)
    kind[1, :5] = -1                                   # pads
    kind[2, 100:130] = 1                               # an image block
    window = 64
    bias = torch.from_numpy(oracle.bias(nonpad, q_start, kind, S_q, T, window)).to(
        torch.float32 if dtype == torch.float32 else torch.bfloat16)
    announce(f"value head size D={D} Dv={Dv} S_q={S_q} {dtype} {variant}")
    scale = 1.0 / math.sqrt(D)
    ref = oracle.attention(q, k, v, bias, nonpad, scale)
    if variant == "bias":
        got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), scale)
    else:
        got = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), scale,
                                   q_start=dev(q_start), slot_kind=dev(kind), window=window)
    assert got.shape == (B, Hq, S_q, Dv)
    check_parity(to_f64(got), ref, dtype, dead_rows(bias.float().numpy(), nonpad, Hq), f"Dv/{variant}")


@pytest.mark.parametrize("variant,cap", [("bf16", 0.0), ("f32", 0.0), ("rules", 0.0), ("rules", 20.0),
                                         ("bf16", 20.0)])
@pytest.mark.parametrize("D,Dv", [(256, 512), (512, 256)])
def test_value_head_size_prefill_mfma(D, Dv, variant, cap):
    """Prefill with V's own head size on the direct-to-LDS matrix-core kernel
    (64-row workgroups here: 16 query tokens of the 4 heads of a KV head): ten
    query tiles (the last ragged), eleven key tiles (the last partial), a batch
    row whose nonpad ends inside a tile, pads, an image block, and the
    live-tile map of the bias variant (the workspace holds it)."""
    rng = wl.rng_for(680 + D + Dv + int(cap))
    B, Hq, Hkv, T, S_q = 3, 8, 2, 344, 150
    q = wl.normal(rng, (B, Hq, S_q, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, Dv), torch.bfloat16)
    nonpad = torch.tensor([T, 201, 150], dtype=torch.int64)
    q_start = (nonpad - S_q).clamp(min=0)
    kind = torch.zeros((B, T), dtype=torch.int32)
    kind[1, :7] = -1
    kind[2, 40:90] = 1
    window = 96
    bias = torch.from_numpy(oracle.bias(nonpad, q_start, kind, S_q, T, window)).to(
        torch.float32 if variant == "f32" else torch.bfloat16)
    assert ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, T, D, Dv) > 65536   # the map fits
    announce(f"value head size prefill D={D} Dv={Dv} {variant} cap={cap}")
    scale = 1.0 / math.sqrt(D)
    ref = oracle.attention(q, k, v, bias, nonpad, scale, softcap=cap)
    if variant == "rules":
        got = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), scale, q_start=dev(q_start),
                                   slot_kind=dev(kind), window=window, softcap=cap)
    else:
        got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), scale, softcap=cap)
    assert got.shape == (B, Hq, S_q, Dv)
    check_parity(to_f64(got), ref, torch.bfloat16, dead_rows(bias.float().numpy(), nonpad, Hq),
                 f"Dv prefill/{variant}/cap{cap}")


@pytest.mark.parametrize("D,Dv", [(256, 512), (512, 256)])
def test_value_head_size_prefill_shapes(D, Dv):
    """The same kernel (64-row workgroups) over group sizes and tile counts:
    G = 2 with a chunk just above the decode limit (one query tile, two key
    tiles), G = 16 (4 tokens per query tile, eighteen tiles), G = 2 with
    32-token tiles (ten, the last ragged) over 32 key tiles; bias and rules
    variants each."""
    for idx, (Hq, Hkv, S_q, T, npv) in enumerate([(16, 8, 9, 64, [64, 41]),
                                                   (32, 2, 70, 520, [520, 333]),
                                                   (4, 2, 300, 1024, [1000, 300])]):
        rng = wl.rng_for(700 + idx + D // 64)
        B = len(npv)
        q = wl.normal(rng, (B, Hq, S_q, D), torch.bfloat16)
        k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
        v = wl.normal(rng, (B, Hkv, T, Dv), torch.bfloat16)
        nonpad = torch.tensor(npv, dtype=torch.int64)
        q_start = (nonpad - S_q).clamp(min=0)
        kind = torch.zeros((B, T), dtype=torch.int32)
        kind[1, :3] = -1
        window = 0 if idx == 1 else 48
        bias = torch.from_numpy(oracle.bias(nonpad, q_start, kind, S_q, T, window)).to(torch.bfloat16)
        scale = 1.0 / math.sqrt(D)
        ref = oracle.attention(q, k, v, bias, nonpad, scale)
        dead = dead_rows(bias.float().numpy(), nonpad, Hq)
        announce(f"value head size prefill shapes D={D} Dv={Dv} Hq={Hq} Hkv={Hkv} S_q={S_q} T={T}")
        got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), scale)
        check_parity(to_f64(got), ref, torch.bfloat16, dead, f"Dv shapes/bias/{idx}")
        got = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), scale, q_start=dev(q_start),
                                   slot_kind=dev(kind), window=window)
        check_parity(to_f64(got), ref, torch.bfloat16, dead, f"Dv shapes/rules/{idx}")


def test_attention_fp32_bias_dtype():
    w = SMALL["prefill_vision"]()
    step = w.steps[0]
    announce("prefill with an fp32 bias tensor")
    _, _, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache)
    _, out = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), bias_dtype=torch.float32)
    check_parity(to_f64(out), ref, w.dtype, dead_rows(bias_ref, step.nonpad, w.Hq), "fp32-bias")


def test_tiny_fp32_prefill_then_decode():
    """Prefill S_q=16 at slots 0..15, then decode at 16 (nonpad 17), fp32."""
    w = wl.tiny_fp32()
    k_d, v_d = dev(w.k_cache), dev(w.v_cache)
    k_h, v_h = w.k_cache, w.v_cache
    for i, step in enumerate(w.steps):
        for variant in ("bias", "rules"):
            announce(f"tiny fp32 step {i} {variant}")
            k_run, v_run = k_d.clone(), v_d.clone()
            _, out = gpu_step(w, step, k_run, v_run, rules=(variant == "rules"))
            k_ref, v_ref, bias_ref, ref = oracle_step(w, step, k_h, v_h)
            assert torch.equal(k_run.cpu(), k_ref) and torch.equal(v_run.cpu(), v_ref)
            check_parity(to_f64(out), ref, torch.float32,
                         dead_rows(bias_ref, step.nonpad, w.Hq), f"tiny/{i}/{variant}")
        k_d, v_d, k_h, v_h = k_run, v_run, k_ref, v_ref


# --------------------------------------------------------------------------- #
# edge cases
# --------------------------------------------------------------------------- #
def test_empty_batch_and_negative_offset():
    """nonpad = 0 for one batch row (zero output), nonpad < S_q for another."""
    w = wl.prefill_vision(B=3, Hq=4, Hkv=2, D=256, S_q=64, max_seq=256, window=32,
                          start_hi=100, block=16)
    step = w.steps[0]
    # slots below the new nonpad all hold finite data (earlier context or the chunk)
    step.nonpad = torch.tensor([0, 20, int(step.nonpad[2])], dtype=torch.int64)
    for dq in (True, False):
        announce(f"empty batch / nonpad < S_q default_q_start={dq}")
        _, _, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache, default_q_start=dq)
        for rules in (False, True):
            _, out = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), rules=rules,
                              default_q_start=dq)
            got = to_f64(out)
            assert np.all(got[0] == 0.0)
            check_parity(got, ref, w.dtype, dead_rows(bias_ref, step.nonpad, w.Hq),
                         f"edge/dq={dq}/rules={rules}")


def test_decode_empty_and_single_key():
    # every slot valid (nonpad drawn = max_seq), then nonpad overridden
    w = wl.decode_full(B=4, Hq=8, Hkv=2, D=512, max_seq=256, nonpad_lo=256, kv_shared=True)
    step = w.steps[0]
    step.nonpad = torch.tensor([0, 1, 2, 256], dtype=torch.int64)
    step.q_start = (step.nonpad - 1).clamp(min=0)
    announce("decode nonpad in {0,1,2,max}")
    _, _, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache)
    _, out = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache))
    got = to_f64(out)
    assert np.all(got[0] == 0.0)
    check_parity(got, ref, w.dtype, dead_rows(bias_ref, step.nonpad, w.Hq), "decode-edge")


@pytest.mark.parametrize("variant", ["bias", "rules"])
def test_decode_many_rows_vector_path(variant):
    """Decode with more (batch row, kv head) pairs than the split kernel's
    arrival counts cover (B * Hkv > 16384): the vector kernel serves it, with
    no workspace."""
    rng = wl.rng_for(720)
    B, Hq, Hkv, T, D = 1100, 32, 16, 40, 64
    assert ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, 1, T, D) == 0
    q = wl.normal(rng, (B, Hq, 1, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.from_numpy(rng.integers(0, T, size=B, endpoint=True).astype(np.int64))
    q_start = (nonpad - 1).clamp(min=0)
    bias = torch.from_numpy(oracle.bias(nonpad, q_start, None, 1, T, 16)).to(torch.bfloat16)
    announce(f"decode B*Hkv={B * Hkv} {variant}")
    if variant == "bias":
        got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), 0.125)
    else:
        got = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), 0.125, q_start=dev(q_start),
                                   window=16)
    ref = oracle.attention(q, k, v, bias, nonpad, 0.125)
    check_parity(to_f64(got), ref, torch.bfloat16, dead_rows(bias.float().numpy(), nonpad, Hq),
                 f"many rows/{variant}")


@pytest.mark.parametrize("B,Hq,Hkv,D,T,S_q,causal", [
    (3, 8, 2, 256, 300, 1, True),      # decode: bottom-right = every valid key
    (2, 8, 2, 128, 200, 40, True),     # prefill chunk, some rows with nonpad < S_q
    (2, 4, 2, 256, 512, 100, True),
    (2, 8, 2, 512, 256, 33, True),
    (3, 8, 2, 256, 300, 1, False),     # is_causal=0: every valid key
    (2, 4, 2, 128, 200, 40, False)])
def test_maskless_static_cache(B, Hq, Hkv, D, T, S_q, causal):
    """Maskless Attention over the external cache (no bias tensor): is_causal=1
    is the in-kernel-rules call with no window, no slot kinds and the default
    query offset (bottom-right from nonpad); is_causal=0 passes q_start =
    max_seq so that every valid slot precedes every query."""
    announce(f"maskless causal={causal} B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} S_q={S_q}")
    rng = wl.rng_for(500 + T + S_q + D)
    dt = torch.bfloat16
    q = wl.normal(rng, (B, Hq, S_q, D), dt)
    k = wl.normal(rng, (B, Hkv, T, D), dt)
    v = wl.normal(rng, (B, Hkv, T, D), dt)
    nonpad = torch.from_numpy(rng.integers(max(1, S_q // 2), T, size=B, endpoint=True).astype(np.int64))
    nonpad[0] = min(int(nonpad[0]), S_q - 1) if S_q > 1 else nonpad[0]   # an offset clamped at 0
    qs = None if causal else torch.full((B,), T, dtype=torch.int64)
    scale = 1.0 / math.sqrt(D)
    ws_bytes = ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, T, D)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
    out = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), scale, q_start=dev(qs),
                               slot_kind=None, window=0, workspace=ws)
    bias = oracle.bias(nonpad, qs, None, S_q, T, 0)
    ref = oracle.attention(q, k, v, bias, nonpad, scale)
    check_parity(to_f64(out.cpu()), ref, dt, dead_rows(bias, nonpad, Hq), what="maskless")


@pytest.mark.parametrize("S_q", [1, 3, 40])
def test_random_finite_bias(S_q):
    """A caller-supplied float bias with arbitrary finite values and -inf holes."""
    rng = wl.rng_for(400 + S_q)
    B, Hq, Hkv, T, D = 2, 8, 2, 333, 256
    q = wl.normal(rng, (B, Hq, S_q, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.tensor([T, 200], dtype=torch.int64)
    k[1, :, 200:] = wl.garbage(rng, (Hkv, T - 200, D), torch.bfloat16)
    v[1, :, 200:] = wl.garbage(rng, (Hkv, T - 200, D), torch.bfloat16)
    bias = (3.0 * wl.normal(rng, (B, 1, S_q, T), torch.float32)).to(torch.bfloat16)
    bias[torch.from_numpy(rng.random((B, 1, S_q, T)) < 0.5)] = float("-inf")
    bias[0, 0, 0, :] = float("-inf")          # one fully-masked row
    announce(f"random finite bias S_q={S_q}")
    ref = oracle.attention(q, k, v, bias, nonpad, 1 / math.sqrt(D))
    out = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), 1 / math.sqrt(D))
    bias64 = bias.to(torch.float64).numpy()
    check_parity(to_f64(out), ref, torch.bfloat16, dead_rows(bias64, nonpad, Hq), f"randbias/{S_q}")


@pytest.mark.parametrize("name", ["decode_sliding", "prefill_long"])
def test_poison_at_masked_slots(name):
    """Huge finite K/V at slots below nonpad that the bias masks for every row
    (pads, out-of-window) change nothing: their weight is exactly 0."""
    w = SMALL[name]()
    step = w.steps[0]
    announce(f"poison masked slots {name}")
    k_h, v_h, bias_ref, _ = oracle_step(w, step, w.k_cache, w.v_cache)
    step2 = wl.Step(step.q, None, None, None, step.nonpad, step.q_start, step.slot_kind)
    _, base = gpu_step(w, step2, dev(k_h), dev(v_h))
    masked_all = (bias_ref[:, 0] == float("-inf")).all(axis=1)      # [B, T]
    k2, v2 = k_h.clone(), v_h.clone()
    for b in range(w.B):
        idx = torch.from_numpy(np.nonzero(masked_all[b])[0])
        idx = idx[idx < int(step.nonpad[b])]
        k2[b][:, idx] = 1.0e30
        v2[b][:, idx] = -1.0e30
    _, out = gpu_step(w, step2, dev(k2), dev(v2))
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


def test_determinism():
    for name in ("decode_full", "prefill_vision"):
        w = SMALL[name]()
        step = w.steps[0]
        announce(f"determinism {name}")
        _, a = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache))
        _, b = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache))
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("variant", ["bias", "rules"])
def test_graph_replay_decode_and_prefill(variant):
    """Calls captured in a HIP graph (a decode step with its in-kernel merge of
    the splits and a prefill with its live-tile map, sharing one workspace)
    replay bit-identically to the eager calls, several times, with eager work
    and synchronisations between the replays; the decode arrival counts are
    zero after every replay."""
    dec = wl.decode_sliding(B=4, Hq=16, Hkv=8, D=256, max_seq=1024, window=256)
    pre = SMALL["prefill_vision"]()
    ws = poisoned_workspace(8 << 20)
    jobs = []
    for w in (dec, pre):
        st = w.steps[0]
        k, v = dev(w.k_cache), dev(w.v_cache)
        if st.k_new is not None:
            ab.kv_tensor_scatter(k, dev(st.k_new), dev(st.write_indices))
            ab.kv_tensor_scatter(v, dev(st.v_new), dev(st.write_indices))
        q, npd, qs = dev(st.q), dev(st.nonpad), dev(st.q_start)
        kind = None if st.slot_kind is None else dev(st.slot_kind)
        bias = ab.build_static_cache_bias(npd, qs, kind, st.S_q, w.max_seq, w.window, dtype=w.dtype)
        out = poisoned((w.B, w.Hq, st.S_q, w.Dv), w.dtype)
        jobs.append((w, q, k, v, bias, npd, qs, kind, out))

    def run_all():
        for w, q, k, v, bias, npd, qs, kind, out in jobs:
            if variant == "bias":
                ab.attn_bias_gqa_fwd(q, k, v, bias, npd, w.scale, out=out, workspace=ws)
            else:
                ab.attn_bias_gqa_fwd(q, k, v, None, npd, w.scale, q_start=qs, slot_kind=kind,
                                     window=w.window, out=out, workspace=ws)

    announce(f"graph replay decode + prefill {variant}")
    run_all()
    torch.cuda.synchronize()
    eager = [j[-1].clone() for j in jobs]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        run_all()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            run_all()
    torch.cuda.synchronize()
    for rep in range(4):
        for j in jobs:
            poison_(j[-1])
        g.replay()
        torch.cuda.synchronize()
        for j, ref in zip(jobs, eager):
            assert torch.equal(j[-1].view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
        run_all()   # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("S_q,T,D,W", [
    (1, 70000, 64, 3000),     # decode over a cache longer than the prefill fast path's limit
    (24, 65536, 128, 3000),   # prefill at the direct-to-LDS path's longest cache (64 map words)
    (40, 65536, 512, 0),      # the same on the 32-row kernel, no window: all 2048 tiles live
    (24, 70000, 128, 3000),   # prefill past it: the register-staged kernel
])
def test_long_cache(S_q, T, D, W):
    """The longest caches each path takes, every slot valid, a bias (a window or none)."""
    rng = wl.rng_for(730 + S_q + T)
    B, Hq, Hkv = 1, 4, 2
    q = wl.normal(rng, (B, Hq, S_q, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.tensor([T], dtype=torch.int64)
    q_start = nonpad - S_q
    bias = torch.from_numpy(oracle.bias(nonpad, q_start, None, S_q, T, W)).to(torch.bfloat16)
    announce(f"long cache S_q={S_q} T={T} D={D} W={W}")
    scale = 1.0 / math.sqrt(D)
    got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), scale)
    ref = oracle.attention(q, k, v, bias, nonpad, scale)
    check_parity(to_f64(got), ref, torch.bfloat16, dead_rows(bias.float().numpy(), nonpad, Hq), f"long/{T}")
    got_r = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), scale, q_start=dev(q_start), window=W)
    check_parity(to_f64(got_r), ref, torch.bfloat16, dead_rows(bias.float().numpy(), nonpad, Hq), f"long/{T}/rules")


def test_prefill_cache_too_long_raises():
    """A prefill whose live-tile list does not fit beside two K/V stages in LDS
    is refused with a clear error, before any kernel runs."""
    B, Hq, Hkv, S_q, T, D = 1, 4, 2, 32, 600000, 512
    q = torch.empty((B, Hq, S_q, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((B, Hkv, T, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((B, Hkv, T, D), dtype=torch.bfloat16, device="cuda")
    nonpad = torch.tensor([T], dtype=torch.int64, device="cuda")
    with pytest.raises(RuntimeError, match="max_seq too large"):
        ab.attn_bias_gqa_fwd(q, k, v, None, nonpad, 0.05)


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 16, 64])
def test_decode_split_sweep(splits, monkeypatch):
    """Decode with a forced split count (ABGQA_DECODE_SPLITS, read at every
    call): one split per row (the direct write), a few, and more splits than a
    short row has 16-key blocks (splits without keys merge as empty); rows of
    very different live length; both variants; poisoned workspace and output."""
    monkeypatch.setenv("ABGQA_DECODE_SPLITS", str(splits))
    rng = wl.rng_for(750)
    B, Hq, Hkv, T, D = 5, 8, 2, 900, 256
    q = wl.normal(rng, (B, Hq, 1, D), torch.bfloat16)
    k = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    v = wl.normal(rng, (B, Hkv, T, D), torch.bfloat16)
    nonpad = torch.tensor([T, 1, 333, 0, 40], dtype=torch.int64)
    q_start = (nonpad - 1).clamp(min=0)
    bias = torch.from_numpy(oracle.bias(nonpad, q_start, None, 1, T, 300)).to(torch.bfloat16)
    ref = oracle.attention(q, k, v, bias, nonpad, 1.0 / math.sqrt(D))
    dead = dead_rows(bias.float().numpy(), nonpad, Hq)
    announce(f"decode split sweep splits={splits}")
    got = fwd(dev(q), dev(k), dev(v), dev(bias), dev(nonpad), 1.0 / math.sqrt(D))
    check_parity(to_f64(got), ref, torch.bfloat16, dead, f"splits{splits}/bias")
    got_r = fwd(dev(q), dev(k), dev(v), None, dev(nonpad), 1.0 / math.sqrt(D), q_start=dev(q_start),
                window=300)
    check_parity(to_f64(got_r), ref, torch.bfloat16, dead, f"splits{splits}/rules")


def test_check_mode(monkeypatch):
    """ABGQA_CHECK=1: device-side index values are validated before anything is
    enqueued (the kernels never see the bad values), decode arrival counts of
    the workspace must be zero, and valid calls still give the oracle's result."""
    monkeypatch.setenv("ABGQA_CHECK", "1")
    rng = wl.rng_for(760)
    B, Hq, Hkv, T, D = 2, 8, 2, 128, 256
    q = dev(wl.normal(rng, (B, Hq, 1, D), torch.bfloat16))
    k = dev(wl.normal(rng, (B, Hkv, T, D), torch.bfloat16))
    v = dev(wl.normal(rng, (B, Hkv, T, D), torch.bfloat16))
    announce("check mode: bad device values refused")
    with pytest.raises(RuntimeError, match="ABGQA_CHECK: nonpad_kv_seqlen\\[1\\] = 129"):
        fwd(q, k, v, None, dev(torch.tensor([5, T + 1])), 0.1)
    with pytest.raises(RuntimeError, match="ABGQA_CHECK: nonpad_kv_seqlen\\[0\\] = -1"):
        ab.build_static_cache_bias(dev(torch.tensor([-1, 3])), None, None, 1, T, 0)
    with pytest.raises(RuntimeError, match="ABGQA_CHECK: q_start\\[0\\] = -3"):
        fwd(q, k, v, None, dev(torch.tensor([5, 9])), 0.1, q_start=dev(torch.tensor([-3, 2])))
    upd = dev(wl.normal(rng, (B, Hkv, 4, D), torch.bfloat16))
    with pytest.raises(RuntimeError, match="ABGQA_CHECK: write_indices\\[1\\] = 125"):
        ab.kv_tensor_scatter(k, upd, dev(torch.tensor([0, 125])))
    with pytest.raises(RuntimeError, match="ABGQA_CHECK: write_indices\\[0\\] = -1"):
        ab.kv_scatter_and_bias(k, v, upd, upd, dev(torch.tensor([-1, 0])), dev(torch.tensor([3, 4])),
                               None, None, 4, 0, bias=torch.empty((B, 1, 4, T), dtype=torch.bfloat16,
                                                                   device="cuda"))
    need = ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, 1, T, D)
    ws = poisoned_workspace(need)
    ws[0:4] = torch.tensor([7, 0, 0, 0], dtype=torch.uint8)    # arrival count 0 left at 7
    with pytest.raises(RuntimeError, match="ABGQA_CHECK: decode arrival count 0"):
        fwd(q, k, v, None, dev(torch.tensor([5, 9])), 0.1, workspace=ws)
    # a good scatter and decode under the check, against the oracle
    announce("check mode: valid calls")
    nonpad = torch.tensor([70, T], dtype=torch.int64)
    k_h, v_h = k.cpu(), v.cpu()
    ab.kv_tensor_scatter(k, upd, dev(torch.tensor([60, T - 4])))
    k_h = oracle.scatter(k_h, upd.cpu(), torch.tensor([60, T - 4]))
    assert torch.equal(k.cpu().view(torch.int16), k_h.view(torch.int16))
    q_start = nonpad - 1
    bias = ab.build_static_cache_bias(dev(nonpad), dev(q_start), None, 1, T, 50)
    got = fwd(q, k, v, bias, dev(nonpad), 0.1)
    b_ref = oracle.bias(nonpad, q_start, None, 1, T, 50)
    ref = oracle.attention(q.cpu(), k_h, v_h, b_ref, nonpad, 0.1)
    check_parity(to_f64(got), ref, torch.bfloat16, dead_rows(b_ref, nonpad, Hq), "check mode")


def test_invalid_arguments_raise():
    q = torch.zeros((1, 3, 1, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 64, 256), dtype=torch.bfloat16, device="cuda")
    n = torch.tensor([10], dtype=torch.int64, device="cuda")
    with pytest.raises(RuntimeError, match="multiple of Hkv"):
        ab.attn_bias_gqa_fwd(q, k, k, None, n, 0.1)
    q = torch.zeros((1, 4, 1, 96), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="D and D_v must be"):
        ab.attn_bias_gqa_fwd(q, k, k, None, n, 0.1)


# --------------------------------------------------------------------------- #
# circular (window-sized) cache: position p in slot p mod capacity
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 256, 512])
def test_circular_scatter_bit_exact(dtype, D):
    announce(f"circular scatter dtype={dtype} D={D}")
    rng = wl.rng_for(800 + D)
    B, H, C, S_new = 5, 3, 37, 9
    cache = wl.garbage(rng, (B, H, C, D), dtype)
    upd = wl.garbage(rng, (B, H, S_new, D), dtype)
    w = torch.tensor([0, 30, 3 * C + 2, -4, C - S_new], dtype=torch.int64)   # wrap, laps, negative
    ref = oracle.scatter_circular(cache, upd, w)
    c = dev(cache)
    ab.kv_tensor_scatter_circular(c, dev(upd), dev(w))
    ibits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(c.cpu().view(ibits), ref.view(ibits))
    with pytest.raises(RuntimeError, match="at most capacity"):
        ab.kv_tensor_scatter_circular(c, dev(wl.garbage(rng, (B, H, C + 1, D), dtype)), dev(w))


@pytest.mark.parametrize("bias_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("C,S_q,W", [(64, 16, 8), (1001, 33, 100), (1024, 1, 1024), (256, 200, 0),
                                     (40, 40, 1000)])
def test_circular_bias_bit_exact(bias_dtype, C, S_q, W):
    announce(f"circular bias dtype={bias_dtype} C={C} S_q={S_q} W={W}")
    rng = wl.rng_for(820 + C + S_q)
    B = 4
    L = torch.from_numpy(rng.integers(0, 3 * C, size=B, endpoint=True).astype(np.int64))
    L[0] = C // 2                                                    # not wrapped
    kind = _rand_kinds(rng, B, C)
    q_start = torch.from_numpy(np.maximum(L.numpy() - S_q - rng.integers(-3, 5, size=B), 0))
    for qs in (q_start, None):
        for kd in (kind, None):
            ref = oracle.bias_circular(L, qs, kd, S_q, C, W)
            got = ab.build_circular_cache_bias(dev(L), dev(qs), dev(kd), S_q, C, W, dtype=bias_dtype,
                                               out=poisoned((B, 1, S_q, C), bias_dtype))
            g = got.cpu().to(torch.float32)
            r = torch.from_numpy(ref).to(torch.float32)
            assert torch.equal(g.view(torch.int32), r.view(torch.int32)), (qs is None, kd is None)


def test_circular_fused_prepare_bit_exact():
    rng = wl.rng_for(840)
    B, H, C, D, S_new, W = 4, 2, 520, 128, 130, 64
    announce("circular fused prepare")
    kc, vc = wl.garbage(rng, (B, H, C, D), torch.bfloat16), wl.garbage(rng, (B, H, C, D), torch.bfloat16)
    ku, vu = wl.garbage(rng, (B, H, S_new, D), torch.bfloat16), wl.garbage(rng, (B, H, S_new, D), torch.bfloat16)
    pos = torch.tensor([0, 450, 1900, 7], dtype=torch.int64)
    L = pos + S_new
    kind = _rand_kinds(rng, B, C)
    k_d, v_d = dev(kc), dev(vc)
    bias = poisoned((B, 1, S_new, C), torch.bfloat16)
    ab.kv_scatter_and_bias_circular(k_d, v_d, dev(ku), dev(vu), dev(pos), dev(L), None, dev(kind), S_new,
                                    W, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(k_d.cpu().view(torch.int16), oracle.scatter_circular(kc, ku, pos).view(torch.int16))
    assert torch.equal(v_d.cpu().view(torch.int16), oracle.scatter_circular(vc, vu, pos).view(torch.int16))
    ref = torch.from_numpy(oracle.bias_circular(L, None, kind, S_new, C, W)).to(torch.float32)
    assert torch.equal(bias.cpu().to(torch.float32).view(torch.int32), ref.view(torch.int32))


CIRCULAR = {
    # window < capacity, the cache wrapped several times or not yet
    "decode_d256_w": lambda: wl.decode_sliding_circular(B=5, Hq=8, Hkv=4, D=256, capacity=300, window=200,
                                                        len_lo=1, len_hi=1000),
    # window = capacity (every held token allowed)
    "decode_d512": lambda: wl.decode_sliding_circular(B=4, Hq=16, Hkv=4, D=512, capacity=256, window=256,
                                                      len_lo=100, len_hi=900),
    # direct-to-LDS prefill (D 256 key split, D 512 32-row, D 128), chunks that wrap
    "prefill_d256": lambda: wl.prefill_vision_circular(B=3, Hq=8, Hkv=4, D=256, S_q=100, capacity=352,
                                                       window=200, start_hi=900, block=40),
    "prefill_d512": lambda: wl.prefill_vision_circular(B=2, Hq=8, Hkv=2, D=512, S_q=130, capacity=320,
                                                       window=150, start_hi=700, block=50),
    "prefill_d128": lambda: wl.prefill_vision_circular(B=2, Hq=6, Hkv=2, D=128, S_q=90, capacity=200,
                                                       window=90, start_hi=500, block=30),
    # capacity whose bf16 bias rows are not 16-byte chunks: the register-staged kernel
    "prefill_d256_ragged": lambda: wl.prefill_vision_circular(B=2, Hq=8, Hkv=4, D=256, S_q=70, capacity=201,
                                                              window=100, start_hi=600, block=20),
    "prefill_fp32": lambda: wl.prefill_vision_circular(B=2, Hq=4, Hkv=2, D=64, S_q=20, capacity=48,
                                                       window=16, start_hi=100, block=8,
                                                       dtype=torch.float32),
}


@pytest.mark.parametrize("variant", ["bias", "rules"])
@pytest.mark.parametrize("name", list(CIRCULAR))
def test_circular_attention(name, variant):
    """Attention over a circular cache (scatter of the step's tokens, the
    circular bias or the circular rules in the kernel) against the oracle's
    circular path, every element, every kernel path."""
    w = CIRCULAR[name]()
    step = w.steps[0]
    announce(f"circular attention {name} variant={variant} {w.describe()}")
    k_h, v_h, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache)
    k_d, v_d = dev(w.k_cache), dev(w.v_cache)
    bias, out = gpu_step(w, step, k_d, v_d, rules=(variant == "rules"))
    torch.cuda.synchronize()
    ibits = torch.int16 if w.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(k_d.cpu().view(ibits), k_h.view(ibits))
    if bias is not None:
        g = bias.cpu().to(torch.float32).view(torch.int32)
        assert torch.equal(g, torch.from_numpy(bias_ref).to(torch.float32).view(torch.int32))
    check_parity(to_f64(out), ref, w.dtype, dead_rows(bias_ref, step.nonpad, w.Hq), f"circular/{name}/{variant}")


def test_circular_rules_equal_bias_bitwise():
    for name in ("decode_d256_w", "prefill_d256", "prefill_d512"):
        w = CIRCULAR[name]()
        step = w.steps[0]
        announce(f"circular rules == bias {name}")
        _, o_bias = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), rules=False)
        _, o_rules = gpu_step(w, step, dev(w.k_cache), dev(w.v_cache), rules=True)
        assert torch.equal(o_bias.view(torch.int16), o_rules.view(torch.int16)), name


# --------------------------------------------------------------------------- #
# the five full-size workloads
# --------------------------------------------------------------------------- #
# rows compared: "all", or one row per workgroup of a prefill kernel whose
# workgroups hold `n` query tokens of the G heads of one KV head (plus every
# query head's first and last row)
FULL = {
    "decode_sliding": (lambda: wl.decode_sliding(), "all"),
    "decode_full": (lambda: wl.decode_full(), "all"),
    "decode_full_kvshared": (lambda: wl.decode_full(kv_shared=True), "all"),
    "prefill_vision": (lambda: wl.prefill_vision(), "all"),
    # 128-row workgroups of 32 tokens (G = 4)
    "prefill_long": (lambda: wl.prefill_long(), 32),
    # V of another head size: the 16-row kernel at the vision chunk's grid
    # (128 workgroups of 128 rows would not fill the CUs), the 32-row one with
    # O^T in the accumulation registers at the long prefill's grid and at the
    # vision chunk's with twice the batch (256 workgroups of 128 rows)
    "prefill_vision_dv512": (lambda: wl.prefill_vision(Dv=512), "all"),
    "prefill_vision_b4_dv512": (lambda: wl.prefill_vision(B=4, Dv=512), "all"),
    "prefill_long_dv256": (lambda: wl.prefill_long(Dv=256), 32),
    # the circular (window-sized) cache: the sliding decode layer with 1024
    # slots, the vision chunk with 1536 (window + chunk)
    "decode_sliding_circular": (lambda: wl.decode_sliding_circular(), "all"),
    "prefill_vision_circular": (lambda: wl.prefill_vision_circular(), "all"),
    # decode batches that do not divide the 256 CUs: 96 (b, kv head) pairs x 5
    # splits (480 workgroups, two to a CU), 320 pairs x 1 split (more
    # workgroups than CUs), and the full layer's 96 pairs x 5 splits (two
    # rounds of one workgroup per CU)
    "decode_sliding_b12": (lambda: wl.decode_sliding(B=12), "all"),
    "decode_sliding_b40": (lambda: wl.decode_sliding(B=40), "all"),
    "decode_full_b24": (lambda: wl.decode_full(B=24), "all"),
}


_full_cache = {}


def _full_reference(name):
    """Inputs, compared rows and oracle results of one full-size workload
    (shared by the bias and rules variants)."""
    if name not in _full_cache:
        _full_cache.clear()
        make, which = FULL[name]
        w = make()
        step = w.steps[0]
        n_all = w.B * w.Hq * step.S_q
        # every row, one batch entry at a time in the oracle (its fp64 copies
        # of the repeated KV heads stay one entry's worth)
        rows = np.arange(n_all, dtype=np.int64) if which == "all" else tile_rows(w, step, which, seed=500)
        announce(f"oracle for {name} rows={len(rows)} of {n_all}")
        k_h, v_h, bias_ref, ref = oracle_step(w, step, w.k_cache, w.v_cache, rows=rows)
        _full_cache[name] = (w, rows, k_h, v_h, bias_ref, ref)
    return _full_cache[name]


@pytest.mark.parametrize("variant", ["bias", "rules"])
@pytest.mark.parametrize("name", list(FULL))
def test_attention_full_size(name, variant):
    w, rows, k_h, v_h, bias_ref, ref = _full_reference(name)
    step = w.steps[0]
    announce(f"attention full {name} variant={variant} rows={len(rows)} {w.describe()}")
    k_d, v_d = dev(w.k_cache), dev(w.v_cache)
    bias, out = gpu_step(w, step, k_d, v_d, rules=(variant == "rules"))
    torch.cuda.synchronize()
    if step.k_new is not None:   # the scatter landed bit-exactly (a circular cache's too)
        assert torch.equal(k_d.cpu().view(torch.int16), k_h.view(torch.int16))
        assert torch.equal(v_d.cpu().view(torch.int16), v_h.view(torch.int16))
    if bias is not None:         # and so did the bias
        g = bias.cpu().to(torch.float32).view(torch.int32)
        assert torch.equal(g, torch.from_numpy(bias_ref).to(torch.float32).view(torch.int32))
    del k_d, v_d, bias
    got_all = to_f64(out).reshape(-1, w.Dv)
    # every element of the output was written (poisoned before the call), also
    # in the rows the oracle does not compute
    assert np.isfinite(got_all).all(), f"{name}/{variant}: unwritten or non-finite output"
    dead = dead_rows(bias_ref, step.nonpad, w.Hq).reshape(-1)[rows]
    check_parity(got_all[rows], ref.reshape(-1, w.Dv), w.dtype, np.repeat(dead[:, None], w.Dv, axis=1),
                 f"full/{name}/{variant}")

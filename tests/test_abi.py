"""The C-ABI library, host side only (no GPU): it loads, exports every entry
point include/abgqa.h declares, and rejects bad arguments with a stable status
and message before anything reaches the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import additive_bias_gqa_amd as ab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "abgqa.h")
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    return ab.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"kv_tensor_scatter", "build_static_cache_bias", "attn_bias_gqa_fwd",
                          "attn_bias_gqa_workspace_bytes", "abgqa_last_error"}
    out = subprocess.run(["nm", "-D", "--defined-only", ab.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def _fwd(lib, **kw):
    a = dict(out=None, q=None, k=None, v=None, bias=None, bdt=1, nonpad=None, qs=None, kind=None,
             B=1, Hq=4, Hkv=2, S_q=1, T=64, D=64, Dv=64, scale=0.125, softcap=0.0, window=0, dtype=1,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.attn_bias_gqa_fwd(a["out"], a["q"], a["k"], a["v"], a["bias"], a["bdt"],
                                 a["nonpad"], a["qs"], a["kind"], a["B"], a["Hq"], a["Hkv"],
                                 a["S_q"], a["T"], a["D"], a["Dv"], a["scale"], a["softcap"], a["window"],
                                 a["dtype"],
                                 a["ws"], a["wsb"], a["stream"])


FAKE = 1 << 20  # a 256-byte aligned address that is never dereferenced


@pytest.mark.parametrize("kw,status,msg", [
    (dict(B=0), INVALID, "must be positive"),
    (dict(Hq=6, Hkv=4), INVALID, "multiple of Hkv"),
    (dict(S_q=65), INVALID, "must not exceed max_seq"),
    (dict(D=96), UNSUPPORTED, "D and D_v must be"),
    (dict(Dv=80), UNSUPPORTED, "D and D_v must be"),
    (dict(Dv=0), INVALID, "must be positive"),
    (dict(softcap=-1.0), INVALID, "softcap"),
    (dict(softcap=float("inf")), INVALID, "softcap"),
    (dict(softcap=float("nan")), INVALID, "softcap"),
    (dict(dtype=7), UNSUPPORTED, "dtype"),
    (dict(out=FAKE, q=FAKE + 4096, k=FAKE + 8192, v=FAKE + 12288), INVALID, "null"),
    (dict(out=FAKE + 8, q=FAKE + 4096, k=FAKE + 8192, v=FAKE + 12288, nonpad=FAKE), INVALID,
     "misaligned"),
    (dict(out=FAKE, q=FAKE, k=FAKE + 8192, v=FAKE + 12288, nonpad=FAKE + 16384), INVALID, "alias"),
    (dict(out=FAKE, q=FAKE + 4096, k=FAKE + 8192, v=FAKE + 12288, nonpad=FAKE + 16384), WORKSPACE,
     "workspace"),
])
def test_attn_validation(lib, kw, status, msg):
    assert _fwd(lib, **kw) == status
    assert msg in ab.abgqa_last_error()


def test_scatter_and_bias_validation(lib):
    assert lib.kv_tensor_scatter(None, None, None, 1, 1, 8, 0, 64, 1, None) == OK  # S_new = 0
    assert lib.kv_tensor_scatter(None, None, None, 1, 1, 8, 2, 64, 1, None) == INVALID
    assert lib.kv_tensor_scatter(FAKE, FAKE, None, 1, 1, 8, 2, 12, 1, None) == UNSUPPORTED
    assert "multiple of 16 bytes" in ab.abgqa_last_error()
    assert lib.kv_tensor_scatter(FAKE, FAKE, None, 1, 1, 8, -1, 64, 1, None) == INVALID
    assert lib.build_static_cache_bias(None, 1, FAKE, None, None, 1, 1, 8, 0, None) == INVALID
    assert lib.build_static_cache_bias(FAKE, 5, FAKE, None, None, 1, 1, 8, 0, None) == UNSUPPORTED
    assert lib.build_static_cache_bias(FAKE + 2, 1, FAKE, None, None, 1, 1, 8, 0, None) == INVALID
    assert "misaligned" in ab.abgqa_last_error()


def test_workspace_size(lib):
    CNT = 64 * 1024   # decode arrival counts at the start of every workspace
    r256 = lib.attn_bias_gqa_workspace_bytes(8, 16, 8, 1, 4096, 256, 256)
    # 64 (b, kv head) pairs x 4 splits, records of 2 rows x 256 + m, l (16-byte padded)
    assert r256 == CNT + 8 * 8 * 4 * ((2 * 256 + 4 + 3) // 4 * 4) * 4
    # decode partial records hold the V head size
    assert lib.attn_bias_gqa_workspace_bytes(8, 16, 8, 1, 4096, 256, 512) > r256
    assert lib.attn_bias_gqa_workspace_bytes(8, 16, 8, 1, 4096, 64, 512) == 0   # vector path
    # prefill (D 256, G 2: 64-row workgroups of 32 tokens): one bit per batch
    # row x 16 query tiles x 128 key tiles
    assert lib.attn_bias_gqa_workspace_bytes(2, 16, 8, 512, 4096, 256, 256) == CNT + 2 * 16 * 4 * 4
    # a V head size of its own (256 beside 512): 64-row workgroups of 32 tokens
    # while 128-row ones would number fewer than 256 (here 2 x 8 x 8)...
    assert lib.attn_bias_gqa_workspace_bytes(2, 16, 8, 512, 4096, 256, 512) == CNT + 2 * 16 * 4 * 4
    assert lib.attn_bias_gqa_workspace_bytes(2, 16, 8, 512, 4096, 512, 256) == CNT + 2 * 16 * 4 * 4
    # ... and 128-row workgroups (G 4: 32 tokens) beyond: 4 x 4 x 64 of them
    assert lib.attn_bias_gqa_workspace_bytes(4, 16, 4, 2048, 8192, 512, 256) == CNT + 4 * 64 * 8 * 4
    assert lib.attn_bias_gqa_workspace_bytes(2, 16, 8, 512, 4096, 128, 512) == 0   # vector path
    assert lib.attn_bias_gqa_workspace_bytes(2, 8, 8, 512, 4096, 256, 256) == 0    # G = 1: no map
    assert lib.attn_bias_gqa_workspace_bytes(1, 6, 4, 1, 64, 64, 64) == 0         # invalid heads
    # more (b, kv head) pairs than the counts cover: the vector path, no workspace
    assert lib.attn_bias_gqa_workspace_bytes(2049, 16, 8, 1, 64, 64, 64) == 0
    assert lib.attn_bias_gqa_workspace_bytes(2048, 16, 8, 1, 64, 64, 64) > CNT


def test_fused_prepare_validation(lib):
    f = lib.kv_scatter_and_bias
    # nothing to do: no new tokens, no bias
    assert f(None, None, None, None, None, 1, 1, 8, 0, 64, 1, None, 1, None, None, None, 1, 0, None) == OK
    # new tokens but null caches / updates
    assert f(None, None, None, None, None, 1, 1, 8, 2, 64, 1, None, 1, None, None, None, 1, 0, None) == INVALID
    assert "null cache or update" in ab.abgqa_last_error()
    # rows that are not a multiple of 16 bytes
    assert f(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 8, 2, 12, 1, None, 1, None, None, None, 1, 0, None) == UNSUPPORTED
    # misaligned V update
    assert f(FAKE, FAKE + 4096, FAKE + 8192, FAKE + 8200, None, 1, 1, 8, 2, 64, 1, None, 1, None, None,
             None, 1, 0, None) == INVALID
    assert "misaligned" in ab.abgqa_last_error()
    # a bias without nonpad, with a bad dtype, with S_q = 0
    assert f(None, None, None, None, None, 1, 1, 8, 0, 64, 1, FAKE, 1, None, None, None, 1, 0, None) == INVALID
    assert "nonpad" in ab.abgqa_last_error()
    assert f(None, None, None, None, None, 1, 1, 8, 0, 64, 1, FAKE, 4, FAKE, None, None, 1, 0, None) == UNSUPPORTED
    assert f(None, None, None, None, None, 1, 1, 8, 0, 64, 1, FAKE, 1, FAKE, None, None, 0, 0, None) == INVALID
    assert f(None, None, None, None, None, 0, 1, 8, 0, 64, 1, None, 1, None, None, None, 1, 0, None) == INVALID


def test_prefill_tile_index_limit(lib):
    """Live key tiles of a prefill are numbered in 16 bits: a cache of more than
    65535 tiles of 32 keys is refused before any launch (D = 64 leaves room in
    LDS for such a tile list, so the size of the list alone would not refuse it)."""
    T = 32 * 65537
    args = dict(out=FAKE, q=FAKE + 4096, k=FAKE + 8192, v=FAKE + 12288, nonpad=FAKE + 16384,
                B=1, Hq=4, Hkv=2, S_q=32, T=T, D=64, Dv=64)
    assert _fwd(lib, **args) == UNSUPPORTED
    assert "max_seq too large for the prefill tile list" in ab.abgqa_last_error()
    args.update(T=32 * 65536)
    assert _fwd(lib, **args) == UNSUPPORTED


def test_workspace_per_stream():
    """The binding's default workspace is one per (device, stream): two streams
    never share one, a stream reuses its own, a buffer that grows leaves the
    old one alive (a captured graph may still hold its address), and growth
    during graph capture is refused."""
    import torch
    ab._workspaces.clear()
    alloc = lambda n: torch.zeros(n, dtype=torch.uint8)
    a = ab._workspace_for((0, 111), 1000, False, alloc)
    b = ab._workspace_for((0, 222), 1000, False, alloc)
    assert a.data_ptr() != b.data_ptr()
    assert ab._workspace_for((0, 111), 800, False, alloc) is a
    assert ab._workspace_for((0, 111), 1000, True, alloc) is a      # no growth: fine under capture
    big = ab._workspace_for((0, 111), 5000, False, alloc)
    assert big.numel() >= 5000 and big is not a
    assert any(t is a for t in ab._workspaces[(0, 111)])           # the old buffer is kept
    assert ab._workspace_for((1, 111), 100, False, alloc) is not a  # another device
    with pytest.raises(RuntimeError, match="during graph capture"):
        ab._workspace_for((0, 222), 4000, True, alloc)
    ab._workspaces.clear()


def test_noalloc_refuses_large_scratch(lib):
    """The entry point that allocates nothing holds 8 MiB of scratch per GPU:
    a shape that needs more is refused with a clear message before any HIP
    call (16384 (batch row, kv head) pairs of 2-row decode records at D = 512)."""
    need = lib.attn_bias_gqa_workspace_bytes(2048, 16, 8, 1, 64, 512, 512)
    assert need > 8 << 20
    st = lib.attn_bias_gqa_fwd_noalloc(FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, None, 1,
                                       FAKE + 16384, None, None, 2048, 16, 8, 1, 64, 512, 512,
                                       0.05, 0.0, 0, 1, None)
    assert st == WORKSPACE
    msg = ab.abgqa_last_error()
    assert "needs %d bytes of scratch" % need in msg and "holds 8388608" in msg


def _step(lib, circular=False, **kw):
    a = dict(out=None, q=None, k=None, v=None, ku=None, vu=None, wi=None, S_new=1, bias=None, bdt=1,
             nonpad=None, qs=None, kind=None, B=1, Hq=4, Hkv=2, S_q=1, T=64, D=64, Dv=64, scale=0.125,
             softcap=0.0, window=0, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    f = lib.attn_bias_gqa_decode_step_circular if circular else lib.attn_bias_gqa_decode_step
    return f(a["out"], a["q"], a["k"], a["v"], a["ku"], a["vu"], a["wi"], a["S_new"], a["bias"], a["bdt"],
             a["nonpad"], a["qs"], a["kind"], a["B"], a["Hq"], a["Hkv"], a["S_q"], a["T"], a["D"], a["Dv"],
             a["scale"], a["softcap"], a["window"], a["dtype"], a["ws"], a["wsb"], a["stream"])


PTRS = dict(out=FAKE, q=FAKE + 4096, k=FAKE + 8192, v=FAKE + 12288, ku=FAKE + 16384, vu=FAKE + 20480,
            nonpad=FAKE + 24576)


@pytest.mark.parametrize("kw,circular,status,msg", [
    (dict(B=0), False, INVALID, "must be positive"),
    (dict(S_new=-1), False, INVALID, "S_new must be >= 0"),
    (dict(S_new=65), True, INVALID, "at most capacity"),
    (dict(S_new=17), False, UNSUPPORTED, "fused step takes bf16 decode shapes"),
    (dict(dtype=0), False, UNSUPPORTED, "fused step takes bf16 decode shapes"),   # fp32
    (dict(S_q=16, Hq=4, Hkv=2), False, UNSUPPORTED, "fused step"),                 # 32 rows: prefill
    (dict(D=96), False, UNSUPPORTED, "fused step"),
    (dict(B=8193, Hkv=2, Hq=4), False, UNSUPPORTED, "fused step"),                 # > 16384 pairs
    (dict(softcap=-1.0), False, INVALID, "softcap"),
    (dict(), False, INVALID, "null out"),
    (dict(PTRS, ku=None), False, INVALID, "null update"),
    (dict(PTRS, vu=FAKE + 20488), False, INVALID, "misaligned"),
    (dict(PTRS, wi=FAKE + 28676), False, INVALID, "misaligned"),
    (dict(PTRS, out=FAKE + 16384), False, INVALID, "alias"),
    (dict(PTRS, bias=FAKE + 4096), False, INVALID, "alias"),
    (dict(PTRS, bias=FAKE + 32768, bdt=5), False, UNSUPPORTED, "bias dtype"),
    (dict(PTRS), False, WORKSPACE, "workspace"),
    (dict(PTRS, S_new=0, ku=None, vu=None), True, WORKSPACE, "workspace"),
])
def test_decode_step_validation(lib, kw, circular, status, msg):
    assert _step(lib, circular, **kw) == status
    assert msg in ab.abgqa_last_error()


def test_decode_split_count(lib, monkeypatch):
    """The decode grid's split count, read off the workspace size (one record
    per (kv head, batch row, split)): among the counts that keep B * Hkv *
    n_split within two rounds of 256 workgroups (at most max_seq / 64 and 64),
    the one whose rounds are fullest, ties to fewer splits."""
    monkeypatch.delenv("ABGQA_DECODE_SPLITS", raising=False)
    CNT = 64 * 1024

    def splits(B, Hq, Hkv, T, D):
        G = Hq // Hkv
        nr = 1
        while nr < G:
            nr *= 2
        rec = (nr * D + 2 * nr + 3) // 4 * 4 * 4
        got = lib.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, 1, T, D, D) - CNT
        assert got % (B * Hkv * rec) == 0
        return got // (B * Hkv * rec)

    # sliding layers (Hkv 8, head 256, 4096 slots): 64 pairs fill one round at
    # 4 splits; 96 -> 5 (480 of 512); 136 -> 3 (408 of 512); 200 and more: 1
    assert [splits(B, 16, 8, 4096, 256) for B in (8, 12, 17, 25, 40, 64)] == [4, 5, 3, 1, 1, 1]
    # full-attention layers (Hkv 4, head 512, 8192 slots): 48 pairs -> 5
    # (240 of 256), 64 -> 4, 96 -> 5, 160 -> 3
    assert [splits(B, 16, 4, 8192, 512) for B in (12, 16, 24, 40)] == [5, 4, 5, 3]
    # few pairs: capped at 64 splits and at one split per 64 slots
    assert splits(1, 8, 8, 4096, 128) == 32
    assert splits(1, 2, 1, 8192, 128) == 64
    assert splits(1, 2, 1, 300, 128) == 5
    # the override is read at every call
    monkeypatch.setenv("ABGQA_DECODE_SPLITS", "7")
    assert splits(8, 16, 8, 4096, 256) == 7

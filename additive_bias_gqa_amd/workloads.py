"""Seeded synthetic inputs for additive-bias GQA attention over a static KV cache.

This module holds random draws and input layout only (shapes, value
distributions, which cache slots hold valid data or garbage, slot kinds for
padding and image blocks). It holds none of the method's arithmetic, so the
same host tensors can feed both the fp64 oracle and the HIP path.

Every workload draws from ``numpy.random.Generator(PCG64(1000 + index))`` in the
fixed order written in each builder. Values are drawn as float32 and rounded to
bf16 with torch's round-to-nearest-even cast. "Garbage" slots hold uniformly
random bit patterns (NaN and Inf included) and stand for stale cache contents
beyond ``nonpad_kv_seqlen``.

The default sizes are the five workload shapes of the method's statement:
  tiny_fp32        B1 Hq4 Hkv2 D64 max_seq64, fp32: prefill 16 then decode 1
  decode_sliding   B8 Hq16 Hkv8 D256 max_seq4096, window 1024 (S_q = 1)
  decode_full      B16 Hq16 Hkv4 D512 max_seq8192, no window (S_q = 1),
                   optionally KV-shared (no scatter, borrowed cache)
  prefill_vision   B2 Hq16 Hkv8 D256 S_q512 max_seq4096, window 1024,
                   two 256-token image blocks inside the chunk
  prefill_long     B4 Hq16 Hkv4 D512 S_q2048 max_seq8192, left padding,
                   one 256-token image block per row
and two layers over a circular (window-sized) cache, where the token of
absolute position p sits in slot p mod capacity:
  decode_sliding_circular   the sliding decode layer with 1024 slots
  prefill_vision_circular   the vision chunk with 1536 slots (window + chunk)
Smaller sizes are used by the parity tests through the same builders.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

SEED_BASE = 1000
PAD = -1  # slot kind of a padding token; 0 = text, k > 0 = image block k


def rng_for(index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(SEED_BASE + index))


def normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """N(0,1) draws (float32), cast to ``dtype`` with round-to-nearest-even."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def garbage(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """Uniformly random bit patterns of ``dtype`` (may be NaN, Inf, denormal)."""
    if dtype == torch.bfloat16:
        bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    if dtype == torch.float32:
        bits = rng.integers(0, 1 << 32, size=shape, dtype=np.uint32)
        return torch.from_numpy(bits.view(np.int32)).view(torch.float32)
    raise ValueError(f"unsupported dtype {dtype}")


@dataclasses.dataclass
class Step:
    """One pass of the hot path: scatter K/V (unless KV-shared), bias, attention."""
    q: torch.Tensor                        # [B, Hq, S_q, D]
    k_new: Optional[torch.Tensor]          # [B, Hkv, S_new, D]; None = no scatter
    v_new: Optional[torch.Tensor]
    write_indices: Optional[torch.Tensor]  # int64 [B]
    nonpad: torch.Tensor                   # int64 [B]
    q_start: torch.Tensor                  # int64 [B]
    slot_kind: Optional[torch.Tensor]      # int32 [B, max_seq]; None = all text

    @property
    def S_q(self) -> int:
        return int(self.q.shape[2])


@dataclasses.dataclass
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    D: int
    max_seq: int
    window: int            # <= 0: no sliding window
    scale: float
    k_cache: torch.Tensor  # [B, Hkv, max_seq, D], contents before the first step
    v_cache: torch.Tensor  # [B, Hkv, max_seq, Dv]
    steps: List[Step]
    # circular cache of capacity max_seq: write_indices are absolute positions
    # (slot = position mod capacity) and nonpad is the count of tokens written
    circular: bool = False

    @property
    def Dv(self) -> int:
        return int(self.v_cache.shape[3])

    def describe(self) -> dict:
        d = {"workload": self.name, "B": self.B, "Hq": self.Hq, "Hkv": self.Hkv,
             "D": self.D, "S_q": self.steps[-1].S_q, "max_seq": self.max_seq,
             "window": self.window, "dtype": str(self.dtype).replace("torch.", "")}
        if self.Dv != self.D:
            d["Dv"] = self.Dv
        if self.circular:
            d["cache"] = "circular"
        return d


def _fill_cache(rng, B, H, max_seq, D, n_valid, dtype) -> torch.Tensor:
    """Slots [0, n_valid[b]) ~ N(0,1); slots >= n_valid[b] garbage bits.
    Drawn batch row by batch row: normals first, then garbage."""
    cache = torch.empty((B, H, max_seq, D), dtype=dtype)
    for b in range(B):
        n = int(n_valid[b])
        if n > 0:
            cache[b, :, :n] = normal(rng, (H, n, D), dtype)
        if n < max_seq:
            cache[b, :, n:] = garbage(rng, (H, max_seq - n, D), dtype)
    return cache


def tiny_fp32(index: int = 0) -> Workload:
    """Tiny fp32 sequence: prefill S_q=16 at slots 0..15, then one decode step at
    slot 16 (nonpad 17). Caches zero-filled; causal + sliding window 8.
    Draw order: q_prefill, k_prefill, v_prefill, q_decode, k_decode, v_decode."""
    rng = rng_for(index)
    B, Hq, Hkv, D, T = 1, 4, 2, 64, 64
    dt = torch.float32
    qp = normal(rng, (B, Hq, 16, D), dt)
    kp = normal(rng, (B, Hkv, 16, D), dt)
    vp = normal(rng, (B, Hkv, 16, D), dt)
    qd = normal(rng, (B, Hq, 1, D), dt)
    kd = normal(rng, (B, Hkv, 1, D), dt)
    vd = normal(rng, (B, Hkv, 1, D), dt)
    i64 = lambda v: torch.tensor(v, dtype=torch.int64)
    steps = [
        Step(qp, kp, vp, i64([0]), i64([16]), i64([0]), None),
        Step(qd, kd, vd, i64([16]), i64([17]), i64([16]), None),
    ]
    z = torch.zeros((B, Hkv, T, D), dtype=dt)
    return Workload("tiny_fp32_prefill16_decode1", dt, B, Hq, Hkv, D, T, 8,
                    1.0 / math.sqrt(D), z, z.clone(), steps)


def _decode(name, index, B, Hq, Hkv, D, max_seq, window, nonpad_lo, kv_shared, dtype, Dv=None):
    """Decode step (S_q = 1) at slot nonpad-1 with nonpad ~ U{nonpad_lo..max_seq}.
    Scatter variant: slots < nonpad-1 valid, the new token is scattered at
    nonpad-1, slots >= nonpad-1 start as garbage. KV-shared variant: slots
    < nonpad already valid (written by the layer that owns the cache), no scatter.
    Draw order: nonpad, q, K cache, V cache, k_new, v_new (scatter variant only).
    Dv: head size of V (default D; KV-shared layers may read a V of another
    head size)."""
    Dv = D if Dv is None else Dv
    rng = rng_for(index)
    nonpad = rng.integers(nonpad_lo, max_seq, size=B, endpoint=True).astype(np.int64)
    q = normal(rng, (B, Hq, 1, D), dtype)
    n_valid = nonpad if kv_shared else nonpad - 1
    kc = _fill_cache(rng, B, Hkv, max_seq, D, n_valid, dtype)
    vc = _fill_cache(rng, B, Hkv, max_seq, Dv, n_valid, dtype)
    npt = torch.from_numpy(nonpad)
    if kv_shared:
        kn = vn = wi = None
    else:
        kn = normal(rng, (B, Hkv, 1, D), dtype)
        vn = normal(rng, (B, Hkv, 1, Dv), dtype)
        wi = npt - 1
    kind = torch.zeros((B, max_seq), dtype=torch.int32)  # causal + padding, no pads
    step = Step(q, kn, vn, wi, npt, npt - 1, kind)
    return Workload(name, dtype, B, Hq, Hkv, D, max_seq, window, 1.0 / math.sqrt(D),
                    kc, vc, [step])


def decode_sliding(index: int = 1, B=8, Hq=16, Hkv=8, D=256, max_seq=4096, window=1024,
                   nonpad_lo=512, dtype=torch.bfloat16) -> Workload:
    """Sliding-window decode layer (head_dim 256, window 1024)."""
    return _decode(f"decode_sliding_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}_T{max_seq}_W{window}",
                   index, B, Hq, Hkv, D, max_seq, window, nonpad_lo, False, dtype)


def decode_full(index: int = 2, B=16, Hq=16, Hkv=4, D=512, max_seq=8192, nonpad_lo=1024,
                kv_shared: bool = False, dtype=torch.bfloat16, Dv=None) -> Workload:
    """Full-attention decode layer (head_dim 512, no window); ``kv_shared`` reads a
    borrowed cache with nothing to scatter (kv_sequence_length = 0), whose V may
    have another head size (Dv)."""
    tag = "_kvshared" if kv_shared else ""
    vtag = "" if Dv is None or Dv == D else f"_Dv{Dv}"
    return _decode(f"decode_full_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}{vtag}_T{max_seq}{tag}",
                   index, B, Hq, Hkv, D, max_seq, 0, nonpad_lo, kv_shared, dtype, Dv)


def prefill_vision(index: int = 3, B=2, Hq=16, Hkv=8, D=256, S_q=512, max_seq=4096,
                   window=1024, start_hi=2048, block=256, n_blocks=2,
                   dtype=torch.bfloat16, Dv=None) -> Workload:
    """Prefill chunk of S_q tokens at absolute start ~ U{0..start_hi}, with
    ``n_blocks`` image blocks of ``block`` tokens at offsets ~ U{0..S_q-block}
    inside the chunk (ids 1, 2, ...; a later block overwrites an overlap).
    Slots [0, start) hold earlier context ~ N(0,1); slots >= start are garbage
    until the chunk is scattered at start; nonpad = start + S_q. Dv: head size
    of V (default D). Draw order: start, block offsets, q, K cache, V cache,
    k_new, v_new."""
    assert start_hi + S_q <= max_seq and block <= S_q
    Dv = D if Dv is None else Dv
    rng = rng_for(index)
    start = rng.integers(0, start_hi, size=B, endpoint=True).astype(np.int64)
    offs = rng.integers(0, S_q - block, size=(B, n_blocks), endpoint=True)
    q = normal(rng, (B, Hq, S_q, D), dtype)
    kc = _fill_cache(rng, B, Hkv, max_seq, D, start, dtype)
    vc = _fill_cache(rng, B, Hkv, max_seq, Dv, start, dtype)
    kn = normal(rng, (B, Hkv, S_q, D), dtype)
    vn = normal(rng, (B, Hkv, S_q, Dv), dtype)
    kind = torch.zeros((B, max_seq), dtype=torch.int32)
    for b in range(B):
        for i in range(n_blocks):
            lo = int(start[b] + offs[b, i])
            kind[b, lo:lo + block] = i + 1
    st = torch.from_numpy(start)
    step = Step(q, kn, vn, st.clone(), st + S_q, st.clone(), kind)
    vtag = "" if Dv == D else f"_Dv{Dv}"
    return Workload(f"prefill_vision_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}{vtag}_Sq{S_q}_T{max_seq}_W{window}",
                    dtype, B, Hq, Hkv, D, max_seq, window, 1.0 / math.sqrt(D), kc, vc, [step])


def prefill_long(index: int = 4, B=4, Hq=16, Hkv=4, D=512, S_q=2048, max_seq=8192,
                 pad_hi=256, block=256, dtype=torch.bfloat16, Dv=None) -> Workload:
    """Prefill of S_q tokens from slot 0 with left padding pad_b ~ U{0..pad_hi}
    (slot kind PAD, expressed through the bias) and one image block of ``block``
    tokens at an offset ~ U{pad_b..S_q-block}. nonpad = S_q, q_start = 0; the
    cache is garbage before the scatter. Dv: head size of V (default D).
    Draw order: pads, block offsets, q, K cache, V cache, k_new, v_new."""
    Dv = D if Dv is None else Dv
    assert S_q <= max_seq and pad_hi + block <= S_q
    rng = rng_for(index)
    pads = rng.integers(0, pad_hi, size=B, endpoint=True).astype(np.int64)
    offs = np.array([rng.integers(int(pads[b]), S_q - block, endpoint=True)
                     for b in range(B)], dtype=np.int64)
    q = normal(rng, (B, Hq, S_q, D), dtype)
    zero = np.zeros(B, dtype=np.int64)
    kc = _fill_cache(rng, B, Hkv, max_seq, D, zero, dtype)
    vc = _fill_cache(rng, B, Hkv, max_seq, Dv, zero, dtype)
    kn = normal(rng, (B, Hkv, S_q, D), dtype)
    vn = normal(rng, (B, Hkv, S_q, Dv), dtype)
    kind = torch.zeros((B, max_seq), dtype=torch.int32)
    for b in range(B):
        kind[b, :int(pads[b])] = PAD
        kind[b, int(offs[b]):int(offs[b]) + block] = 1
    z = torch.zeros(B, dtype=torch.int64)
    step = Step(q, kn, vn, z.clone(), torch.full((B,), S_q, dtype=torch.int64), z.clone(), kind)
    vtag = "" if Dv == D else f"_Dv{Dv}"
    return Workload(f"prefill_long_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}{vtag}_Sq{S_q}_T{max_seq}",
                    dtype, B, Hq, Hkv, D, max_seq, 0, 1.0 / math.sqrt(D), kc, vc, [step])


def _fill_circular(rng, B, H, C, D, n_written, dtype) -> torch.Tensor:
    """A circular cache of C slots after n_written[b] tokens: slots
    [0, min(n_written, C)) hold written tokens ~ N(0,1), the rest garbage bits.
    Drawn batch row by batch row: normals first, then garbage."""
    return _fill_cache(rng, B, H, C, D, np.minimum(n_written, C), dtype)


def decode_sliding_circular(index: int = 5, B=8, Hq=16, Hkv=8, D=256, capacity=1024, window=1024,
                            len_lo=512, len_hi=4096, dtype=torch.bfloat16) -> Workload:
    """Sliding-window decode over a circular cache of ``capacity`` slots (the
    window: a quarter of the static cache's 4096). L ~ U{len_lo..len_hi} tokens
    are written after the step; the L-1 earlier ones fill min(L-1, capacity)
    slots, and the new token (position L-1) is scattered at slot
    (L-1) mod capacity. Draw order: L, q, K cache, V cache, k_new, v_new."""
    rng = rng_for(index)
    L = rng.integers(len_lo, len_hi, size=B, endpoint=True).astype(np.int64)
    q = normal(rng, (B, Hq, 1, D), dtype)
    kc = _fill_circular(rng, B, Hkv, capacity, D, L - 1, dtype)
    vc = _fill_circular(rng, B, Hkv, capacity, D, L - 1, dtype)
    kn = normal(rng, (B, Hkv, 1, D), dtype)
    vn = normal(rng, (B, Hkv, 1, D), dtype)
    Lt = torch.from_numpy(L)
    kind = torch.zeros((B, capacity), dtype=torch.int32)
    step = Step(q, kn, vn, Lt - 1, Lt, Lt - 1, kind)
    return Workload(f"decode_sliding_circular_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}_C{capacity}_W{window}",
                    dtype, B, Hq, Hkv, D, capacity, window, 1.0 / math.sqrt(D), kc, vc, [step],
                    circular=True)


def prefill_vision_circular(index: int = 6, B=2, Hq=16, Hkv=8, D=256, S_q=512, capacity=1536,
                            window=1024, start_hi=2048, block=256, n_blocks=2,
                            dtype=torch.bfloat16) -> Workload:
    """The vision prefill chunk over a circular cache of ``capacity`` slots
    (window + chunk: every key a query of the chunk may see is still held). The
    chunk's S_q tokens start at absolute position start ~ U{0..start_hi}; the
    start earlier tokens fill min(start, capacity) slots; the chunk is scattered
    at slots (start + t) mod capacity; image blocks of ``block`` tokens at
    offsets ~ U{0..S_q-block} inside the chunk (ids 1, 2, ...; a later block
    overwrites an overlap) mark the slots their tokens land in. Draw order:
    start, block offsets, q, K cache, V cache, k_new, v_new."""
    assert block <= S_q <= capacity
    rng = rng_for(index)
    start = rng.integers(0, start_hi, size=B, endpoint=True).astype(np.int64)
    offs = rng.integers(0, S_q - block, size=(B, n_blocks), endpoint=True)
    q = normal(rng, (B, Hq, S_q, D), dtype)
    kc = _fill_circular(rng, B, Hkv, capacity, D, start, dtype)
    vc = _fill_circular(rng, B, Hkv, capacity, D, start, dtype)
    kn = normal(rng, (B, Hkv, S_q, D), dtype)
    vn = normal(rng, (B, Hkv, S_q, D), dtype)
    kind = torch.zeros((B, capacity), dtype=torch.int32)
    for b in range(B):
        for i in range(n_blocks):
            for t in range(int(offs[b, i]), int(offs[b, i]) + block):
                kind[b, (int(start[b]) + t) % capacity] = i + 1
    st = torch.from_numpy(start)
    step = Step(q, kn, vn, st.clone(), st + S_q, st.clone(), kind)
    return Workload(f"prefill_vision_circular_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}_Sq{S_q}_C{capacity}_W{window}",
                    dtype, B, Hq, Hkv, D, capacity, window, 1.0 / math.sqrt(D), kc, vc, [step],
                    circular=True)

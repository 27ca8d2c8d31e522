"""One pass of the hot path on the GPU (through the C-ABI binding) and the same
pass on the fp64 oracle, plus the parity comparison. The two sides share only
the seeded host inputs."""
from __future__ import annotations

import numpy as np
import torch

import additive_bias_gqa_amd as ab
import oracle
from additive_bias_gqa_amd import workloads as wl

NEG_INF = float("-inf")
# tolerances of the method's statement: fp32 max-abs 1e-5; bf16 inputs with
# fp32 accumulation max-abs 2e-2 and mean-rel 1e-2 (sum|d| / sum|ref|)
TOL = {torch.float32: dict(max_abs=1e-5, mean_rel=None),
       torch.bfloat16: dict(max_abs=2e-2, mean_rel=1e-2)}


def announce(msg: str):
    print(f"[case] {msg}", flush=True)


def dev(t):
    return None if t is None else t.to("cuda")


# Every output and scratch buffer a GPU test hands to the library starts out as
# a NaN with a distinctive payload, so a kernel that leaves an element unwritten
# (a skipped query tile, a skipped merge) fails the finiteness check of
# check_parity instead of passing on memory an earlier call filled correctly.
POISON = {torch.bfloat16: (torch.int16, 0x7FC1), torch.float32: (torch.int32, 0x7FC00001)}


def poisoned(shape, dtype):
    ibits, pattern = POISON[dtype]
    return torch.empty(shape, dtype=dtype, device="cuda").view(ibits).fill_(pattern).view(dtype)


def poison_(t: torch.Tensor) -> torch.Tensor:
    ibits, pattern = POISON[t.dtype]
    t.view(ibits).fill_(pattern)
    return t


def poisoned_workspace(nbytes: int):
    """Arrival counts (the first 64 KiB) zero, as the library requires; every
    byte after them 0xFF (a NaN as fp32), so a partial record or live-tile map
    word that a call reads without having written it shows."""
    if nbytes == 0:
        return None
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    ws[:min(nbytes, 65536)] = 0
    return ws


def fwd(q, k, v, bias, nonpad, scale, out=None, workspace=None, entry=None, **kw):
    """attn_bias_gqa_fwd (or `entry`, a binding of the same arguments) with a
    poisoned output and a poisoned workspace of the size the shape needs,
    unless the caller passes its own."""
    B, Hq, S_q, D = q.shape
    Hkv, T, Dv = k.shape[1], k.shape[2], v.shape[3]
    if out is None:
        out = poisoned((B, Hq, S_q, Dv), q.dtype)
    if workspace is None:
        workspace = poisoned_workspace(ab.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, T, D, Dv))
    entry = entry or ab.attn_bias_gqa_fwd
    return entry(q, k, v, bias, nonpad, scale, out=out, workspace=workspace, **kw)


def gpu_step(w: wl.Workload, step: wl.Step, k_dev, v_dev, rules: bool = False,
             bias_dtype: torch.dtype | None = None, default_q_start: bool = False,
             softcap: float = 0.0):
    """Scatter K/V (unless KV-shared), build the bias (unless rules), attention.
    Returns (bias or None, out) on the device. A circular workload takes the
    circular cache's calls."""
    circ = w.circular
    if step.k_new is not None:
        wi = dev(step.write_indices)
        scatter = ab.kv_tensor_scatter_circular if circ else ab.kv_tensor_scatter
        scatter(k_dev, dev(step.k_new), wi)
        scatter(v_dev, dev(step.v_new), wi)
    nonpad = dev(step.nonpad)
    q_start = None if default_q_start else dev(step.q_start)
    kind = dev(step.slot_kind)
    bias = None
    if not rules:
        bt = bias_dtype or w.dtype
        build = ab.build_circular_cache_bias if circ else ab.build_static_cache_bias
        bias = build(nonpad, q_start, kind, step.S_q, w.max_seq, w.window,
                     dtype=bt, out=poisoned((w.B, 1, step.S_q, w.max_seq), bt))
    out = fwd(dev(step.q), k_dev, v_dev, bias, nonpad, w.scale,
              q_start=q_start, slot_kind=kind, window=w.window, softcap=softcap,
              entry=ab.attn_bias_gqa_fwd_circular if circ else ab.attn_bias_gqa_fwd)
    return bias, out


def fused_step(w: wl.Workload, step: wl.Step, k_dev, v_dev, bias_dtype=torch.bfloat16,
               with_bias=True, softcap=0.0, default_q_start=False):
    """The step through the fused entry point (attn_bias_gqa_decode_step, or
    its circular form) with poisoned bias, output and workspace; returns (bias or
    None, out)."""
    B, Hq, S_q, D = step.q.shape
    Dv = v_dev.shape[3]
    bias = poisoned((w.B, 1, S_q, w.max_seq), bias_dtype) if with_bias else None
    out = poisoned((B, Hq, S_q, Dv), w.dtype)
    ws = poisoned_workspace(ab.attn_bias_gqa_workspace_bytes(B, Hq, w.Hkv, S_q, w.max_seq, D, Dv))
    fn = ab.attn_bias_gqa_decode_step_circular if w.circular else ab.attn_bias_gqa_decode_step
    fn(dev(step.q), k_dev, v_dev, dev(step.k_new), dev(step.v_new), dev(step.write_indices),
       dev(step.nonpad), w.scale, q_start=None if default_q_start else dev(step.q_start),
       slot_kind=dev(step.slot_kind), window=w.window, bias=bias, out=out, workspace=ws,
       softcap=softcap)
    return bias, out


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def oracle_step(w: wl.Workload, step: wl.Step, k_host, v_host, rows=None,
                default_q_start: bool = False, softcap: float = 0.0):
    """The same pass on the oracle. Returns (k_cache, v_cache, bias, out). A
    circular workload: the circular scatter and bias, and attention over the
    min(kv_len, capacity) valid slots."""
    circ = w.circular
    if step.k_new is not None:
        scatter = oracle.scatter_circular if circ else oracle.scatter
        k_host = scatter(k_host, step.k_new, step.write_indices)
        v_host = scatter(v_host, step.v_new, step.write_indices)
    qs = None if default_q_start else step.q_start
    build = oracle.bias_circular if circ else oracle.bias
    bias = build(step.nonpad, qs, step.slot_kind, step.S_q, w.max_seq, w.window)
    valid = step.nonpad.clamp(0, w.max_seq) if circ else step.nonpad
    out = oracle.attention(step.q, k_host, v_host, bias, valid, w.scale, rows=rows,
                           softcap=softcap)
    return k_host, v_host, bias, out


def dead_rows(bias: np.ndarray, nonpad, Hq: int) -> np.ndarray:
    """[B, Hq, S_q] True where a query row has no allowed key below nonpad."""
    B, _, S_q, T = bias.shape
    npd = np.asarray(nonpad, dtype=np.int64).reshape(B, 1, 1)
    live = ((bias[:, 0] != NEG_INF) & (np.arange(T)[None, None, :] < npd)).any(axis=-1)
    return np.repeat(~live[:, None, :], Hq, axis=1)


def check_parity(got: np.ndarray, ref: np.ndarray, dtype: torch.dtype, dead=None, what=""):
    """Element-wise parity at the stated tolerance; dead rows must be exact zeros."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = TOL[dtype]
    max_abs = float(err.max()) if err.size else 0.0
    mean_rel = float(err.sum() / max(np.abs(ref).sum(), 1e-300))
    print(f"[parity] {what}: max_abs={max_abs:.3e} mean_rel={mean_rel:.3e} n={err.size}", flush=True)
    assert max_abs <= tol["max_abs"], f"{what}: max_abs {max_abs:.3e} > {tol['max_abs']}"
    if tol["mean_rel"] is not None:
        assert mean_rel <= tol["mean_rel"], f"{what}: mean_rel {mean_rel:.3e} > {tol['mean_rel']}"
    if dead is not None and dead.any():
        assert np.all(got[dead] == 0.0), f"{what}: fully-masked rows are not exactly zero"
    return max_abs, mean_rel


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def tile_rows(w: wl.Workload, step: wl.Step, tokens: int, seed: int) -> np.ndarray:
    """Flat (b*Hq + h)*S_q + s row indices: one random row (a random head of the
    group, a random token of the tile) of every (batch row, KV head, tile of
    `tokens` query tokens) - one per workgroup of a prefill kernel whose
    workgroups hold `tokens` tokens of the G heads of one KV head - plus the
    first and last row of every (batch row, query head); sorted and unique."""
    B, Hq, Hkv, S_q = w.B, w.Hq, w.Hkv, step.S_q
    G = Hq // Hkv
    rng = np.random.Generator(np.random.PCG64(seed))
    picks = set()
    for b in range(B):
        for hk in range(Hkv):
            for t0 in range(0, S_q, tokens):
                h = hk * G + int(rng.integers(0, G))
                s = int(rng.integers(t0, min(t0 + tokens, S_q)))
                picks.add((b * Hq + h) * S_q + s)
        for h in range(Hq):
            picks.add((b * Hq + h) * S_q)
            picks.add((b * Hq + h) * S_q + S_q - 1)
    return np.array(sorted(picks), dtype=np.int64)

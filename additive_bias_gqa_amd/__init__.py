"""additive_bias_gqa_amd: additive-bias grouped-query attention over an external
static KV cache, for AMD Instinct MI355X (gfx950).

Thin ctypes binding over libabgqa.so (include/abgqa.h). Each function checks
device, dtype, shape and contiguity of its torch tensors, passes raw device
pointers and the current HIP stream, and raises RuntimeError with the
library's message on failure. Every step of the computation runs in the HIP
kernels; there is no fallback: a missing library raises at the first call.

    kv_tensor_scatter(cache, update, write_indices)            in place
    kv_scatter_and_bias(k_cache, v_cache, k_update, v_update, write_indices,
                        nonpad, q_start, slot_kind, S_q, window, bias=None)
                                  both scatters + the bias, one launch
    build_static_cache_bias(nonpad, q_start, slot_kind, S_q, max_seq, window,
                            dtype=torch.bfloat16, out=None)     -> bias
    attn_bias_gqa_fwd(q, k_cache, v_cache, bias, nonpad, scale, q_start=None,
                      slot_kind=None, window=0, out=None)       -> out
    attn_bias_gqa_fwd_noalloc(q, k_cache, v_cache, bias, nonpad, scale, out,
                              q_start=None, slot_kind=None, window=0)
                                  the same with the library's own scratch
    attn_bias_gqa_decode_step(q, k_cache, v_cache, k_update, v_update,
                              write_indices, nonpad, scale, ..., bias=None)
                                  a decode step (both scatters, the bias and
                                  the attention) in one launch
The same calls for a circular (window-sized) cache: kv_tensor_scatter_circular,
build_circular_cache_bias, kv_scatter_and_bias_circular and
attn_bias_gqa_fwd_circular, attn_bias_gqa_decode_step_circular (kv_len tokens
written so far, position p in slot p mod capacity).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["kv_tensor_scatter", "kv_scatter_and_bias", "build_static_cache_bias", "attn_bias_gqa_fwd",
           "attn_bias_gqa_fwd_noalloc", "attn_bias_gqa_workspace_bytes", "abgqa_last_error",
           "kv_tensor_scatter_circular", "build_circular_cache_bias", "kv_scatter_and_bias_circular",
           "attn_bias_gqa_fwd_circular", "attn_bias_gqa_decode_step",
           "attn_bias_gqa_decode_step_circular", "library_path", "load"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libabgqa.so")
_lib = None
_lock = threading.Lock()

F32, BF16 = 0, 1
_DTYPE = {torch.float32: F32, torch.bfloat16: BF16}
_c_i64p = ctypes.c_void_p


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libabgqa.so (built by additive_bias_gqa_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m additive_bias_gqa_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        for name in ("kv_tensor_scatter", "kv_tensor_scatter_circular"):
            getattr(lib, name).argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, vp]
            getattr(lib, name).restype = ctypes.c_int
        for name in ("kv_scatter_and_bias", "kv_scatter_and_bias_circular"):
            getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int,
                                           vp, ctypes.c_int, vp, vp, vp, i64, i64, vp]
            getattr(lib, name).restype = ctypes.c_int
        for name in ("build_static_cache_bias", "build_circular_cache_bias"):
            getattr(lib, name).argtypes = [vp, ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, vp]
            getattr(lib, name).restype = ctypes.c_int
        for name in ("attn_bias_gqa_fwd", "attn_bias_gqa_fwd_circular"):
            getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                           i64, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                           ctypes.c_float, i64, ctypes.c_int, vp, sz, vp]
            getattr(lib, name).restype = ctypes.c_int
        for name in ("attn_bias_gqa_decode_step", "attn_bias_gqa_decode_step_circular"):
            getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, vp, ctypes.c_int, vp, vp,
                                           vp, i64, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                           ctypes.c_float, i64, ctypes.c_int, vp, sz, vp]
            getattr(lib, name).restype = ctypes.c_int
        lib.attn_bias_gqa_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                                  i64, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                                  ctypes.c_float, i64, ctypes.c_int, vp]
        lib.attn_bias_gqa_fwd_noalloc.restype = ctypes.c_int
        lib.attn_bias_gqa_workspace_bytes.argtypes = [i64] * 7
        lib.attn_bias_gqa_workspace_bytes.restype = sz
        lib.abgqa_last_error.argtypes = []
        lib.abgqa_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def abgqa_last_error() -> str:
    return load().abgqa_last_error().decode()


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"{what} failed (status {status}): {abgqa_last_error()}")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _opt(t, name, dtype, shape=None) -> int | None:
    return None if t is None else _dev(t, name, dtype, shape)


def kv_tensor_scatter(cache: torch.Tensor, update: torch.Tensor,
                      write_indices: torch.Tensor | None) -> torch.Tensor:
    """cache[b, h, write_indices[b] + t, :] = update[b, h, t, :] (in place)."""
    return _scatter("kv_tensor_scatter", cache, update, write_indices)


def kv_tensor_scatter_circular(cache: torch.Tensor, update: torch.Tensor,
                               write_pos: torch.Tensor | None) -> torch.Tensor:
    """Circular cache of capacity C = cache.shape[2]: update token t of batch
    row b (absolute position write_pos[b] + t) goes to slot (position) mod C,
    in place; at most C tokens per call."""
    return _scatter("kv_tensor_scatter_circular", cache, update, write_pos)


def _scatter(fn: str, cache, update, write_indices):
    if cache.dim() != 4 or update.dim() != 4:
        raise ValueError("cache and update must be 4-D [B, Hkv, slots, D]")
    B, H, T, D = cache.shape
    if update.shape[0] != B or update.shape[1] != H or update.shape[3] != D:
        raise ValueError("update must be [B, Hkv, S_new, D] matching the cache")
    if cache.dtype not in _DTYPE or update.dtype != cache.dtype:
        raise ValueError("cache/update must both be float32 or bfloat16")
    c = _dev(cache, "cache")
    u = _dev(update, "update") if update.numel() else None
    w = _opt(write_indices, "write_indices", torch.int64, (B,))
    _check(getattr(load(), fn)(c, u, w, B, H, T, update.shape[2], D, _DTYPE[cache.dtype],
                               _stream(cache)), fn)
    return cache


def kv_scatter_and_bias(k_cache: torch.Tensor, v_cache: torch.Tensor,
                        k_update: torch.Tensor, v_update: torch.Tensor,
                        write_indices: torch.Tensor | None, nonpad: torch.Tensor | None,
                        q_start: torch.Tensor | None, slot_kind: torch.Tensor | None,
                        S_q: int, window: int, bias: torch.Tensor | None = None):
    """kv_tensor_scatter(k_cache, k_update, write_indices),
    kv_tensor_scatter(v_cache, v_update, write_indices) and, when `bias` is
    given, build_static_cache_bias(..., out=bias), in one launch."""
    return _prepare("kv_scatter_and_bias", k_cache, v_cache, k_update, v_update, write_indices,
                    nonpad, q_start, slot_kind, S_q, window, bias)


def kv_scatter_and_bias_circular(k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 k_update: torch.Tensor, v_update: torch.Tensor,
                                 write_pos: torch.Tensor | None, kv_len: torch.Tensor | None,
                                 q_start: torch.Tensor | None, slot_kind: torch.Tensor | None,
                                 S_q: int, window: int, bias: torch.Tensor | None = None):
    """kv_scatter_and_bias for a circular cache (kv_tensor_scatter_circular of
    K and V, build_circular_cache_bias), in one launch."""
    return _prepare("kv_scatter_and_bias_circular", k_cache, v_cache, k_update, v_update, write_pos,
                    kv_len, q_start, slot_kind, S_q, window, bias)


def _prepare(fn, k_cache, v_cache, k_update, v_update, write_indices, nonpad, q_start, slot_kind,
             S_q, window, bias):
    if k_cache.dim() != 4 or k_update.dim() != 4:
        raise ValueError("caches and updates must be 4-D [B, Hkv, slots, D]")
    B, H, T, D = k_cache.shape
    S_new = k_update.shape[2]
    for name, t in (("v_cache", v_cache),):
        if tuple(t.shape) != (B, H, T, D) or t.dtype != k_cache.dtype:
            raise ValueError(f"{name} must match k_cache")
    for name, t in (("k_update", k_update), ("v_update", v_update)):
        if tuple(t.shape) != (B, H, S_new, D) or t.dtype != k_cache.dtype:
            raise ValueError(f"{name} must be [B, Hkv, S_new, D] of the cache dtype")
    if k_cache.dtype not in _DTYPE:
        raise ValueError("caches must be float32 or bfloat16")
    kc, vc = _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache")
    ku = _dev(k_update, "k_update") if S_new else None
    vu = _dev(v_update, "v_update") if S_new else None
    w = _opt(write_indices, "write_indices", torch.int64, (B,))
    bp, bdt, npd, qs, sk = None, BF16, None, None, None
    if bias is not None:
        if bias.dtype not in _DTYPE:
            raise ValueError("bias dtype must be float32 or bfloat16")
        bp, bdt = _dev(bias, "bias", None, (B, 1, S_q, T)), _DTYPE[bias.dtype]
        npd = _dev(nonpad, "nonpad", torch.int64, (B,))
        qs = _opt(q_start, "q_start", torch.int64, (B,))
        sk = _opt(slot_kind, "slot_kind", torch.int32, (B, T))
    _check(getattr(load(), fn)(kc, vc, ku, vu, w, B, H, T, S_new, D, _DTYPE[k_cache.dtype],
                               bp, bdt, npd, qs, sk, int(S_q), int(window), _stream(k_cache)), fn)
    return bias


def build_static_cache_bias(nonpad: torch.Tensor, q_start: torch.Tensor | None,
                            slot_kind: torch.Tensor | None, S_q: int, max_seq: int,
                            window: int, dtype: torch.dtype = torch.bfloat16,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """(B, 1, S_q, max_seq) bias: +0.0 where allowed, -inf where masked."""
    return _bias("build_static_cache_bias", nonpad, q_start, slot_kind, S_q, max_seq, window, dtype, out)


def build_circular_cache_bias(kv_len: torch.Tensor, q_start: torch.Tensor | None,
                              slot_kind: torch.Tensor | None, S_q: int, capacity: int,
                              window: int, dtype: torch.dtype = torch.bfloat16,
                              out: torch.Tensor | None = None) -> torch.Tensor:
    """(B, 1, S_q, capacity) bias of a circular cache: kv_len[b] tokens written
    so far, position p in slot p mod capacity; +0.0 allowed, -inf masked."""
    return _bias("build_circular_cache_bias", kv_len, q_start, slot_kind, S_q, capacity, window, dtype,
                 out)


def _bias(fn, nonpad, q_start, slot_kind, S_q, max_seq, window, dtype, out):
    B = nonpad.shape[0]
    if out is None:
        out = torch.empty((B, 1, S_q, max_seq), dtype=dtype, device=nonpad.device)
    if out.dtype not in _DTYPE:
        raise ValueError("bias dtype must be float32 or bfloat16")
    o = _dev(out, "bias", None, (B, 1, S_q, max_seq))
    n = _dev(nonpad, "nonpad", torch.int64, (B,))
    qs = _opt(q_start, "q_start", torch.int64, (B,))
    sk = _opt(slot_kind, "slot_kind", torch.int32, (B, max_seq))
    _check(getattr(load(), fn)(o, _DTYPE[out.dtype], n, qs, sk, B, S_q, max_seq, int(window),
                               _stream(out)), fn)
    return out


def attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, max_seq, D, D_v=None) -> int:
    return int(load().attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, max_seq, D,
                                                    D if D_v is None else D_v))


_workspaces: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor | None:
    """The workspace of the current stream on `device`, grown on demand. One per
    (device, stream): calls on one stream are ordered and can share it, calls on
    two streams may overlap and must not. Zero-filled when allocated: its first
    bytes are the decode kernel's arrival counts, which every call leaves at
    zero. A buffer that has been replaced stays alive (a captured graph may
    still use it), and none is allocated while the stream is being captured."""
    if nbytes == 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    return _workspace_for(key, nbytes, torch.cuda.is_current_stream_capturing(),
                          lambda n: torch.zeros(n, dtype=torch.uint8, device=device))


def _workspace_for(key, nbytes: int, capturing: bool, alloc):
    held = _workspaces.setdefault(key, [])
    if held and held[-1].numel() >= nbytes:
        return held[-1]
    if capturing:
        raise RuntimeError(
            f"attn_bias_gqa_fwd: the stream's workspace must grow to {nbytes} bytes during graph "
            f"capture; make one call of this shape before capturing, or pass a zero-filled "
            f"workspace of attn_bias_gqa_workspace_bytes() bytes")
    ws = alloc(nbytes)
    held.append(ws)
    return ws


def attn_bias_gqa_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      bias: torch.Tensor | None, nonpad: torch.Tensor, scale: float,
                      q_start: torch.Tensor | None = None,
                      slot_kind: torch.Tensor | None = None, window: int = 0,
                      out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None,
                      softcap: float = 0.0) -> torch.Tensor:
    """softmax(cap(scale * Q K^T) + bias) V over the static cache (GQA: head h
    reads KV head h // (Hq // Hkv)); cap(x) = softcap * tanh(x / softcap) when
    softcap > 0, else x. bias=None evaluates the static-cache rules (nonpad,
    q_start, slot_kind, window) inside the kernel instead. V may have another
    head size than Q and K (the output takes V's). Without `workspace`, the
    current stream's own workspace is used, allocated (zero-filled) by the first
    call that needs it: make that call outside HIP graph capture, or pass a
    zero-filled `workspace` of attn_bias_gqa_workspace_bytes() bytes."""
    return _attn("attn_bias_gqa_fwd", q, k_cache, v_cache, bias, nonpad, scale, q_start, slot_kind,
                 window, out, workspace, softcap)


def attn_bias_gqa_fwd_circular(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               bias: torch.Tensor | None, kv_len: torch.Tensor, scale: float,
                               q_start: torch.Tensor | None = None,
                               slot_kind: torch.Tensor | None = None, window: int = 0,
                               out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None,
                               softcap: float = 0.0) -> torch.Tensor:
    """attn_bias_gqa_fwd over a circular cache of capacity k_cache.shape[2]:
    kv_len[b] tokens written so far, position p in slot p mod capacity; with
    bias=None the circular cache's rules are evaluated in the kernel."""
    return _attn("attn_bias_gqa_fwd_circular", q, k_cache, v_cache, bias, kv_len, scale, q_start,
                 slot_kind, window, out, workspace, softcap)


def _attn(fn, q, k_cache, v_cache, bias, nonpad, scale, q_start, slot_kind, window, out, workspace,
          softcap):
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, S_q, D], k_cache [B, Hkv, max_seq, D], "
                         "v_cache [B, Hkv, max_seq, D_v]")
    B, Hq, S_q, D = q.shape
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    Dv = v_cache.shape[3]
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float32 or bfloat16")
    qp = _dev(q, "q")
    kp = _dev(k_cache, "k_cache", q.dtype, (B, Hkv, T, D))
    vp_ = _dev(v_cache, "v_cache", q.dtype, (B, Hkv, T, Dv))
    bp, bdt = None, BF16
    if bias is not None:
        if bias.dtype not in _DTYPE:
            raise ValueError("bias must be float32 or bfloat16")
        bp, bdt = _dev(bias, "bias", None, (B, 1, S_q, T)), _DTYPE[bias.dtype]
    npd = _dev(nonpad, "nonpad", torch.int64, (B,))
    qs = _opt(q_start, "q_start", torch.int64, (B,))
    sk = _opt(slot_kind, "slot_kind", torch.int32, (B, T))
    if out is None:
        out = q.new_empty((B, Hq, S_q, Dv))
    op = _dev(out, "out", q.dtype, (B, Hq, S_q, Dv))
    lib = load()
    need = int(lib.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, T, D, Dv))
    if workspace is None:
        workspace = _workspace(q.device, need)
    wp = None if workspace is None else _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(lib, fn)(op, qp, kp, vp_, bp, bdt, npd, qs, sk, B, Hq, Hkv, S_q, T, D, Dv,
                            float(scale), float(softcap), int(window), _DTYPE[q.dtype], wp, wbytes,
                            _stream(q)), fn)
    return out


def attn_bias_gqa_decode_step(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              k_update: torch.Tensor | None, v_update: torch.Tensor | None,
                              write_indices: torch.Tensor | None, nonpad: torch.Tensor,
                              scale: float, q_start: torch.Tensor | None = None,
                              slot_kind: torch.Tensor | None = None, window: int = 0,
                              bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None,
                              softcap: float = 0.0) -> torch.Tensor:
    """One decode step in one launch, bit-identical to kv_scatter_and_bias
    (k_update / v_update rows into the caches at write_indices; the bias into
    `bias` when given) followed by attn_bias_gqa_fwd. k_update = v_update =
    None: nothing to scatter (a KV-shared layer). Returns out."""
    return _step("attn_bias_gqa_decode_step", q, k_cache, v_cache, k_update, v_update, write_indices,
                 nonpad, scale, q_start, slot_kind, window, bias, out, workspace, softcap)


def attn_bias_gqa_decode_step_circular(q: torch.Tensor, k_cache: torch.Tensor,
                                       v_cache: torch.Tensor, k_update: torch.Tensor | None,
                                       v_update: torch.Tensor | None,
                                       write_pos: torch.Tensor | None, kv_len: torch.Tensor,
                                       scale: float, q_start: torch.Tensor | None = None,
                                       slot_kind: torch.Tensor | None = None, window: int = 0,
                                       bias: torch.Tensor | None = None,
                                       out: torch.Tensor | None = None,
                                       workspace: torch.Tensor | None = None,
                                       softcap: float = 0.0) -> torch.Tensor:
    """attn_bias_gqa_decode_step over a circular cache of capacity
    k_cache.shape[2] (kv_len tokens written so far, position p in slot p mod
    capacity)."""
    return _step("attn_bias_gqa_decode_step_circular", q, k_cache, v_cache, k_update, v_update,
                 write_pos, kv_len, scale, q_start, slot_kind, window, bias, out, workspace, softcap)


def _step(fn, q, k_cache, v_cache, k_update, v_update, write_indices, nonpad, scale, q_start,
          slot_kind, window, bias, out, workspace, softcap):
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, S_q, D], k_cache [B, Hkv, max_seq, D], "
                         "v_cache [B, Hkv, max_seq, D_v]")
    B, Hq, S_q, D = q.shape
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    Dv = v_cache.shape[3]
    if q.dtype != torch.bfloat16:
        raise ValueError("the fused decode step takes bfloat16 tensors")
    qp = _dev(q, "q")
    kp = _dev(k_cache, "k_cache", q.dtype, (B, Hkv, T, D))
    vp_ = _dev(v_cache, "v_cache", q.dtype, (B, Hkv, T, Dv))
    if (k_update is None) != (v_update is None):
        raise ValueError("k_update and v_update must both be given or both be None")
    S_new = 0 if k_update is None else k_update.shape[2]
    ku = _dev(k_update, "k_update", q.dtype, (B, Hkv, S_new, D)) if S_new else None
    vu = _dev(v_update, "v_update", q.dtype, (B, Hkv, S_new, Dv)) if S_new else None
    w = _opt(write_indices, "write_indices", torch.int64, (B,))
    bp, bdt = None, BF16
    if bias is not None:
        if bias.dtype not in _DTYPE:
            raise ValueError("bias must be float32 or bfloat16")
        bp, bdt = _dev(bias, "bias", None, (B, 1, S_q, T)), _DTYPE[bias.dtype]
    npd = _dev(nonpad, "nonpad", torch.int64, (B,))
    qs = _opt(q_start, "q_start", torch.int64, (B,))
    sk = _opt(slot_kind, "slot_kind", torch.int32, (B, T))
    if out is None:
        out = q.new_empty((B, Hq, S_q, Dv))
    op = _dev(out, "out", q.dtype, (B, Hq, S_q, Dv))
    lib = load()
    need = int(lib.attn_bias_gqa_workspace_bytes(B, Hq, Hkv, S_q, T, D, Dv))
    if workspace is None:
        workspace = _workspace(q.device, need)
    wp = None if workspace is None else _dev(workspace, "workspace")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(lib, fn)(op, qp, kp, vp_, ku, vu, w, S_new, bp, bdt, npd, qs, sk, B, Hq, Hkv, S_q,
                            T, D, Dv, float(scale), float(softcap), int(window), BF16, wp, wbytes,
                            _stream(q)), fn)
    return out


def attn_bias_gqa_fwd_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              bias: torch.Tensor | None, nonpad: torch.Tensor, scale: float,
                              out: torch.Tensor, q_start: torch.Tensor | None = None,
                              slot_kind: torch.Tensor | None = None, window: int = 0,
                              softcap: float = 0.0) -> torch.Tensor:
    """attn_bias_gqa_fwd through the entry point that allocates nothing: the
    caller passes `out`, and the scratch is the library's static per-GPU array
    (8 MiB; larger needs are refused). Calls that overlap in time on one GPU
    race."""
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, S_q, D], k_cache [B, Hkv, max_seq, D], "
                         "v_cache [B, Hkv, max_seq, D_v]")
    B, Hq, S_q, D = q.shape
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    Dv = v_cache.shape[3]
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float32 or bfloat16")
    qp = _dev(q, "q")
    kp = _dev(k_cache, "k_cache", q.dtype, (B, Hkv, T, D))
    vp_ = _dev(v_cache, "v_cache", q.dtype, (B, Hkv, T, Dv))
    bp, bdt = None, BF16
    if bias is not None:
        if bias.dtype not in _DTYPE:
            raise ValueError("bias must be float32 or bfloat16")
        bp, bdt = _dev(bias, "bias", None, (B, 1, S_q, T)), _DTYPE[bias.dtype]
    npd = _dev(nonpad, "nonpad", torch.int64, (B,))
    qs = _opt(q_start, "q_start", torch.int64, (B,))
    sk = _opt(slot_kind, "slot_kind", torch.int32, (B, T))
    op = _dev(out, "out", q.dtype, (B, Hq, S_q, Dv))
    _check(load().attn_bias_gqa_fwd_noalloc(op, qp, kp, vp_, bp, bdt, npd, qs, sk, B, Hq, Hkv, S_q, T, D,
                                            Dv, float(scale), float(softcap), int(window),
                                            _DTYPE[q.dtype], _stream(q)), "attn_bias_gqa_fwd_noalloc")
    return out

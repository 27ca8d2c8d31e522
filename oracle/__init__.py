"""fp64 CPU oracle for additive-bias GQA attention over an external static KV cache.

TEST INFRASTRUCTURE ONLY: the pytest suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it. The HIP library never imports, links or
calls anything here, and this package imports nothing from the HIP side.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over output rows);
this module only builds it with gcc, widens inputs to float64 and passes host
pointers. Inputs may be numpy arrays or CPU torch tensors of any float dtype;
widening bf16/fp32 to fp64 is exact.

Functions (each cites its passage in ``oracle.c``):
  scatter(cache, update, write_indices)      TensorScatter, raw-byte copy
  bias(nonpad, q_start, slot_kind, S_q, max_seq, window)   [B,1,S_q,max_seq] fp64
  repeat_kv(x, G)                             KV head h // G for query head h
  attention(q, k_cache, v_cache, bias, nonpad, scale, rows=None)  fp64 output
  scatter_circular(cache, update, write_pos)  TensorScatter into a circular cache
  bias_circular(kv_len, q_start, slot_kind, S_q, capacity, window)  its bias
A circular cache's attention is attention() with nonpad = min(kv_len, capacity)
and the circular bias (the bias carries every rule).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math: IEEE fp64)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC,
             "-o", tmp, "-lm"],
            check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_scatter.argtypes = [_u8p, _u8p, _i64p] + [ctypes.c_int64] * 6
        lib.oracle_scatter.restype = None
        lib.oracle_bias.argtypes = [_f64p, _i64p, _i64p, _i32p] + [ctypes.c_int64] * 4
        lib.oracle_bias.restype = None
        lib.oracle_repeat_kv.argtypes = [_f64p, _f64p] + [ctypes.c_int64] * 5
        lib.oracle_repeat_kv.restype = None
        lib.oracle_attention_mha.argtypes = (
            [_f64p, _f64p, _f64p, _f64p, _f64p, _i64p] + [ctypes.c_int64] * 6
            + [ctypes.c_double, ctypes.c_double, _i64p, ctypes.c_int64, _f64p])
        lib.oracle_attention_mha.restype = None
        lib.oracle_scatter_circular.argtypes = [_u8p, _u8p, _i64p] + [ctypes.c_int64] * 6
        lib.oracle_scatter_circular.restype = None
        lib.oracle_bias_circular.argtypes = [_f64p, _i64p, _i64p, _i32p] + [ctypes.c_int64] * 4
        lib.oracle_bias_circular.restype = None
        _lib = lib
    return _lib


def _np(x) -> np.ndarray:
    """Host array view of a numpy array or CPU torch tensor (no device access)."""
    if isinstance(x, np.ndarray):
        return x
    import torch
    if isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError("the oracle takes host tensors only")
        if x.dtype == torch.bfloat16:
            return x.to(torch.float64).numpy()
        return x.numpy()
    return np.asarray(x)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(_np(x), dtype=np.float64)


def _i64(x) -> np.ndarray | None:
    return None if x is None else np.ascontiguousarray(_np(x), dtype=np.int64)


def _i32(x) -> np.ndarray | None:
    return None if x is None else np.ascontiguousarray(_np(x), dtype=np.int32)


def _ptr(a: np.ndarray | None, typ):
    return None if a is None else a.ctypes.data_as(typ)


def _scatter(fn, cache, update, write_indices):
    import torch
    is_torch = isinstance(cache, torch.Tensor)
    if is_torch:
        out_t = cache.detach().cpu().clone().contiguous()
        upd_t = update.detach().cpu().contiguous()
        if out_t.dtype != upd_t.dtype:
            raise ValueError("cache and update dtypes differ")
        elem = out_t.element_size()
        if upd_t.numel() == 0:
            return out_t
        cache_b = out_t.view(torch.uint8).numpy()
        upd_b = upd_t.view(torch.uint8).numpy()
    else:
        out_n = np.array(cache, copy=True, order="C")
        upd_n = np.ascontiguousarray(update)
        if upd_n.size == 0:
            return out_n
        elem = out_n.itemsize
        cache_b = out_n.view(np.uint8)
        upd_b = upd_n.view(np.uint8)
    B, H, max_seq, D = (out_t.shape if is_torch else out_n.shape)
    S_new = (upd_t.shape if is_torch else upd_n.shape)[2]
    w = _i64(write_indices)
    fn(_ptr(cache_b, _u8p), _ptr(upd_b, _u8p), _ptr(w, _i64p),
                           B, H, max_seq, S_new, D, elem)
    return out_t if is_torch else out_n


def scatter(cache, update, write_indices):
    """Return a copy of ``cache`` [B,H,max_seq,D] with ``update`` [B,H,S_new,D]
    written at slots write_indices[b] + t (raw bytes; out-of-range slots dropped).
    Accepts torch tensors (any dtype) or numpy arrays; returns the same kind."""
    return _scatter(_load().oracle_scatter, cache, update, write_indices)


def scatter_circular(cache, update, write_pos):
    """Return a copy of the circular cache ``cache`` [B,H,C,D] with ``update``
    [B,H,S_new,D] (S_new <= C) written at slots (write_pos[b] + t) mod C (raw
    bytes; negative positions dropped)."""
    if update.shape[2] > cache.shape[2]:
        raise ValueError("a circular scatter writes at most capacity tokens")
    return _scatter(_load().oracle_scatter_circular, cache, update, write_pos)


def bias(nonpad, q_start, slot_kind, S_q: int, max_seq: int, window: int) -> np.ndarray:
    """[B,1,S_q,max_seq] float64 bias of 0.0 (allowed) and -inf (masked)."""
    npd = _i64(nonpad)
    B = npd.shape[0]
    qs = _i64(q_start)
    kind = _i32(slot_kind)
    if kind is not None and kind.shape != (B, max_seq):
        raise ValueError("slot_kind must be [B, max_seq]")
    out = np.empty((B, 1, S_q, max_seq), dtype=np.float64)
    _load().oracle_bias(_ptr(out, _f64p), _ptr(npd, _i64p), _ptr(qs, _i64p),
                        _ptr(kind, _i32p), B, S_q, max_seq, int(window))
    return out


def bias_circular(kv_len, q_start, slot_kind, S_q: int, capacity: int, window: int) -> np.ndarray:
    """[B,1,S_q,capacity] float64 bias of a circular cache (0.0 / -inf): kv_len[b]
    tokens written so far, position p in slot p mod capacity."""
    L = _i64(kv_len)
    B = L.shape[0]
    qs = _i64(q_start)
    kind = _i32(slot_kind)
    if kind is not None and kind.shape != (B, capacity):
        raise ValueError("slot_kind must be [B, capacity]")
    out = np.empty((B, 1, S_q, capacity), dtype=np.float64)
    _load().oracle_bias_circular(_ptr(out, _f64p), _ptr(L, _i64p), _ptr(qs, _i64p),
                                 _ptr(kind, _i32p), B, S_q, capacity, int(window))
    return out


def repeat_kv(x, G: int) -> np.ndarray:
    """[B,Hkv,T,D] -> [B,Hkv*G,T,D] float64, query head h reading KV head h // G."""
    src = _f64(x)
    B, Hkv, T, D = src.shape
    dst = np.empty((B, Hkv * G, T, D), dtype=np.float64)
    _load().oracle_repeat_kv(_ptr(dst, _f64p), _ptr(src, _f64p), B, Hkv, G, T, D)
    return dst


def attention_mha(q, k, v, bias_, nonpad, scale: float, rows=None, softcap: float = 0.0) -> np.ndarray:
    """Dense attention with K/V already at Hq heads: q, k [.., D], v [.., Dv]
    (the value head size may differ). Returns [B,H,S_q,Dv] float64, or
    [len(rows), Dv] for the flat rows (b*H + h)*S_q + s when ``rows`` is given.
    softcap > 0 applies softcap * tanh(score / softcap) to scale * q.k before the
    bias is added (0 = none)."""
    qd, kd, vd, bd = _f64(q), _f64(k), _f64(v), _f64(bias_)
    npd = _i64(nonpad)
    B, H, S_q, D = qd.shape
    T = kd.shape[2]
    Dv = vd.shape[3]
    if kd.shape != (B, H, T, D) or vd.shape != (B, H, T, Dv):
        raise ValueError("k must be [B,H,T,D] and v [B,H,T,Dv] with the query's heads")
    if bd.shape != (B, 1, S_q, T):
        raise ValueError("bias must be [B,1,S_q,T]")
    r = _i64(rows)
    n = B * H * S_q if r is None else r.shape[0]
    out = np.empty((n, Dv), dtype=np.float64)
    scratch = np.empty((n, T), dtype=np.float64)
    _load().oracle_attention_mha(
        _ptr(out, _f64p), _ptr(qd, _f64p), _ptr(kd, _f64p), _ptr(vd, _f64p),
        _ptr(bd, _f64p), _ptr(npd, _i64p), B, H, S_q, T, D, Dv, float(scale), float(softcap),
        _ptr(r, _i64p), 0 if r is None else n, _ptr(scratch, _f64p))
    return out.reshape(B, H, S_q, Dv) if r is None else out


def attention(q, k_cache, v_cache, bias_, nonpad, scale: float, rows=None,
              softcap: float = 0.0) -> np.ndarray:
    """GQA attention: repeat the KV heads (h // G), then dense attention.

    q [B,Hq,S_q,D], k_cache [B,Hkv,T,D], v_cache [B,Hkv,T,Dv], bias [B,1,S_q,T],
    nonpad [B]. With ``rows`` (flat (b*Hq + h)*S_q + s indices) only those rows
    are computed, one batch entry at a time, so the repeated KV heads of one
    entry are the most that is materialised. Returns float64 [B,Hq,S_q,Dv] or
    [len(rows), Dv].
    """
    npd = _i64(nonpad)
    B, Hq, S_q, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if rows is None:
        return attention_mha(_np(q), repeat_kv(_np(k_cache), G), repeat_kv(_np(v_cache), G),
                             _np(bias_), npd, scale, softcap=softcap)
    rows = _i64(rows)
    out = np.empty((rows.shape[0], v_cache.shape[3]), dtype=np.float64)
    per_batch = Hq * S_q
    for b in np.unique(rows // per_batch):
        b = int(b)
        sel = np.nonzero(rows // per_batch == b)[0]
        local = rows[sel] - b * per_batch
        # slice before widening: one batch entry in fp64 at a time
        out[sel] = attention_mha(_np(q[b:b + 1]), repeat_kv(_np(k_cache[b:b + 1]), G),
                                 repeat_kv(_np(v_cache[b:b + 1]), G), _np(bias_[b:b + 1]),
                                 npd[b:b + 1], scale, rows=local, softcap=softcap)
    return out

"""Pins for the fp64 oracle, CPU only (no GPU, no HIP library).

Each test ties an oracle function to something other than itself: a library
routine (torch's tril/triu, scaled_dot_product_attention, numpy indexing and
repeat), hand-derived fixtures under tests/golden/, closed forms, invariants
the pages state, and a 50-digit mpmath brute force on tiny inputs. They are
chosen so that a dropped term, a wrong sign, an off-by-one, a swapped operand
or a wrong head mapping in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from additive_bias_gqa_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEG_INF = float("-inf")


# --------------------------------------------------------------------------- #
# fixture parsing
# --------------------------------------------------------------------------- #
def _bias_cases(fname="bias_cases.txt"):
    cases, cur = [], None
    with open(os.path.join(GOLDEN, fname)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "kind": None, "expect": {}}
                cases.append(cur)
            elif tok[0] == "dims":
                for kv in tok[1:]:
                    k, v = kv.split("=")
                    cur[k] = int(v)
            elif tok[0] == "nonpad":
                cur["nonpad"] = [int(x) for x in tok[1:]]
            elif tok[0] == "q_start":
                cur["q_start"] = None if tok[1] == "default" else [int(x) for x in tok[1:]]
            elif tok[0] == "kind":
                if tok[1] == "none":
                    continue
                if cur["kind"] is None:
                    cur["kind"] = np.zeros((cur["B"], cur["max_seq"]), dtype=np.int32)
                cur["kind"][int(tok[1])] = [int(x) for x in tok[2:]]
            elif tok[0] == "expect":
                cur["expect"][(int(tok[1]), int(tok[2]))] = tok[3]
    return cases


def _attention_cases():
    data, cases = {}, []
    with open(os.path.join(GOLDEN, "attention_cases.txt")) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "data":
                rows = " ".join(tok[2:]).split("|")
                vals = [[float(x) for x in r.split()] for r in rows]
                data[tok[1]] = vals[0] if len(vals) == 1 else vals
            elif tok[0] == "case":
                i_np, i_b, i_e = tok.index("nonpad"), tok.index("bias"), tok.index("expect")
                cases.append({
                    "name": tok[1],
                    "nonpad": int(tok[i_np + 1]),
                    "bias": [float(x) for x in tok[i_b + 1:i_e]],
                    "expect": [float(x) for x in tok[i_e + 1:]],
                })
    return data, cases


def _mask_str(row):
    return "".join("0" if v == 0.0 else "-" for v in row)


# --------------------------------------------------------------------------- #
# bias builder
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("case", _bias_cases(), ids=lambda c: c["name"])
def test_bias_golden(case):
    out = oracle.bias(case["nonpad"], case["q_start"], case["kind"], case["S_q"],
                      case["max_seq"], case["window"])
    assert out.shape == (case["B"], 1, case["S_q"], case["max_seq"])
    # only +0.0 and -inf ever appear
    assert np.all((out == NEG_INF) | ((out == 0.0) & ~np.signbit(out)))
    assert len(case["expect"]) == case["B"] * case["S_q"]
    for (b, s), want in case["expect"].items():
        assert _mask_str(out[b, 0, s]) == want, (case["name"], b, s)


def _torch_mask_to_bias(allowed: torch.Tensor) -> np.ndarray:
    return torch.where(allowed, 0.0, NEG_INF).to(torch.float64).numpy()


def test_bias_textbook_causal_is_tril():
    # S_q == nonpad == max_seq, no window, no kinds: upper-left and bottom-right
    # alignments coincide, and the mask is the lower-triangular matrix.
    T = 37
    out = oracle.bias([T], None, None, S_q=T, max_seq=T, window=0)
    ref = _torch_mask_to_bias(torch.tril(torch.ones(T, T, dtype=torch.bool)))
    np.testing.assert_array_equal(out[0, 0], ref)


@pytest.mark.parametrize("W", [1, 2, 5, 36, 37, 100])
def test_bias_window_is_band(W):
    # keys [q-W+1, q]: the band between tril and triu(diagonal = -(W-1)).
    T = 37
    out = oracle.bias([T], None, None, S_q=T, max_seq=T, window=W)
    ones = torch.ones(T, T, dtype=torch.bool)
    ref = _torch_mask_to_bias(torch.tril(ones) & torch.triu(ones, diagonal=-(W - 1)))
    np.testing.assert_array_equal(out[0, 0], ref)


@pytest.mark.parametrize("S_q,nonpad,T", [(1, 17, 32), (5, 17, 32), (17, 17, 17), (40, 30, 64), (8, 0, 16)])
def test_bias_maskless_causal_is_bottom_right(S_q, nonpad, T):
    # Maskless is_causal=1 over an external cache (onnx#8068, as the skill page's
    # section 11 states it): query i sees key j iff j <= i + max(nonpad - S_q, 0)
    # and j < nonpad. With no window and no slot kinds the default query offset
    # gives exactly that: a lower triangle shifted by the offset (torch.tril with
    # a diagonal), cut at nonpad.
    out = oracle.bias([nonpad], None, None, S_q=S_q, max_seq=T, window=0)
    off = max(nonpad - S_q, 0)
    tri = torch.tril(torch.ones(S_q, T, dtype=torch.bool), diagonal=off)
    tri[:, nonpad:] = False
    np.testing.assert_array_equal(out[0, 0], _torch_mask_to_bias(tri))


def test_bias_decode_row():
    # decode (S_q = 1) with the default q_start: the query sits at slot nonpad-1
    # and, without a window, sees exactly the nonpad valid slots.
    rng = wl.rng_for(60)
    T = 53
    nonpad = rng.integers(0, T, size=16, endpoint=True)
    out = oracle.bias(nonpad, None, None, S_q=1, max_seq=T, window=0)
    for b, n in enumerate(nonpad):
        want = np.where(np.arange(T) < n, 0.0, NEG_INF)
        np.testing.assert_array_equal(out[b, 0, 0], want)
    # with a window W the row keeps only the last W valid slots
    W = 7
    out = oracle.bias(nonpad, None, None, S_q=1, max_seq=T, window=W)
    for b, n in enumerate(nonpad):
        j = np.arange(T)
        want = np.where((j < n) & (j >= n - W), 0.0, NEG_INF)
        np.testing.assert_array_equal(out[b, 0, 0], want)


def _random_kinds(rng, B, T, n_blocks=2):
    kind = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        kind[b, rng.random(T) < 0.15] = wl.PAD
        for blk in range(1, n_blocks + 1):
            lo = int(rng.integers(0, T))
            ln = int(rng.integers(1, max(2, T // 3)))
            kind[b, lo:lo + ln] = blk
    return kind


def _allowed_by_sets(nonpad, q_start, kind, S_q, T, W):
    """The rule restated with set algebra, one query at a time."""
    B = len(nonpad)
    res = np.zeros((B, S_q, T), dtype=bool)
    for b in range(B):
        n = min(max(int(nonpad[b]), 0), T)
        qs = int(q_start[b]) if q_start is not None else max(n - S_q, 0)
        pads = {j for j in range(T) if kind[b, j] < 0}
        valid = set(range(n)) - pads
        for s in range(S_q):
            q = qs + s
            lo = (q - W + 1) if W > 0 else 0
            seen = set(range(max(lo, 0), min(q, T - 1) + 1)) if q >= 0 else set()
            kq = int(kind[b, q]) if 0 <= q < T else 0
            if kq > 0:
                seen |= {j for j in range(T) if kind[b, j] == kq}
            for j in valid & seen:
                res[b, s, j] = True
    return res


@pytest.mark.parametrize("seed", range(6))
def test_bias_matches_set_enumeration(seed):
    rng = wl.rng_for(70 + seed)
    B, T = 3, int(rng.integers(8, 33))
    S_q = int(rng.integers(1, T + 1))
    W = int(rng.integers(-1, T + 3))
    nonpad = rng.integers(0, T, size=B, endpoint=True)
    kind = _random_kinds(rng, B, T)
    explicit = rng.integers(-3, T + 2, size=B)
    for q_start in (None, explicit):
        out = oracle.bias(nonpad, q_start, kind, S_q, T, W)
        want = _allowed_by_sets(nonpad, q_start, kind, S_q, T, W)
        np.testing.assert_array_equal(out[:, 0] == 0.0, want)


def test_bias_invariants():
    rng = wl.rng_for(80)
    B, T, S_q, W = 4, 40, 12, 6
    kind = _random_kinds(rng, B, T)
    q_start = rng.integers(0, T - S_q, size=B, endpoint=True)
    nonpad = rng.integers(0, T, size=B, endpoint=True)
    out = oracle.bias(nonpad, q_start, kind, S_q, T, W)
    allowed = out[:, 0] == 0.0
    for b in range(B):
        # a pad slot is never an allowed key, whatever the query
        assert not allowed[b][:, kind[b] < 0].any()
        # nothing at or beyond nonpad
        assert not allowed[b][:, int(nonpad[b]):].any()
        # two valid tokens of one block inside the chunk see each other both ways
        for s1 in range(S_q):
            for s2 in range(S_q):
                q1, q2 = int(q_start[b]) + s1, int(q_start[b]) + s2
                if kind[b, q1] > 0 and kind[b, q1] == kind[b, q2] and max(q1, q2) < nonpad[b]:
                    assert allowed[b, s1, q2] and allowed[b, s2, q1]
    # raising nonpad (fixed q_start) only ever adds allowed keys
    more = oracle.bias(np.minimum(nonpad + 5, T), q_start, kind, S_q, T, W)[:, 0] == 0.0
    assert not (allowed & ~more).any()


# --------------------------------------------------------------------------- #
# scatter
# --------------------------------------------------------------------------- #
def test_scatter_matches_numpy_indexing():
    rng = wl.rng_for(90)
    B, H, T, D, S_new = 5, 3, 20, 8, 6
    cache = wl.garbage(rng, (B, H, T, D), torch.bfloat16)
    upd = wl.garbage(rng, (B, H, S_new, D), torch.bfloat16)
    w = np.array([0, 3, T - S_new, T - 2, -2], dtype=np.int64)  # last two run off the ends
    out = oracle.scatter(cache, upd, w)
    want = cache.view(torch.int16).numpy().copy()
    u = upd.view(torch.int16).numpy()
    for b in range(B):
        idx = np.arange(S_new) + w[b]
        ok = (idx >= 0) & (idx < T)
        want[b][:, idx[ok]] = u[b][:, ok]
    np.testing.assert_array_equal(out.view(torch.int16).numpy(), want)


def test_scatter_keeps_bits_and_noop():
    rng = wl.rng_for(91)
    cache = wl.garbage(rng, (2, 2, 9, 4), torch.float32)
    upd = wl.garbage(rng, (2, 2, 0, 4), torch.float32)
    out = oracle.scatter(cache, upd, np.array([1, 2]))
    np.testing.assert_array_equal(out.view(torch.int32).numpy(), cache.view(torch.int32).numpy())
    upd = wl.garbage(rng, (2, 2, 2, 4), torch.float32)
    out = oracle.scatter(cache, upd, None)  # NULL write indices -> slot 0
    np.testing.assert_array_equal(out[:, :, :2].view(torch.int32).numpy(),
                                  upd.view(torch.int32).numpy())
    np.testing.assert_array_equal(out[:, :, 2:].view(torch.int32).numpy(),
                                  cache[:, :, 2:].view(torch.int32).numpy())


# --------------------------------------------------------------------------- #
# attention
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("case", _attention_cases()[1], ids=lambda c: c["name"])
def test_attention_golden(case):
    data, _ = _attention_cases()
    q = np.array(data["q"], dtype=np.float64).reshape(1, 1, 1, -1)
    k = np.array(data["k"], dtype=np.float64).reshape(1, 1, 3, -1)
    v = np.array(data["v"], dtype=np.float64).reshape(1, 1, 3, -1)
    bias = np.array(case["bias"], dtype=np.float64).reshape(1, 1, 1, 3)
    y = oracle.attention(q, k, v, bias, [case["nonpad"]], float(data["scale"][0]))
    np.testing.assert_allclose(y[0, 0, 0], case["expect"], rtol=0, atol=1e-12)


def _rand(rng, shape):
    return rng.standard_normal(size=shape)


def _sdpa(q, k, v, mask, scale):
    import torch.nn.functional as F
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return F.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else t(mask), scale=scale,
        enable_gqa=True).numpy()


def test_attention_zero_bias_is_sdpa():
    rng = wl.rng_for(100)
    B, Hq, Hkv, S_q, T, D = 2, 6, 2, 5, 11, 8
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    bias = np.zeros((B, 1, S_q, T))
    y = oracle.attention(q, k, v, bias, [T] * B, 0.37)
    np.testing.assert_allclose(y, _sdpa(q, k, v, None, 0.37), rtol=0, atol=1e-12)


def test_attention_float_bias_is_sdpa():
    rng = wl.rng_for(101)
    B, Hq, Hkv, S_q, T, D = 2, 4, 1, 7, 13, 5
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    bias = 3.0 * _rand(rng, (B, 1, S_q, T))
    y = oracle.attention(q, k, v, bias, [T] * B, 1 / math.sqrt(D))
    np.testing.assert_allclose(y, _sdpa(q, k, v, bias, 1 / math.sqrt(D)), rtol=0, atol=1e-12)


def test_attention_masks_and_nonpad_are_sdpa():
    rng = wl.rng_for(102)
    B, Hq, Hkv, S_q, T, D = 3, 8, 2, 6, 17, 4
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    bias = _rand(rng, (B, 1, S_q, T))
    bias[rng.random(bias.shape) < 0.4] = NEG_INF
    bias[1, 0, 2, :] = NEG_INF                     # one fully-masked row
    nonpad = np.array([T, 9, 0])                   # batch 2: empty cache
    y = oracle.attention(q, k, v, bias, nonpad, 0.5)
    full = bias.copy()
    for b in range(B):
        full[b, :, :, nonpad[b]:] = NEG_INF
    live = np.isfinite(full).any(axis=-1)          # [B,1,S_q]
    ref = _sdpa(q, k, v, full, 0.5)
    for b in range(B):
        for s in range(S_q):
            if live[b, 0, s]:
                np.testing.assert_allclose(y[b, :, s], ref[b, :, s], rtol=0, atol=1e-12)
            else:
                # fully-masked row and empty batch: exact zeros, never NaN
                assert np.all(y[b, :, s] == 0.0)


@pytest.mark.parametrize("D,Dv", [(4, 12), (12, 4)])
def test_value_head_size_is_sdpa(D, Dv):
    # head_size != v_head_size (K and V of different head sizes, as KV-shared
    # layers borrowing another layer's V produce): the scores use D, the
    # output takes V's Dv columns; SDPA defines the same product
    rng = wl.rng_for(104 + D)
    B, Hq, Hkv, S_q, T = 2, 6, 3, 5, 13
    q, k = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D))
    v = _rand(rng, (B, Hkv, T, Dv))
    bias = _rand(rng, (B, 1, S_q, T))
    bias[rng.random(bias.shape) < 0.3] = NEG_INF
    nonpad = np.array([T, 8])
    y = oracle.attention(q, k, v, bias, nonpad, 0.6)
    assert y.shape == (B, Hq, S_q, Dv)
    full = bias.copy()
    for b in range(B):
        full[b, :, :, nonpad[b]:] = NEG_INF
    live = np.isfinite(full).any(axis=-1)
    ref = _sdpa(q, k, v, full, 0.6)
    for b in range(B):
        for s in range(S_q):
            if live[b, 0, s]:
                np.testing.assert_allclose(y[b, :, s], ref[b, :, s], rtol=0, atol=1e-12)
            else:
                assert np.all(y[b, :, s] == 0.0)


def test_value_head_size_columns_are_independent():
    # each output column is the same weighted mean of one V column: a V of
    # Dv columns gives what Dv single-column V's give, and the weights do not
    # depend on V at all (a closed form of softmax(.) V)
    rng = wl.rng_for(106)
    B, Hq, Hkv, S_q, T, D, Dv = 1, 2, 1, 3, 9, 5, 7
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, Dv))
    bias = oracle.bias(np.array([T]), None, None, S_q, T, 0)
    y = oracle.attention(q, k, v, bias, [T], 0.4)
    for c in range(Dv):
        yc = oracle.attention(q, k, v[..., c:c + 1], bias, [T], 0.4)
        np.testing.assert_allclose(y[..., c:c + 1], yc, rtol=0, atol=0)
    ones = oracle.attention(q, k, np.ones((B, Hkv, T, 3)), bias, [T], 0.4)
    np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-14)


def test_attention_mpmath_bruteforce():
    import mpmath as mp
    mp.mp.dps = 50
    rng = wl.rng_for(103)
    B, Hq, Hkv, S_q, T, D = 2, 4, 2, 3, 6, 4
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    bias = 2.0 * _rand(rng, (B, 1, S_q, T))
    bias[rng.random(bias.shape) < 0.3] = NEG_INF
    nonpad = [5, 6]
    scale = 0.41
    y = oracle.attention(q, k, v, bias, nonpad, scale)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for s in range(S_q):
                keys = [j for j in range(T) if j < nonpad[b] and bias[b, 0, s, j] != NEG_INF]
                if not keys:
                    assert np.all(y[b, h, s] == 0.0)
                    continue
                xs = {j: mp.mpf(scale) * mp.fsum(mp.mpf(q[b, h, s, d]) * mp.mpf(k[b, h // G, j, d])
                                                 for d in range(D)) + mp.mpf(bias[b, 0, s, j])
                      for j in keys}
                ws = {j: mp.exp(xs[j]) for j in keys}
                tot = mp.fsum(ws.values())
                for d in range(D):
                    ref = mp.fsum(ws[j] * mp.mpf(v[b, h // G, j, d]) for j in keys) / tot
                    assert abs(float(ref) - y[b, h, s, d]) <= 1e-13


def test_attention_masked_slots_contribute_nothing():
    rng = wl.rng_for(104)
    B, Hq, Hkv, S_q, T, D = 2, 4, 2, 5, 24, 8
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    kind = np.zeros((B, T), dtype=np.int32)
    kind[0, [1, 4, 9]] = wl.PAD
    kind[1, [0, 2]] = wl.PAD
    nonpad = np.array([17, 21])
    bias = oracle.bias(nonpad, None, kind, S_q, T, 9)
    y = oracle.attention(q, k, v, bias, nonpad, 0.3)
    dead = np.ones((B, T), dtype=bool)          # slots masked for every query row
    dead &= (bias[:, 0] == NEG_INF).all(axis=1)
    assert dead[0, 1] and dead[0, 20] and not dead[0, 16]
    for poison in (np.nan, np.inf, -np.inf, 1e30):
        k2, v2 = k.copy(), v.copy()
        for b in range(B):
            k2[b][:, dead[b]] = poison
            v2[b][:, dead[b]] = poison
        y2 = oracle.attention(q, k2, v2, bias, nonpad, 0.3)
        np.testing.assert_array_equal(y2, y)
    # per-row: poisoning a key that only this row masks leaves this row alone
    s, b = 0, 0
    row_dead = np.nonzero((bias[b, 0, s] == NEG_INF) & ~dead[b])[0]
    assert row_dead.size > 0
    v3 = v.copy()
    v3[b][:, row_dead] = 1e30
    y3 = oracle.attention(q, k, v3, bias, nonpad, 0.3)
    np.testing.assert_array_equal(y3[b, :, s], y[b, :, s])


def test_attention_decode_is_prefill_row():
    rng = wl.rng_for(105)
    B, Hq, Hkv, T, D, W = 2, 4, 2, 30, 8, 6
    k, v = _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    kind = np.zeros((B, T), dtype=np.int32)
    kind[0, 10:16] = 1
    kind[1, :3] = wl.PAD
    for p in (0, 5, 12, 13, 21):
        n = p + 1
        qp = _rand(rng, (B, Hq, n, D))
        bp = oracle.bias([n] * B, [0] * B, kind, n, T, W)
        yp = oracle.attention(qp, k, v, bp, [n] * B, 0.35)
        bd = oracle.bias([n] * B, None, kind, 1, T, W)     # default q_start = n - 1 = p
        yd = oracle.attention(qp[:, :, p:p + 1], k, v, bd, [n] * B, 0.35)
        np.testing.assert_array_equal(yd[:, :, 0], yp[:, :, p])


def test_attention_gqa_is_mha_with_repeated_kv():
    rng = wl.rng_for(106)
    B, Hq, Hkv, S_q, T, D = 2, 12, 3, 4, 9, 5
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    bias = _rand(rng, (B, 1, S_q, T))
    bias[rng.random(bias.shape) < 0.3] = NEG_INF
    nonpad = [7, 9]
    y = oracle.attention(q, k, v, bias, nonpad, 0.6)
    G = Hq // Hkv
    y_mha = oracle.attention_mha(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                 bias, nonpad, 0.6)
    np.testing.assert_array_equal(y, y_mha)
    np.testing.assert_array_equal(oracle.repeat_kv(k, G), np.repeat(k, G, axis=1))


def test_attention_head_mapping_contiguous_groups():
    # query head h reads KV head h // G: with constant V per KV head the output
    # of each query head is that constant.
    B, Hq, Hkv, T, D = 1, 6, 3, 4, 2
    q = np.ones((B, Hq, 1, D))
    k = np.zeros((B, Hkv, T, D))
    v = np.stack([np.full((T, D), c) for c in (1.0, 2.0, 3.0)])[None]
    y = oracle.attention(q, k, v, np.zeros((B, 1, 1, T)), [T], 1.0)
    np.testing.assert_array_equal(y[0, :, 0, 0], [1, 1, 2, 2, 3, 3])


def test_attention_closed_forms():
    rng = wl.rng_for(107)
    B, Hq, Hkv, S_q, T, D = 1, 2, 1, 3, 10, 6
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    # one live key -> exactly that V row
    bias = np.full((B, 1, S_q, T), NEG_INF)
    bias[0, 0, :, 4] = 0.0
    y = oracle.attention(q, k, v, bias, [T], 0.5)
    for h in range(Hq):
        for s in range(S_q):
            np.testing.assert_array_equal(y[0, h, s], v[0, 0, 4])
    # identical keys -> the mean of the live V rows
    kk = np.repeat(k[:, :, :1], T, axis=2)
    bias = np.zeros((B, 1, S_q, T))
    bias[0, 0, :, [2, 7]] = NEG_INF
    y = oracle.attention(q, kk, v, bias, [8], 0.5)
    live = [0, 1, 3, 4, 5, 6]
    np.testing.assert_allclose(y[0, 0, 0], v[0, 0, live].mean(axis=0), rtol=0, atol=1e-14)
    # a constant added to every live bias entry changes nothing (large: an
    # implementation without the max subtraction overflows)
    b0 = _rand(rng, (B, 1, S_q, T))
    b0[0, 0, 1, 3] = NEG_INF
    y0 = oracle.attention(q, k, v, b0, [T], 0.5)
    y1 = oracle.attention(q, k, v, b0 + 1e4, [T], 0.5)
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-11)
    # weights sum to one: V = ones gives ones
    y = oracle.attention(q, k, np.ones_like(v), b0, [T], 0.5)
    np.testing.assert_allclose(y, 1.0, rtol=0, atol=1e-15)
    # no live key -> zeros
    y = oracle.attention(q, k, v, np.full((B, 1, S_q, T), NEG_INF), [T], 0.5)
    assert np.all(y == 0.0)


def test_attention_rows_subset_matches_full():
    rng = wl.rng_for(108)
    B, Hq, Hkv, S_q, T, D = 3, 4, 2, 5, 12, 8
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    bias = oracle.bias([12, 7, 3], None, None, S_q, T, 4)
    y = oracle.attention(q, k, v, bias, [12, 7, 3], 0.3)
    rows = np.array([0, 7, 19, 20, 44, 59])
    ys = oracle.attention(q, k, v, bias, [12, 7, 3], 0.3, rows=rows)
    np.testing.assert_array_equal(ys, y.reshape(-1, D)[rows])


def test_workload_generator_is_seeded():
    a = wl.decode_sliding(B=2, Hq=4, Hkv=2, D=64, max_seq=128, window=16, nonpad_lo=8)
    b = wl.decode_sliding(B=2, Hq=4, Hkv=2, D=64, max_seq=128, window=16, nonpad_lo=8)
    assert torch.equal(a.steps[0].q, b.steps[0].q)
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    s = a.steps[0]
    assert torch.equal(s.write_indices, s.nonpad - 1) and torch.equal(s.q_start, s.nonpad - 1)


# --------------------------------------------------------------------------- #
# softcap (the skill page, section 4 "Softcap Ordering"): stage 1 between the
# scaled scores and the bias
# --------------------------------------------------------------------------- #
def test_softcap_mpmath_bruteforce():
    # 50-digit brute force with the stage order of the page: scale*QK^T, then
    # c * tanh(. / c), then + bias (a -inf bias stays -inf), softmax, times V
    import mpmath as mp
    mp.mp.dps = 50
    rng = wl.rng_for(120)
    B, Hq, Hkv, S_q, T, D = 1, 4, 2, 3, 7, 4
    q, k, v = _rand(rng, (B, Hq, S_q, D)), 3.0 * _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    bias = 2.0 * _rand(rng, (B, 1, S_q, T))
    bias[rng.random(bias.shape) < 0.3] = NEG_INF
    nonpad, scale, cap = [6], 0.9, 1.7
    y = oracle.attention(q, k, v, bias, nonpad, scale, softcap=cap)
    G = Hq // Hkv
    for h in range(Hq):
        for s in range(S_q):
            keys = [j for j in range(T) if j < nonpad[0] and bias[0, 0, s, j] != NEG_INF]
            if not keys:
                assert np.all(y[0, h, s] == 0.0)
                continue
            xs = {}
            for j in keys:
                raw = mp.mpf(scale) * mp.fsum(mp.mpf(q[0, h, s, d]) * mp.mpf(k[0, h // G, j, d])
                                              for d in range(D))
                xs[j] = mp.mpf(cap) * mp.tanh(raw / mp.mpf(cap)) + mp.mpf(bias[0, 0, s, j])
            ws = {j: mp.exp(xs[j]) for j in keys}
            tot = mp.fsum(ws.values())
            for d in range(D):
                ref = mp.fsum(ws[j] * mp.mpf(v[0, h // G, j, d]) for j in keys) / tot
                assert abs(float(ref) - y[0, h, s, d]) <= 1e-13


def test_softcap_limits():
    rng = wl.rng_for(121)
    B, Hq, Hkv, S_q, T, D = 2, 4, 2, 5, 20, 8
    q, k, v = _rand(rng, (B, Hq, S_q, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    nonpad = np.array([17, 20])
    bias = oracle.bias(nonpad, None, None, S_q, T, 0)
    plain = oracle.attention(q, k, v, bias, nonpad, 0.5)
    # a cap far above every score: tanh(y) = y + O(y^3), the cap changes nothing
    big = oracle.attention(q, k, v, bias, nonpad, 0.5, softcap=1e7)
    np.testing.assert_allclose(big, plain, rtol=0, atol=1e-12)
    # a vanishing cap flattens every score to ~0: the weights become uniform and
    # each row is the plain mean of its live V rows
    flat = oracle.attention(q, k, v, bias, nonpad, 0.5, softcap=1e-12)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for s in range(S_q):
                live = [j for j in range(T) if j < nonpad[b] and bias[b, 0, s, j] != NEG_INF]
                np.testing.assert_allclose(flat[b, h, s], v[b, h // G, live].mean(axis=0),
                                           rtol=0, atol=1e-10)


def test_softcap_keeps_masks_and_bounds_weights():
    # the ordering property the page motivates: with a small cap, a -inf bias
    # entry still removes its key (poison V there changes nothing), because the
    # cap acts before the bias; and two live keys with equal bias have weights
    # within a factor e^(2c) of each other
    rng = wl.rng_for(122)
    B, Hq, Hkv, S_q, T, D = 1, 2, 1, 4, 12, 12
    q, k, v = 4.0 * _rand(rng, (B, Hq, S_q, D)), 4.0 * _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    nonpad = np.array([T])
    bias = np.zeros((B, 1, S_q, T))
    bias[0, 0, :, 3] = NEG_INF
    cap = 0.5
    y = oracle.attention(q, k, v, bias, nonpad, 1.0, softcap=cap)
    for poison in (np.nan, np.inf, 1e30):
        v2 = v.copy()
        v2[0, :, 3] = poison
        np.testing.assert_array_equal(oracle.attention(q, k, v2, bias, nonpad, 1.0, softcap=cap), y)
    # the weights themselves, from one-hot V rows (V = identity over the keys)
    eye = np.zeros((B, Hkv, T, D))
    eye[0, 0] = np.eye(T)
    w = oracle.attention(q, k, eye, bias, nonpad, 1.0, softcap=cap)   # [B,Hq,S_q,T] = weights
    live = w[0][..., [j for j in range(T) if j != 3]]
    assert np.all(w[0][..., 3] == 0.0)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(live.max(axis=-1) / live.min(axis=-1) <= math.exp(2 * cap) * (1 + 1e-12))
    # without the cap the same scores spread far wider (the bound above is not vacuous)
    w0 = oracle.attention(q, k, eye, bias, nonpad, 1.0)
    live0 = w0[0][..., [j for j in range(T) if j != 3]]
    assert np.any(live0.max(axis=-1) / live0.min(axis=-1) > math.exp(2 * cap))


# --------------------------------------------------------------------------- #
# circular (window-sized) cache: position p in slot p mod C, kv_len = L tokens
# written so far
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("case", _bias_cases("circular_bias_cases.txt"), ids=lambda c: c["name"])
def test_circular_bias_golden(case):
    out = oracle.bias_circular(case["nonpad"], case["q_start"], case["kind"], case["S_q"],
                               case["max_seq"], case["window"])
    assert out.shape == (case["B"], 1, case["S_q"], case["max_seq"])
    assert np.all((out == NEG_INF) | ((out == 0.0) & ~np.signbit(out)))
    assert len(case["expect"]) == case["B"] * case["S_q"]
    for (b, s), want in case["expect"].items():
        assert _mask_str(out[b, 0, s]) == want, (case["name"], b, s)


def _held_positions(L, C):
    """slot -> absolute position held, walking the writes in order (position p
    overwrites slot p % C): an independent statement of the layout."""
    held = {}
    for p in range(L):
        held[p % C] = p
    return held


def test_circular_scatter_matches_numpy_modular_indexing():
    rng = wl.rng_for(900)
    B, H, C, D, S = 3, 2, 7, 4, 5
    cache = rng.standard_normal((B, H, C, D))
    upd = rng.standard_normal((B, H, S, D))
    w = np.array([0, 5, 19], dtype=np.int64)           # no wrap, wrap, several laps
    got = oracle.scatter_circular(cache, upd, w)
    ref = cache.copy()
    for b in range(B):
        ref[b][:, (w[b] + np.arange(S)) % C] = upd[b]
    assert np.array_equal(got, ref)
    # negative positions are dropped, the rest land; S_new = C fills every slot
    w2 = np.array([-2, 3, 0], dtype=np.int64)
    got2 = oracle.scatter_circular(cache, upd, w2)
    ref2 = cache.copy()
    for b in range(B):
        for t in range(S):
            if w2[b] + t >= 0:
                ref2[b][:, (w2[b] + t) % C] = upd[b][:, t]
    assert np.array_equal(got2, ref2)
    full = rng.standard_normal((B, H, C, D))
    got3 = oracle.scatter_circular(cache, full, np.array([4, 4, 4], dtype=np.int64))
    assert np.array_equal(np.sort(got3.reshape(-1)), np.sort(full.reshape(-1)))
    with pytest.raises(ValueError):
        oracle.scatter_circular(cache, rng.standard_normal((B, H, C + 1, D)), w)


@pytest.mark.parametrize("seed", range(8))
def test_circular_bias_is_linear_bias_at_held_positions(seed):
    """The bias of a circular cache at slot j equals the bias of a linear cache
    of the same tokens at the position slot j holds, and is -inf at slots that
    hold no token yet (L < C). Queries anywhere from the oldest held position to
    past the newest, blocks and pads among the held tokens."""
    rng = wl.rng_for(910 + seed)
    for _ in range(12):
        C = int(rng.integers(3, 40))
        L = int(rng.integers(0, 3 * C + 1))
        S_q = int(rng.integers(1, C + 1))
        W = int(rng.integers(-1, C + 3))
        oldest = max(L - C, 0)
        Tl = L + S_q + 4
        klin = np.zeros(Tl, dtype=np.int32)
        klin[oldest:L] = rng.choice([-1, 0, 0, 1, 2], size=L - oldest)
        held = _held_positions(L, C)
        kcirc = rng.integers(-1, 3, size=C).astype(np.int32)    # slots holding no token: any kind
        for j, p in held.items():
            kcirc[j] = klin[p]
        qs = None if rng.random() < 0.3 else np.array([int(rng.integers(oldest, L + 3))], dtype=np.int64)
        circ = oracle.bias_circular([L], qs, kcirc[None], S_q, C, W)
        qs_lin = qs if qs is not None else np.array([max(L - S_q, 0)], dtype=np.int64)
        lin = oracle.bias([L], qs_lin, klin[None], S_q, Tl, W)
        for j in range(C):
            if j in held:
                assert np.array_equal(circ[0, 0, :, j], lin[0, 0, :, held[j]]), (C, L, S_q, W, j)
            else:
                assert np.all(circ[0, 0, :, j] == NEG_INF)


def test_circular_decode_closed_forms():
    """Decode at the newest position, text only: the allowed slots are exactly
    those of the last min(W, L) positions, (L-1-k) mod C; a window wider than
    the cache sees every held slot."""
    for C in (1, 4, 7, 32):
        for L in range(0, 3 * C + 2):
            for W in (1, 2, C - 1, C, C + 5):
                if W <= 0:
                    continue
                row = oracle.bias_circular([L], None, None, 1, C, W)[0, 0, 0]
                want = {(L - 1 - k) % C for k in range(min(W, L))}
                got = {j for j in range(C) if row[j] == 0.0}
                assert got == want, (C, L, W)


@pytest.mark.parametrize("seed", range(4))
def test_circular_attention_is_linear_attention(seed):
    """With room for the window and the chunk (C >= W + S_q - 1) and image
    blocks among the held tokens, attention over a circular cache equals
    attention over the linear cache of the same tokens (the keys are the same,
    in another order); slots holding no token carry NaN and never leak."""
    rng = wl.rng_for(930 + seed)
    B, Hq, Hkv, D = 2, 4, 2, 8
    W, S_q = 5, 3
    C = W + S_q - 1 + int(rng.integers(0, 4))
    Ls = [int(rng.integers(S_q, C)), int(rng.integers(C, 4 * C))]   # not wrapped, wrapped
    Tl = max(Ls) + 1
    q = rng.standard_normal((B, Hq, S_q, D))
    k_lin = rng.standard_normal((B, Hkv, Tl, D))
    v_lin = rng.standard_normal((B, Hkv, Tl, D))
    klin = np.zeros((B, Tl), dtype=np.int32)
    k_c = np.full((B, Hkv, C, D), np.nan)
    v_c = np.full((B, Hkv, C, D), np.nan)
    kcirc = np.zeros((B, C), dtype=np.int32)
    for b, L in enumerate(Ls):
        oldest = max(L - C, 0)
        blk = int(rng.integers(oldest, max(oldest + 1, L - 2)))
        klin[b, blk:min(blk + 3, L)] = 1
        klin[b, oldest] = -1 if L - oldest > 4 else klin[b, oldest]
        for j, p in _held_positions(L, C).items():
            k_c[b, :, j], v_c[b, :, j], kcirc[b, j] = k_lin[b, :, p], v_lin[b, :, p], klin[b, p]
    L_arr = np.array(Ls, dtype=np.int64)
    scale = 1 / math.sqrt(D)
    b_lin = oracle.bias(L_arr, None, klin, S_q, Tl, W)
    y_lin = oracle.attention(q, k_lin, v_lin, b_lin, L_arr, scale)
    b_circ = oracle.bias_circular(L_arr, None, kcirc, S_q, C, W)
    y_circ = oracle.attention(q, k_c, v_c, b_circ, np.minimum(L_arr, C), scale)
    assert np.isfinite(y_circ).all()
    np.testing.assert_allclose(y_circ, y_lin, rtol=0, atol=1e-12)
    assert np.abs(y_lin).max() > 0.1

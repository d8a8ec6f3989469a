"""Independent numpy references used to pin the oracle (tests only).

Nothing here is shared with the oracle's C code: rounding to bf16 is done by a
different method (search in the sorted table of every finite bf16 value), MXFP4
is decoded from the hand-written OCP table in ``tests/golden``, and the block is
evaluated densely over every (token, expert) pair with numpy matmuls.
"""

from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table() -> np.ndarray:
    vals = np.zeros(16, np.float64)
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, v = line.split()
            vals[int(code, 16)] = float(v)
    return vals


# every finite non-negative bf16 value, ascending with its bit pattern
_POS_BITS = np.arange(0x0000, 0x7F80, dtype=np.uint32)
_POS_VALS = (_POS_BITS << 16).view(np.float32).astype(np.float64)
_MAX = _POS_VALS[-1]
_HALF_ULP_TOP = 2.0 ** (127 - 8)  # half the spacing at the top binade


def nearest_bf16_bits(v) -> np.ndarray:
    """Round fp64 values to bf16 by nearest search, ties to even bits."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    hi = np.searchsorted(_POS_VALS, a, side="left").clip(0, len(_POS_VALS) - 1)
    lo = (hi - 1).clip(0, None)
    vh, vl = _POS_VALS[hi], _POS_VALS[lo]
    dh, dl = vh - a, a - vl
    pick_hi = (dh < dl) | ((dh == dl) & ((_POS_BITS[hi] & 1) == 0))
    pick_hi |= a <= vl  # a at or below the lowest candidate
    bits = np.where(pick_hi, _POS_BITS[hi], _POS_BITS[lo]).astype(np.uint32)
    bits = np.where(a == vh, _POS_BITS[hi], bits)
    over = a >= _MAX + _HALF_ULP_TOP  # the tie at the top goes to even (infinity)
    bits = np.where(over, 0x7F80, bits)
    bits = np.where(np.signbit(v), bits | 0x8000, bits)
    bits = np.where(np.isnan(v), 0x7FC0, bits)
    return bits.astype(np.uint16)


def bf16_val(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_mx(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """[..., N, K/2] nibbles + [..., N, K/32] e8m0 -> [..., N, K] fp64."""
    tab = e2m1_table()
    lo = tab[q & 0xF]
    hi = tab[q >> 4]
    el = np.stack([lo, hi], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    scale = np.ldexp(1.0, s.astype(np.int64) - 127)
    scale = np.where(s == 0xFF, np.nan, scale)  # e8m0 0xFF: NaN (OCP MX v1.0)
    v = el * np.repeat(scale, 32, axis=-1)
    # the decoded weight is an fp32 / bf16 operand: magnitudes from 2^128 on
    # (binary32's largest finite value is (2 - 2^-23) 2^127) are infinite
    with np.errstate(invalid="ignore"):
        big = np.abs(v) >= 2.0**128
    return np.where(big, np.copysign(np.inf, v), v)


def silu_hp(g) -> np.ndarray:
    """silu at 50 digits through mpmath, rounded to fp64."""
    import mpmath

    mpmath.mp.dps = 50
    g = np.asarray(g, np.float64)
    out = np.empty_like(g)
    for i, v in np.ndenumerate(g):
        x = mpmath.mpf(float(v))
        out[i] = float(x / (1 + mpmath.exp(-x)))
    return out


def dense_block(inp: dict, ids: np.ndarray | None = None) -> dict:
    """Brute force over every (token, local expert) pair, masked by routing.

    Routing: fp64 logits by matmul, order by a stable argsort of -logits; the
    weights through mpmath's sigmoid. With ``bias_mode`` 1 the bias enters the
    sort key only and the weights use the unbiased logits. ``ids`` overrides
    the routing choice."""
    import mpmath

    cfg = inp["cfg"]
    S, d, E, k, n, I = cfg.S, cfg.d, cfg.E, cfg.topk, cfg.n_local, cfg.I  # noqa: E741
    x = bf16_val(inp["x"])
    logits = x @ inp["wr"].astype(np.float64).T
    key = logits
    if inp.get("bias") is not None:
        key = logits + inp["bias"].astype(np.float64)
        if cfg.bias_mode == 0:
            logits = key
    if ids is None:
        ids = np.argsort(-key, axis=1, kind="stable")[:, :k].astype(np.int32)
    mpmath.mp.dps = 50
    w = np.zeros((S, k), np.float32)
    for t in range(S):
        s = [1 / (1 + mpmath.exp(-mpmath.mpf(float(logits[t, e])))) for e in ids[t]]
        tot = sum(s)
        w[t] = [float(si / tot) if cfg.renorm else float(si) for si in s]
    W13 = decode_mx(inp["w13q"], inp["w13s"])  # [n, 2I, d]
    W2 = decode_mx(inp["w2q"], inp["w2s"])  # [n, d, I]
    gamma = np.ones(d) if inp.get("gamma") is None else bf16_val(inp["gamma"])
    out = np.zeros((S, d), np.float64)
    y_all = np.zeros((S, n, d), np.uint16)
    for el in range(n):
        gu = bf16_val(nearest_bf16_bits(x @ W13[el].T))  # [S, 2I]
        h = bf16_val(nearest_bf16_bits(silu_hp(gu[:, :I]) * gu[:, I:]))
        yb = nearest_bf16_bits(h @ W2[el].T)  # [S, d]
        y_all[:, el] = yb
        y = bf16_val(yb)
        z = y / np.sqrt((y * y).sum(axis=1, keepdims=True) / d + float(np.float32(cfg.eps))) * gamma
        for t in range(S):
            for slot in range(k):
                if ids[t, slot] == cfg.local_base + el:
                    out[t] += float(w[t, slot]) * z[t]
    if cfg.shared_I:  # always-on dense expert, weight 1, no norm
        Is = cfg.shared_I
        gus = bf16_val(nearest_bf16_bits(x @ bf16_val(inp["ws13"]).T))  # [S, 2 Is]
        hs = bf16_val(nearest_bf16_bits(silu_hp(gus[:, :Is]) * gus[:, Is:]))
        out += bf16_val(nearest_bf16_bits(hs @ bf16_val(inp["ws2"]).T))
    return dict(logits=logits, ids=ids, w=w, y_all=y_all, out=out)

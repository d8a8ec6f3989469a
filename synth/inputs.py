"""Seeded input generator (numpy PCG64 streams, one per array).

Every array is drawn from its own stream, ``default_rng([seed, stream_id])``, so
one array can be regenerated without the others and two seeds never share a
stream. Layouts are the canonical row-major ones the C ABI documents:

=========  ====================================  =======
key        shape                                 dtype
=========  ====================================  =======
x          [S, d]                                bf16 bits (uint16)
wr         [E, d]                                float32 (wr_kind)
bias       [E] or None                           float32
w13q       [n_local, 2 I, d / 2]  (2 e2m1/byte)  uint8
w13s       [n_local, 2 I, d / 32] (e8m0)         uint8
w2q        [n_local, d, I / 2]                   uint8
w2s        [n_local, d, I / 32]                  uint8
gamma      [d] or None (None = ones)             bf16 bits
ws13       [2 I_s, d] or None                    bf16 bits
ws2        [d, I_s] or None                      bf16 bits
=========  ====================================  =======

Nibble k of an MXFP4 row sits in byte k // 2, low nibble for even k; scale byte
k // 32 covers elements 32 (k // 32) .. + 32. Nibbles are uniform over 0..15 and
scale bytes uniform over [e8m0_lo, e8m0_hi].
"""

from __future__ import annotations

import numpy as np

from .configs import MoeConfig, ProjConfig

# stream ids: fixed forever so stored seeds keep their meaning
_STREAM = {
    "x": 1,
    "wr": 2,
    "w13q": 3,
    "w13s": 4,
    "w2q": 5,
    "w2s": 6,
    "gamma": 7,
    "ws13": 8,
    "ws2": 9,
    "ffn_in": 10,
    "w_pre": 11,
    "wr_pre": 12,
    "gamma_l": 13,
    "h_raw": 14,
    "partial": 15,
    "w_post": 16,
}


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), _STREAM[name]])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even.

    Used only to draw bf16-valued inputs; NaN is not expected here."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def router_bias(cfg: MoeConfig) -> np.ndarray | None:
    E = cfg.E
    if cfg.bias_kind == "none":
        return None
    if cfg.bias_kind == "local":
        b = np.zeros(E, np.float32)
        b[cfg.local_base : cfg.local_base + cfg.n_local] = cfg.beta
        return b
    if cfg.bias_kind == "zipf":
        # interleaved popularity ranks 1..E (a permutation when E = 256,
        # n_local = 32): local expert j gets rank 8 j + 3
        e = np.arange(E)
        per = max(E // max(cfg.n_local, 1), 1)
        rank = ((per * (e % cfg.n_local) + e // cfg.n_local + 2) % E) + 1
        return (-cfg.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    raise ValueError(f"unknown bias_kind {cfg.bias_kind!r}")


def _mx_values(rng, shape):
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def _mx_scales(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.uint8)


def make_inputs(
    cfg: MoeConfig,
    seed: int = 0,
    *,
    gamma: str = "ones",
    parts: tuple[str, ...] | None = None,
) -> dict:
    """Draw every input of ``cfg`` (or only ``parts``) for ``seed``.

    ``gamma``: "ones" (None is returned: the norm weight is all ones) or
    "random" (1 + 0.1 N(0, 1), rounded to bf16)."""
    want = set(parts) if parts is not None else None

    def need(k):
        return want is None or k in want

    S, d, E, n, I = cfg.S, cfg.d, cfg.E, cfg.n_local, cfg.I  # noqa: E741
    out: dict = {"cfg": cfg, "seed": seed}
    if need("x"):
        out["x"] = f32_to_bf16_bits(
            _rng(seed, "x").standard_normal((S, d), dtype=np.float32) * cfg.x_std
        )
    if need("wr"):
        if cfg.wr_kind == "wide":
            r = _rng(seed, "wr")
            mag = r.uniform(1.0, 2.0, (E, d)) * np.exp2(r.uniform(-40.0, 4.0, (E, d)))
            sign = np.where(r.random((E, d)) < 0.5, -1.0, 1.0)
            keep = r.random((E, d)) >= 0.05
            out["wr"] = (sign * mag * keep).astype(np.float32)
        else:
            out["wr"] = (
                _rng(seed, "wr").standard_normal((E, d), dtype=np.float32) * cfg.wr_std
            ).astype(np.float32)
    if need("bias"):
        out["bias"] = router_bias(cfg)
    if need("w13q"):
        out["w13q"] = _mx_values(_rng(seed, "w13q"), (n, 2 * I, d // 2))
    if need("w13s"):
        out["w13s"] = _mx_scales(
            _rng(seed, "w13s"), (n, 2 * I, d // 32), cfg.e8m0_lo, cfg.e8m0_hi
        )
    if need("w2q"):
        out["w2q"] = _mx_values(_rng(seed, "w2q"), (n, d, I // 2))
    if need("w2s"):
        out["w2s"] = _mx_scales(
            _rng(seed, "w2s"), (n, d, I // 32), cfg.e8m0_lo, cfg.e8m0_hi
        )
    if need("gamma"):
        if gamma == "ones":
            out["gamma"] = None
        elif gamma == "random":
            g = 1.0 + 0.1 * _rng(seed, "gamma").standard_normal(d, dtype=np.float32)
            out["gamma"] = f32_to_bf16_bits(g)
        else:
            raise ValueError(gamma)
    Is = cfg.shared_I
    if need("ws13"):
        out["ws13"] = (
            f32_to_bf16_bits(
                _rng(seed, "ws13").standard_normal((2 * Is, d), dtype=np.float32)
                * cfg.ws_std
            )
            if Is
            else None
        )
    if need("ws2"):
        out["ws2"] = (
            f32_to_bf16_bits(
                _rng(seed, "ws2").standard_normal((d, Is), dtype=np.float32)
                * cfg.ws_std
            )
            if Is
            else None
        )
    return out


def make_proj_inputs(pc: ProjConfig, seed: int = 0, *, gamma: str = "random") -> dict:
    """Inputs of the steps around the block:

    =========  =====================  ==============================
    ffn_in     [S, D]                 bf16 bits, N(0, x_std)
    w_pre      [n_pre, D]             bf16 bits, N(0, w_std)
    wr_pre     [e_router, D]          float32, N(0, wr_std)
    gamma_l    [L] or None            bf16 bits, 1 + 0.1 N(0, 1)
    h_raw      [S, L]                 bf16 bits, N(0, w_std sqrt(D)): a
                                      gathered projection for the norm
    partial    [S, L]                 float32, N(0, partial_std)
    w_post     [n_post, L]            bf16 bits, N(0, w_std)
    =========  =====================  =============================="""
    S, D, L = pc.S, pc.D, pc.L
    out: dict = {"cfg": pc, "seed": seed}
    out["ffn_in"] = f32_to_bf16_bits(_rng(seed, "ffn_in").standard_normal((S, D), dtype=np.float32) * pc.x_std)
    out["w_pre"] = f32_to_bf16_bits(_rng(seed, "w_pre").standard_normal((pc.n_pre, D), dtype=np.float32) * pc.w_std)
    out["wr_pre"] = (
        _rng(seed, "wr_pre").standard_normal((pc.e_router, D), dtype=np.float32) * pc.wr_std
    ).astype(np.float32)
    if gamma == "ones":
        out["gamma_l"] = None
    else:
        out["gamma_l"] = f32_to_bf16_bits(1.0 + 0.1 * _rng(seed, "gamma_l").standard_normal(L, dtype=np.float32))
    std_h = pc.w_std * float(np.sqrt(D))
    out["h_raw"] = f32_to_bf16_bits(_rng(seed, "h_raw").standard_normal((S, L), dtype=np.float32) * std_h)
    out["partial"] = (
        _rng(seed, "partial").standard_normal((S, L), dtype=np.float32) * pc.partial_std
    ).astype(np.float32)
    out["w_post"] = f32_to_bf16_bits(
        _rng(seed, "w_post").standard_normal((pc.n_post, L), dtype=np.float32) * pc.w_std
    )
    return out

"""ctypes wrapper of the C oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The GPU path never does.

Arrays are numpy, in the canonical layouts of ``synth.inputs`` (bf16 as uint16
bit patterns). Every function here is a thin marshalling layer over the C
function of the same name without the ``orc_`` prefix.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from ._build import LIB, build_oracle

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_D = ctypes.c_double


def _declare(L):
    L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f64.restype = _D
    L.orc_f64_to_bf16.argtypes = [_D]
    L.orc_f64_to_bf16.restype = ctypes.c_uint16
    L.orc_e2m1.argtypes = [ctypes.c_uint]
    L.orc_e2m1.restype = _D
    L.orc_e8m0.argtypes = [ctypes.c_uint]
    L.orc_e8m0.restype = _D
    L.orc_mx_elem.argtypes = [_P, _P, ctypes.c_long]
    L.orc_mx_elem.restype = _D
    L.orc_router_logits.argtypes = [_I, _I, _I, _P, _P, _P, _P]
    L.orc_route_weights.argtypes = [_I, _I, _I, _I, _P, _P, _P]
    L.orc_topk.argtypes = [_I, _I, _I, _I, _P, _P, _P]
    L.orc_bucket.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_expert_row.argtypes = [_I, _I, _P, _P, _P, _P, _P, _P, _P, _P]
    L.orc_shared_row.argtypes = [_I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_mx_gate_up.argtypes = [_I, _I, _P, _P, _P, _P, _P]
    L.orc_mx_down.argtypes = [_I, _I, _P, _P, _P, _P]
    L.orc_bf_gate_up.argtypes = [_I, _I, _P, _P, _P, _P]
    L.orc_bf_down.argtypes = [_I, _I, _P, _P, _P]
    L.orc_expert_ffn.argtypes = [_I] * 6 + [_P] * 11
    L.orc_norm_row.argtypes = [_I, _P, _P, _D, _P]
    L.orc_combine.argtypes = [_I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P]
    L.orc_topk_sel.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
    L.orc_dense_proj.argtypes = [_I, _I, _I, _P, _P, _P]
    L.orc_latent_norm.argtypes = [_I, _I, ctypes.c_double, _P, _P, _P]
    L.orc_post_proj.argtypes = [_I, _I, _I, _P, _P, _P]
    L.orc_forward.argtypes = [_I] * 8 + [_F, _I, _I] + [_P] * 20
    L.orc_set_threads.argtypes = [_I]
    L.orc_set_threads.restype = None
    L.orc_max_threads.argtypes = []
    L.orc_max_threads.restype = _I
    for f in (
        "orc_router_logits",
        "orc_route_weights",
        "orc_topk",
        "orc_topk_sel",
        "orc_bucket",
        "orc_expert_row",
        "orc_shared_row",
        "orc_mx_gate_up",
        "orc_mx_down",
        "orc_bf_gate_up",
        "orc_bf_down",
        "orc_expert_ffn",
        "orc_norm_row",
        "orc_combine",
        "orc_dense_proj",
        "orc_latent_norm",
        "orc_post_proj",
        "orc_forward",
    ):
        getattr(L, f).restype = _I


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous, "contiguous numpy array"
    return a.ctypes.data


def _chk(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- threads


def set_threads(n: int) -> None:
    """OpenMP threads of the batch functions (results do not depend on it)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- scalars


def bf16_to_f64(b: int) -> float:
    return lib().orc_bf16_to_f64(int(b))


def f64_to_bf16(v: float) -> int:
    return lib().orc_f64_to_bf16(float(v))


def e2m1(nib: int) -> float:
    return lib().orc_e2m1(int(nib))


def e8m0(x: int) -> float:
    return lib().orc_e8m0(int(x))


def mx_elem(q_row: np.ndarray, s_row: np.ndarray, k: int) -> float:
    q_row = _c(q_row, np.uint8)
    s_row = _c(s_row, np.uint8)
    return lib().orc_mx_elem(_ptr(q_row), _ptr(s_row), int(k))


# ---------------------------------------------------------------- routing


def router_logits(x, wr, bias=None) -> np.ndarray:
    x = _c(x, np.uint16)
    wr = _c(wr, np.float32)
    bias = _c(bias, np.float32)
    S, d = x.shape
    E = wr.shape[0]
    out = np.empty((S, E), np.float64)
    _chk(lib().orc_router_logits(S, d, E, _ptr(x), _ptr(wr), _ptr(bias), _ptr(out)), "router_logits")
    return out


def route_weights(logits, ids, renorm=1) -> np.ndarray:
    logits = _c(logits, np.float64)
    ids = _c(ids, np.int32)
    S, E = logits.shape
    k = ids.shape[1]
    w = np.empty((S, k), np.float32)
    _chk(lib().orc_route_weights(S, E, k, int(renorm), _ptr(logits), _ptr(ids), _ptr(w)), "route_weights")
    return w


def topk(logits, k, renorm=1):
    logits = _c(logits, np.float64)
    S, E = logits.shape
    ids = np.empty((S, k), np.int32)
    w = np.empty((S, k), np.float32)
    _chk(lib().orc_topk(S, E, int(k), int(renorm), _ptr(logits), _ptr(ids), _ptr(w)), "topk")
    return ids, w


def topk_sel(logits, bias, k, renorm=1):
    """Selection-only bias: top-k of logits + bias, weights from the logits."""
    logits = _c(logits, np.float64)
    bias = _c(bias, np.float32)
    S, E = logits.shape
    ids = np.empty((S, k), np.int32)
    w = np.empty((S, k), np.float32)
    _chk(lib().orc_topk_sel(S, E, int(k), int(renorm), _ptr(logits), _ptr(bias), _ptr(ids), _ptr(w)), "topk_sel")
    return ids, w


def bucket(ids, n_local, local_base=0) -> dict:
    ids = _c(ids, np.int32)
    S, k = ids.shape
    kk = min(k, n_local)
    counts = np.empty(n_local, np.int32)
    offsets = np.empty(n_local + 1, np.int32)
    rows = np.empty(max(S * kk, 1), np.int32)
    pick_pos = np.empty((S, k), np.int32)
    active = np.empty(n_local + 1, np.int32)
    _chk(
        lib().orc_bucket(
            S, k, int(n_local), int(local_base), _ptr(ids), _ptr(counts), _ptr(offsets),
            _ptr(rows), _ptr(pick_pos), _ptr(active),
        ),
        "bucket",
    )
    return dict(counts=counts, offsets=offsets, rows=rows[: S * kk], pick_pos=pick_pos, active=active)


# ---------------------------------------------------------------- experts


def expert_row(x_row, w13q_e, w13s_e, w2q_e, w2s_e):
    """One token row (bf16 bits [d]) through one expert -> (gu, h, y) bf16 bits."""
    x_row = _c(x_row, np.uint16)
    w13q_e, w13s_e, w2q_e, w2s_e = (_c(a, np.uint8) for a in (w13q_e, w13s_e, w2q_e, w2s_e))
    d = x_row.shape[0]
    I = w2q_e.shape[1] * 2  # noqa: E741
    gu = np.empty(2 * I, np.uint16)
    h = np.empty(I, np.uint16)
    y = np.empty(d, np.uint16)
    _chk(
        lib().orc_expert_row(
            d, I, _ptr(x_row), _ptr(w13q_e), _ptr(w13s_e), _ptr(w2q_e), _ptr(w2s_e),
            _ptr(gu), _ptr(h), _ptr(y),
        ),
        "expert_row",
    )
    return gu, h, y


def mx_gate_up(x_row, w13q_e, w13s_e):
    """gate_up + SwiGLU of one row through one MXFP4 expert -> (gu, h) bf16 bits."""
    x_row = _c(x_row, np.uint16)
    w13q_e, w13s_e = _c(w13q_e, np.uint8), _c(w13s_e, np.uint8)
    d = x_row.shape[0]
    I = w13q_e.shape[0] // 2  # noqa: E741
    gu = np.empty(2 * I, np.uint16)
    h = np.empty(I, np.uint16)
    _chk(lib().orc_mx_gate_up(d, I, _ptr(x_row), _ptr(w13q_e), _ptr(w13s_e), _ptr(gu), _ptr(h)), "mx_gate_up")
    return gu, h


def mx_down(h_row, w2q_e, w2s_e):
    """down of one SwiGLU row through one MXFP4 expert -> y bf16 bits."""
    h_row = _c(h_row, np.uint16)
    w2q_e, w2s_e = _c(w2q_e, np.uint8), _c(w2s_e, np.uint8)
    d, I = w2q_e.shape[0], h_row.shape[0]  # noqa: E741
    y = np.empty(d, np.uint16)
    _chk(lib().orc_mx_down(d, I, _ptr(h_row), _ptr(w2q_e), _ptr(w2s_e), _ptr(y)), "mx_down")
    return y


def bf_gate_up(x_row, ws13):
    x_row, ws13 = _c(x_row, np.uint16), _c(ws13, np.uint16)
    d, Is = x_row.shape[0], ws13.shape[0] // 2
    gu = np.empty(2 * Is, np.uint16)
    h = np.empty(Is, np.uint16)
    _chk(lib().orc_bf_gate_up(d, Is, _ptr(x_row), _ptr(ws13), _ptr(gu), _ptr(h)), "bf_gate_up")
    return gu, h


def bf_down(h_row, ws2):
    h_row, ws2 = _c(h_row, np.uint16), _c(ws2, np.uint16)
    d, Is = ws2.shape[0], h_row.shape[0]
    y = np.empty(d, np.uint16)
    _chk(lib().orc_bf_down(d, Is, _ptr(h_row), _ptr(ws2), _ptr(y)), "bf_down")
    return y


def shared_row(x_row, ws13, ws2):
    x_row = _c(x_row, np.uint16)
    ws13 = _c(ws13, np.uint16)
    ws2 = _c(ws2, np.uint16)
    d = x_row.shape[0]
    Is = ws2.shape[1]
    gu = np.empty(2 * Is, np.uint16)
    h = np.empty(Is, np.uint16)
    y = np.empty(d, np.uint16)
    _chk(
        lib().orc_shared_row(d, Is, _ptr(x_row), _ptr(ws13), _ptr(ws2), _ptr(gu), _ptr(h), _ptr(y)),
        "shared_row",
    )
    return gu, h, y


def expert_ffn(inp: dict, bk: dict) -> np.ndarray:
    """All bucket rows (and the shared expert) -> y [R_max (+S)][d] bf16 bits.
    Rows past the bucket total are zero."""
    cfg = inp["cfg"]
    S, d, I, n, k, Is = cfg.S, cfg.d, cfg.I, cfg.n_local, cfg.topk, cfg.shared_I  # noqa: E741
    R_max = S * min(k, n)
    y = np.zeros((R_max + (S if Is else 0), d), np.uint16)
    rows = np.ascontiguousarray(np.concatenate([bk["rows"], np.full(1, -1, np.int32)]), np.int32)
    args = [_c(inp[key], np.uint8) for key in ("w13q", "w13s", "w2q", "w2s")]
    _chk(
        lib().orc_expert_ffn(
            S, d, I, n, k, Is, _ptr(_c(inp["x"], np.uint16)), *[_ptr(a) for a in args],
            _ptr(_c(bk["counts"], np.int32)), _ptr(_c(bk["offsets"], np.int32)), _ptr(rows),
            _ptr(_c(inp.get("ws13"), np.uint16)), _ptr(_c(inp.get("ws2"), np.uint16)), _ptr(y),
        ),
        "expert_ffn",
    )
    return y


# ---------------------------------------------------------------- norm + sum


def norm_row(y_row, gamma=None, eps=1e-6) -> np.ndarray:
    y_row = _c(y_row, np.uint16)
    gamma = _c(gamma, np.uint16)
    z = np.empty(y_row.shape[0], np.float64)
    _chk(lib().orc_norm_row(y_row.shape[0], _ptr(y_row), _ptr(gamma), float(eps), _ptr(z)), "norm_row")
    return z


def combine(cfg, y, w, pick_pos, gamma=None) -> np.ndarray:
    y = _c(y, np.uint16)
    w = _c(w, np.float32)
    pick_pos = _c(pick_pos, np.int32)
    gamma = _c(gamma, np.uint16)
    out = np.empty((cfg.S, cfg.d), np.float32)
    _chk(
        lib().orc_combine(
            cfg.S, cfg.d, cfg.topk, cfg.n_local, cfg.shared_I, float(cfg.eps), _ptr(y), _ptr(w),
            _ptr(pick_pos), _ptr(gamma), _ptr(out),
        ),
        "combine",
    )
    return out


def forward(inp: dict) -> dict:
    """The whole block on one set of inputs; returns every intermediate."""
    cfg = inp["cfg"]
    S, d, E, k, n, I, Is = cfg.S, cfg.d, cfg.E, cfg.topk, cfg.n_local, cfg.I, cfg.shared_I  # noqa: E741
    R_max = S * min(k, n)
    logits = np.empty((S, E), np.float64)
    ids = np.empty((S, k), np.int32)
    w = np.empty((S, k), np.float32)
    counts = np.empty(n, np.int32)
    offsets = np.empty(n + 1, np.int32)
    rows = np.empty(max(R_max, 1), np.int32)
    pick_pos = np.empty((S, k), np.int32)
    active = np.empty(n + 1, np.int32)
    y = np.zeros((R_max + (S if Is else 0), d), np.uint16)
    out = np.empty((S, d), np.float32)
    ins = [
        _c(inp["x"], np.uint16), _c(inp["wr"], np.float32), _c(inp.get("bias"), np.float32),
        _c(inp["w13q"], np.uint8), _c(inp["w13s"], np.uint8), _c(inp["w2q"], np.uint8),
        _c(inp["w2s"], np.uint8), _c(inp.get("gamma"), np.uint16), _c(inp.get("ws13"), np.uint16),
        _c(inp.get("ws2"), np.uint16),
    ]
    outs = [logits, ids, w, counts, offsets, rows, pick_pos, active, y, out]
    _chk(
        lib().orc_forward(
            S, d, E, k, n, cfg.local_base, I, cfg.renorm, float(cfg.eps), Is, int(cfg.bias_mode),
            *[_ptr(a) for a in ins], *[_ptr(a) for a in outs],
        ),
        "forward",
    )
    return dict(
        logits=logits, ids=ids, w=w, counts=counts, offsets=offsets, rows=rows[:R_max],
        pick_pos=pick_pos, active=active, y=y, out=out,
    )


# ---------------------------------------------------------------- around the block


def dense_proj(inp, w) -> np.ndarray:
    """bf16 bits [S][K] x bf16 bits [N][K] -> bf16 bits [S][N] (fp64 sums)."""
    inp = _c(inp, np.uint16)
    w = _c(w, np.uint16)
    S, K = inp.shape
    N = w.shape[0]
    out = np.empty((S, N), np.uint16)
    _chk(lib().orc_dense_proj(S, K, N, _ptr(inp), _ptr(w), _ptr(out)), "dense_proj")
    return out


def latent_norm(h_raw, gamma=None, eps=1e-6) -> np.ndarray:
    h_raw = _c(h_raw, np.uint16)
    gamma = _c(gamma, np.uint16)
    S, L = h_raw.shape
    out = np.empty((S, L), np.uint16)
    _chk(lib().orc_latent_norm(S, L, float(eps), _ptr(h_raw), _ptr(gamma), _ptr(out)), "latent_norm")
    return out


def post_proj(partial, w) -> np.ndarray:
    """fp32 [S][K] (rounded to bf16 first) x bf16 bits [N][K] -> bf16 bits [S][N]."""
    partial = _c(partial, np.float32)
    w = _c(w, np.uint16)
    S, K = partial.shape
    N = w.shape[0]
    out = np.empty((S, N), np.uint16)
    _chk(lib().orc_post_proj(S, K, N, _ptr(partial), _ptr(w), _ptr(out)), "post_proj")
    return out

"""moe_decode_layer_router_amd -- local-expert MoE block for AMD MI355X (gfx950).

A thin ctypes binding of ``libmoeblk.so`` (C ABI: ``include/moeblk.h``). The
functions below carry the C entry points' names and only marshal arguments:
torch tensors supply device memory and the current HIP stream, every step of
the block runs in the library's HIP kernels. There is no fallback: without the
built library (or without a GPU) the calls raise.
"""

from __future__ import annotations

import ctypes
import os

from ._build import LIB as _LIB_PATH

__all__ = [
    "MoeDims",
    "MoeError",
    "lib",
    "dims_from",
    "moe_abi_version",
    "moe_status_string",
    "moe_check_dims",
    "moe_packed_mxfp4_bytes",
    "moe_pack_mxfp4",
    "moe_packed_bf16_bytes",
    "moe_pack_bf16",
    "moe_route",
    "moe_route_workspace_bytes",
    "moe_bucket",
    "moe_ffn_workspace_bytes",
    "moe_expert_ffn",
    "moe_combine",
    "moe_forward_workspace_bytes",
    "moe_forward",
    "moe_forward_static",
    "moe_forward_one_launch",
    "MOE_STATIC_SCRATCH_BYTES",
    "MoeProjDims",
    "proj_dims_from",
    "moe_check_proj_dims",
    "moe_packed_dense_bytes",
    "moe_pack_dense",
    "moe_proj_workspace_bytes",
    "moe_pre_expert",
    "moe_latent_norm",
    "moe_post_expert",
    "moe_topk",
    "MOE_W13",
    "MOE_W2",
]

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_UNSUPPORTED = -4
MOE_ERR_WORKSPACE = -5
MOE_ERR_HIP = -6
MOE_W13 = 0
MOE_W2 = 1
MOE_STATIC_SCRATCH_BYTES = 16 << 20  # moe_forward_static's static scratch a GPU


# the layout of moe_dims and the entry points below (MOEBLK_ABI_VERSION)
ABI_VERSION = 4


class MoeDims(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("n_local", ctypes.c_int32),
        ("local_base", ctypes.c_int32),
        ("I", ctypes.c_int32),
        ("renorm", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("shared_I", ctypes.c_int32),
        ("bias_mode", ctypes.c_int32),
    ]

    @property
    def r_max(self) -> int:
        return self.S * min(self.topk, self.n_local)


class MoeProjDims(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("bias_mode", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {moe_status_string(code)} (status {code})")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_DP = ctypes.POINTER(MoeDims)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built: run __graft_entry__.build() or "
                "python -m moe_decode_layer_router_amd._build"
            )
        L = ctypes.CDLL(_LIB_PATH)
        L.moe_abi_version.restype = ctypes.c_int
        if L.moe_abi_version() != ABI_VERSION:
            raise RuntimeError(
                f"{_LIB_PATH} has ABI version {L.moe_abi_version()}, this binding expects "
                f"{ABI_VERSION}: rebuild it"
            )
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_check_dims.argtypes = [_DP]
        L.moe_check_dims.restype = ctypes.c_int
        for f in ("moe_packed_mxfp4_bytes", "moe_packed_bf16_bytes"):
            getattr(L, f).argtypes = [_DP, ctypes.c_int]
            getattr(L, f).restype = ctypes.c_size_t
        L.moe_ffn_workspace_bytes.argtypes = [_DP]
        L.moe_ffn_workspace_bytes.restype = ctypes.c_size_t
        L.moe_pack_mxfp4.argtypes = [_DP, ctypes.c_int, _P, _P, _P, _P]
        L.moe_pack_bf16.argtypes = [_DP, ctypes.c_int, _P, _P, _P]
        L.moe_route_workspace_bytes.argtypes = [_DP]
        L.moe_route_workspace_bytes.restype = ctypes.c_size_t
        L.moe_route.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_bucket.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P]
        L.moe_expert_ffn.argtypes = [_DP] + [_P] * 11 + [ctypes.c_size_t, _P]
        L.moe_combine.argtypes = [_DP, _P, _P, _P, _P, _P, _P]
        L.moe_forward_workspace_bytes.argtypes = [_DP]
        L.moe_forward_workspace_bytes.restype = ctypes.c_size_t
        L.moe_forward.argtypes = [_DP] + [_P] * 19 + [ctypes.c_size_t, _P]
        L.moe_forward_static.argtypes = [_DP] + [_P] * 19 + [_P]
        L.moe_forward_one_launch.argtypes = [_DP] + [_P] * 17 + [ctypes.c_size_t, _P]
        _PD = ctypes.POINTER(MoeProjDims)
        L.moe_check_proj_dims.argtypes = [_PD]
        for f in ("moe_packed_dense_bytes", "moe_proj_workspace_bytes"):
            getattr(L, f).argtypes = [_PD]
            getattr(L, f).restype = ctypes.c_size_t
        L.moe_pack_dense.argtypes = [_PD, _P, _P, _P]
        L.moe_pre_expert.argtypes = [_PD] + [_P] * 7 + [ctypes.c_size_t, _P]
        L.moe_latent_norm.argtypes = [_PD, _P, _P, _P, _P]
        L.moe_post_expert.argtypes = [_PD] + [_P] * 4 + [ctypes.c_size_t, _P]
        L.moe_topk.argtypes = [_DP, _P, _P, _P, _P, _P]
        for f in (
            "moe_pack_mxfp4", "moe_pack_bf16", "moe_route", "moe_bucket", "moe_expert_ffn", "moe_combine",
            "moe_forward", "moe_forward_static", "moe_forward_one_launch", "moe_check_proj_dims", "moe_pack_dense", "moe_pre_expert", "moe_latent_norm",
            "moe_post_expert", "moe_topk",
        ):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def dims_from(cfg) -> MoeDims:
    """MoeDims from an object or dict with the moe_dims field names."""
    get = cfg.get if isinstance(cfg, dict) else (lambda k, dflt=None: getattr(cfg, k, dflt))
    return MoeDims(
        S=get("S"), d=get("d"), E=get("E"), topk=get("topk"), n_local=get("n_local"),
        local_base=get("local_base"), I=get("I"), renorm=get("renorm"), eps=get("eps"),
        shared_I=get("shared_I"), bias_mode=get("bias_mode", 0),
    )


# ---------------------------------------------------------------- marshalling


def _ptr(t) -> int | None:
    """A tensor's device pointer (None -> NULL). Raw ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor is not on a GPU device")
    if not t.is_contiguous():
        raise ValueError("tensor is not contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(fn: str, *args) -> None:
    rc = getattr(lib(), fn)(*args)
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def _d(dims) -> MoeDims:
    return dims if isinstance(dims, MoeDims) else dims_from(dims)


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def moe_check_dims(dims) -> int:
    return lib().moe_check_dims(ctypes.byref(_d(dims)))


def moe_packed_mxfp4_bytes(dims, which: int) -> int:
    return lib().moe_packed_mxfp4_bytes(ctypes.byref(_d(dims)), int(which))


def moe_packed_bf16_bytes(dims, which: int) -> int:
    return lib().moe_packed_bf16_bytes(ctypes.byref(_d(dims)), int(which))


def moe_ffn_workspace_bytes(dims) -> int:
    return lib().moe_ffn_workspace_bytes(ctypes.byref(_d(dims)))


def moe_pack_mxfp4(dims, which, q, scales, packed, stream=None) -> None:
    _call("moe_pack_mxfp4", ctypes.byref(_d(dims)), int(which), _ptr(q), _ptr(scales), _ptr(packed), _stream(stream))


def moe_pack_bf16(dims, which, w, packed, stream=None) -> None:
    _call("moe_pack_bf16", ctypes.byref(_d(dims)), int(which), _ptr(w), _ptr(packed), _stream(stream))


def moe_route_workspace_bytes(dims) -> int:
    return int(lib().moe_route_workspace_bytes(ctypes.byref(_d(dims))))


def moe_route(dims, x, w_router, bias, logits, topk_ids, topk_w, workspace=None, stream=None) -> None:
    """``workspace``: a device tensor of at least moe_route_workspace_bytes
    (None when that is 0)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call(
        "moe_route", ctypes.byref(_d(dims)), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits),
        _ptr(topk_ids), _ptr(topk_w), _ptr(workspace), ctypes.c_size_t(nbytes), _stream(stream),
    )


def moe_bucket(dims, topk_ids, counts, offsets, rows, pick_pos, active, stream=None) -> None:
    _call(
        "moe_bucket", ctypes.byref(_d(dims)), _ptr(topk_ids), _ptr(counts), _ptr(offsets), _ptr(rows),
        _ptr(pick_pos), _ptr(active), _stream(stream),
    )


def moe_expert_ffn(dims, x, w13_packed, w2_packed, counts, offsets, rows, active, ws13_packed,
                   ws2_packed, y, workspace, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _call(
        "moe_expert_ffn", ctypes.byref(_d(dims)), _ptr(x), _ptr(w13_packed), _ptr(w2_packed), _ptr(counts),
        _ptr(offsets), _ptr(rows), _ptr(active), _ptr(ws13_packed), _ptr(ws2_packed), _ptr(y),
        _ptr(workspace), int(workspace_bytes), _stream(stream),
    )


def moe_combine(dims, y, topk_w, pick_pos, gamma, out, stream=None) -> None:
    _call(
        "moe_combine", ctypes.byref(_d(dims)), _ptr(y), _ptr(topk_w), _ptr(pick_pos), _ptr(gamma), _ptr(out),
        _stream(stream),
    )


def moe_forward_workspace_bytes(dims) -> int:
    return lib().moe_forward_workspace_bytes(ctypes.byref(_d(dims)))


def moe_forward(dims, x, w_router, bias, w13_packed, w2_packed, ws13_packed, ws2_packed, gamma, logits,
                topk_ids, topk_w, counts, offsets, rows, pick_pos, active, y, out, workspace,
                workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _call(
        "moe_forward", ctypes.byref(_d(dims)), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w13_packed),
        _ptr(w2_packed), _ptr(ws13_packed), _ptr(ws2_packed), _ptr(gamma), _ptr(logits), _ptr(topk_ids),
        _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(rows), _ptr(pick_pos), _ptr(active), _ptr(y), _ptr(out),
        _ptr(workspace), int(workspace_bytes), _stream(stream),
    )


def moe_forward_one_launch(dims, x, w_router, bias, w13_packed, w2_packed, gamma, logits, topk_ids, topk_w,
                           counts, offsets, rows, pick_pos, active, y, out, workspace, workspace_bytes=None,
                           stream=None) -> None:
    """moe_forward as one launch (S <= 16, d <= 4096, no shared expert)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _call(
        "moe_forward_one_launch", ctypes.byref(_d(dims)), _ptr(x), _ptr(w_router), _ptr(bias),
        _ptr(w13_packed), _ptr(w2_packed), _ptr(gamma), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
        _ptr(counts), _ptr(offsets), _ptr(rows), _ptr(pick_pos), _ptr(active), _ptr(y), _ptr(out),
        _ptr(workspace), int(workspace_bytes), _stream(stream),
    )


def moe_forward_static(dims, x, w_router, bias, w13_packed, w2_packed, ws13_packed, ws2_packed, gamma,
                       logits, topk_ids, topk_w, counts, offsets, rows, pick_pos, active, y, out,
                       wait_error=None, stream=None) -> None:
    """moe_forward on the library's static per-GPU scratch (no workspace)."""
    _call(
        "moe_forward_static", ctypes.byref(_d(dims)), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w13_packed),
        _ptr(w2_packed), _ptr(ws13_packed), _ptr(ws2_packed), _ptr(gamma), _ptr(logits), _ptr(topk_ids),
        _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(rows), _ptr(pick_pos), _ptr(active), _ptr(y), _ptr(out),
        _ptr(wait_error), _stream(stream),
    )


# ---------------------------------------------------------------- around the block


def proj_dims_from(cfg) -> MoeProjDims:
    """MoeProjDims from an object or dict with the moe_proj_dims field names."""
    get = cfg.get if isinstance(cfg, dict) else (lambda k, dflt=None: getattr(cfg, k, dflt))
    return MoeProjDims(
        S=get("S"), K=get("K"), N=get("N"), E=get("E", 0), bias_mode=get("bias_mode", 0), eps=get("eps", 1e-6),
    )


def _pd(dims) -> MoeProjDims:
    return dims if isinstance(dims, MoeProjDims) else proj_dims_from(dims)


def moe_check_proj_dims(dims) -> int:
    return lib().moe_check_proj_dims(ctypes.byref(_pd(dims)))


def moe_packed_dense_bytes(dims) -> int:
    return lib().moe_packed_dense_bytes(ctypes.byref(_pd(dims)))


def moe_pack_dense(dims, w, packed, stream=None) -> None:
    _call("moe_pack_dense", ctypes.byref(_pd(dims)), _ptr(w), _ptr(packed), _stream(stream))


def moe_proj_workspace_bytes(dims) -> int:
    return lib().moe_proj_workspace_bytes(ctypes.byref(_pd(dims)))


def moe_pre_expert(dims, ffn_in, w_packed, w_router, bias, logits, h_raw, workspace, workspace_bytes=None,
                   stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _call(
        "moe_pre_expert", ctypes.byref(_pd(dims)), _ptr(ffn_in), _ptr(w_packed), _ptr(w_router), _ptr(bias),
        _ptr(logits), _ptr(h_raw), _ptr(workspace), int(workspace_bytes), _stream(stream),
    )


def moe_latent_norm(dims, h_raw, gamma, h, stream=None) -> None:
    _call("moe_latent_norm", ctypes.byref(_pd(dims)), _ptr(h_raw), _ptr(gamma), _ptr(h), _stream(stream))


def moe_post_expert(dims, partial, w_packed, out, workspace, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _call(
        "moe_post_expert", ctypes.byref(_pd(dims)), _ptr(partial), _ptr(w_packed), _ptr(out), _ptr(workspace),
        int(workspace_bytes), _stream(stream),
    )


def moe_topk(dims, logits, bias, topk_ids, topk_w, stream=None) -> None:
    _call(
        "moe_topk", ctypes.byref(_d(dims)), _ptr(logits), _ptr(bias), _ptr(topk_ids), _ptr(topk_w),
        _stream(stream),
    )

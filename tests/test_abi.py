"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments with the documented status codes before any HIP call
(no GPU is needed: every call below fails its host-side checks)."""

import ctypes
import os
import re

import pytest

import moe_decode_layer_router_amd as mb
from synth import CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moeblk.h")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced (checks fail first)
MIS = FAKE + 4


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12, names
    L = mb.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert mb.moe_abi_version() == mb.ABI_VERSION == 4
    for code in range(-6, 1):
        s = mb.moe_status_string(code)
        assert s and s != "unknown status"
    assert mb.moe_status_string(-99) == "unknown status"


def dims(**kw):
    base = dict(CONFIGS["s8_uniform"].dims())
    base.update(kw)
    return mb.dims_from(base)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workload_dims_are_valid(name):
    assert mb.moe_check_dims(mb.dims_from(CONFIGS[name])) == mb.MOE_OK


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(S=0), mb.MOE_ERR_SHAPE),
        (dict(S=129), mb.MOE_ERR_SHAPE),
        (dict(d=4000), mb.MOE_ERR_SHAPE),
        (dict(d=64), mb.MOE_ERR_SHAPE),
        (dict(E=0), mb.MOE_ERR_SHAPE),
        (dict(E=257), mb.MOE_ERR_SHAPE),
        (dict(topk=0), mb.MOE_ERR_SHAPE),
        (dict(topk=9), mb.MOE_ERR_SHAPE),
        (dict(E=4, topk=5, n_local=4), mb.MOE_ERR_SHAPE),
        (dict(n_local=0), mb.MOE_ERR_SHAPE),
        (dict(n_local=33), mb.MOE_ERR_SHAPE),
        (dict(local_base=-1), mb.MOE_ERR_SHAPE),
        (dict(local_base=240), mb.MOE_ERR_SHAPE),
        (dict(I=100), mb.MOE_ERR_SHAPE),
        (dict(I=0), mb.MOE_ERR_SHAPE),
        (dict(shared_I=64), mb.MOE_ERR_SHAPE),
        (dict(renorm=2), mb.MOE_ERR_UNSUPPORTED),
        (dict(bias_mode=2), mb.MOE_ERR_UNSUPPORTED),
        (dict(bias_mode=-1), mb.MOE_ERR_UNSUPPORTED),
        (dict(eps=-1.0), mb.MOE_ERR_UNSUPPORTED),
        (dict(eps=float("nan")), mb.MOE_ERR_UNSUPPORTED),
        (dict(S=1, topk=1, n_local=1, E=1, I=128, d=128), mb.MOE_OK),
        (dict(S=128, topk=8, E=256, local_base=224), mb.MOE_OK),
    ],
)
def test_check_dims(kw, code):
    assert mb.moe_check_dims(dims(**kw)) == code


def test_check_dims_null():
    assert mb.lib().moe_check_dims(None) == mb.MOE_ERR_NULL


def test_sizes():
    d = dims()
    assert mb.moe_packed_mxfp4_bytes(d, mb.MOE_W13) == 32 * 4096 * 4096 * 17 // 32
    assert mb.moe_packed_mxfp4_bytes(d, mb.MOE_W2) == 32 * 4096 * 2048 * 17 // 32
    assert mb.moe_packed_mxfp4_bytes(d, 7) == 0
    assert mb.moe_packed_bf16_bytes(d, mb.MOE_W13) == 0  # no shared expert
    d4 = mb.dims_from(CONFIGS["s128_shared"])
    assert mb.moe_packed_bf16_bytes(d4, mb.MOE_W13) == 4096 * 7168 * 2
    assert mb.moe_packed_bf16_bytes(d4, mb.MOE_W2) == 7168 * 2048 * 2
    R = 128 * 8
    assert mb.moe_ffn_workspace_bytes(d4) >= R * 2048 * 2 + 128 * 2048 * 2
    assert mb.moe_ffn_workspace_bytes(dims(S=0)) == 0


def _rc(fn, *args):
    return getattr(mb.lib(), fn)(*args)


def test_route_rejects():
    d = ctypes.byref(dims())
    ok = [FAKE] * 6
    assert _rc("moe_route", None, *ok, None, 0, None) == mb.MOE_ERR_NULL
    assert _rc("moe_route", ctypes.byref(dims(S=0)), *ok, None, 0, None) == mb.MOE_ERR_SHAPE
    for i in (0, 1, 3, 4, 5):  # bias (2) may be NULL
        a = list(ok)
        a[i] = None
        assert _rc("moe_route", d, *a, None, 0, None) == mb.MOE_ERR_NULL, i
    for i in range(6):
        a = list(ok)
        a[i] = MIS
        assert _rc("moe_route", d, *a, None, 0, None) == mb.MOE_ERR_ALIGN, i


def test_route_workspace():
    """S <= 32 needs no scratch; beyond, the router's K parts [P, S, E] fp32
    with P a power of two up to 32 that divides d / 32: every part is a whole
    number of the kernel's 32-K blocks, for every d the dims allow."""
    assert mb.moe_route_workspace_bytes(dims(S=16)) == 0
    assert mb.moe_route_workspace_bytes(dims(S=32)) == 0
    assert mb.moe_route_workspace_bytes(dims(S=0)) == 0
    for S, d, E in ((33, 256, 8), (64, 4096, 256), (128, 7168, 256), (33, 384, 32)):
        n = mb.moe_route_workspace_bytes(dims(S=S, d=d, E=E, n_local=min(E, 8), topk=2))
        P = n // (S * E * 4)
        assert n == P * S * E * 4 or (n - P * S * E * 4) < 256
        assert P >= 1 and P & (P - 1) == 0 and P <= 32 and (d // 32) % P == 0, (S, d, E, P)
    for S in (33, 64, 65, 128):
        for d in range(128, 16385, 128):
            n = mb.moe_route_workspace_bytes(dims(S=S, d=d, E=256, n_local=32, topk=8))
            P = n // (S * 256 * 4)
            assert P >= 1 and P & (P - 1) == 0 and (d // P) % 32 == 0, (S, d, P)
    wd = ctypes.byref(dims(S=64, d=4096, E=256, n_local=32, topk=8))
    need = mb.moe_route_workspace_bytes(dims(S=64, d=4096, E=256, n_local=32, topk=8))
    ok = [FAKE] * 6
    assert _rc("moe_route", wd, *ok, None, need, None) == mb.MOE_ERR_NULL
    assert _rc("moe_route", wd, *ok, MIS, need, None) == mb.MOE_ERR_ALIGN
    assert _rc("moe_route", wd, *ok, FAKE, need - 1, None) == mb.MOE_ERR_WORKSPACE
    # the forward workspace holds the router's scratch and the FFN's
    fd = dims(S=64, d=4096, E=256, n_local=32, topk=8)
    assert mb.moe_forward_workspace_bytes(fd) == need + mb.moe_ffn_workspace_bytes(fd)


def test_bucket_rejects():
    d = ctypes.byref(dims())
    ok = [FAKE] * 6
    assert _rc("moe_bucket", ctypes.byref(dims(topk=0)), *ok, None) == mb.MOE_ERR_SHAPE
    for i in range(6):
        a = list(ok)
        a[i] = None
        assert _rc("moe_bucket", d, *a, None) == mb.MOE_ERR_NULL, i
        a[i] = MIS
        assert _rc("moe_bucket", d, *a, None) == mb.MOE_ERR_ALIGN, i


def test_expert_ffn_rejects():
    d = dims()
    need = mb.moe_ffn_workspace_bytes(d)
    ok = [FAKE] * 7 + [None, None] + [FAKE, FAKE]  # no shared expert: ws13/ws2 may be NULL
    call = lambda dd, a, n=need: _rc("moe_expert_ffn", ctypes.byref(dd), *a, n, None)  # noqa: E731
    assert call(dims(I=100), ok) == mb.MOE_ERR_SHAPE
    for i in (0, 1, 2, 3, 4, 5, 6, 9, 10):
        a = list(ok)
        a[i] = None
        assert call(d, a) == mb.MOE_ERR_NULL, i
        a[i] = MIS
        assert call(d, a) == mb.MOE_ERR_ALIGN, i
    assert call(d, ok, need - 1) == mb.MOE_ERR_WORKSPACE
    d4 = mb.dims_from(CONFIGS["s128_shared"])  # shared expert: its weights are required
    assert call(d4, ok, mb.moe_ffn_workspace_bytes(d4)) == mb.MOE_ERR_NULL
    a = list(ok)
    a[7], a[8] = FAKE, MIS
    assert call(d4, a, mb.moe_ffn_workspace_bytes(d4)) == mb.MOE_ERR_ALIGN


def test_combine_rejects():
    d = ctypes.byref(dims())
    ok = [FAKE, FAKE, FAKE, None, FAKE]  # gamma may be NULL
    assert _rc("moe_combine", None, *ok, None) == mb.MOE_ERR_NULL
    for i in (0, 1, 2, 4):
        a = list(ok)
        a[i] = None
        assert _rc("moe_combine", d, *a, None) == mb.MOE_ERR_NULL, i
    for i in range(5):
        a = list(ok)
        a[i] = MIS
        assert _rc("moe_combine", d, *a, None) == mb.MOE_ERR_ALIGN, i


def test_pack_rejects():
    d = ctypes.byref(dims())
    assert _rc("moe_pack_mxfp4", d, 5, FAKE, FAKE, FAKE, None) == mb.MOE_ERR_UNSUPPORTED
    assert _rc("moe_pack_mxfp4", d, 0, None, FAKE, FAKE, None) == mb.MOE_ERR_NULL
    assert _rc("moe_pack_mxfp4", d, 0, MIS, FAKE, FAKE, None) == mb.MOE_ERR_ALIGN
    assert _rc("moe_pack_bf16", d, 0, FAKE, FAKE, None) == mb.MOE_ERR_UNSUPPORTED  # no shared expert
    d4 = ctypes.byref(mb.dims_from(CONFIGS["s128_shared"]))
    assert _rc("moe_pack_bf16", d4, 0, None, FAKE, None) == mb.MOE_ERR_NULL
    assert _rc("moe_pack_bf16", d4, 1, FAKE, MIS, None) == mb.MOE_ERR_ALIGN


def test_python_binding_refuses_cpu_tensors():
    import torch

    with pytest.raises(ValueError):
        mb.moe_combine(dims(), torch.zeros(4), torch.zeros(4), torch.zeros(4), None, torch.zeros(4))


# ------------------------------------------------------------ around the block


def pdims(**kw):
    base = dict(S=8, K=8192, N=512, E=32, bias_mode=0, eps=1e-6)
    base.update(kw)
    return mb.proj_dims_from(base)


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(), mb.MOE_OK),
        (dict(E=0), mb.MOE_OK),
        (dict(S=128, K=16384, N=16384, E=256), mb.MOE_OK),
        (dict(S=1, K=128, N=64), mb.MOE_OK),
        (dict(S=0), mb.MOE_ERR_SHAPE),
        (dict(S=129), mb.MOE_ERR_SHAPE),
        (dict(K=100), mb.MOE_ERR_SHAPE),
        (dict(K=16512), mb.MOE_ERR_SHAPE),
        (dict(N=32), mb.MOE_ERR_SHAPE),
        (dict(N=96), mb.MOE_ERR_SHAPE),
        (dict(E=-1), mb.MOE_ERR_SHAPE),
        (dict(E=257), mb.MOE_ERR_SHAPE),
        (dict(bias_mode=2), mb.MOE_ERR_UNSUPPORTED),
        (dict(eps=-1.0), mb.MOE_ERR_UNSUPPORTED),
        (dict(eps=float("inf")), mb.MOE_ERR_UNSUPPORTED),
    ],
)
def test_check_proj_dims(kw, code):
    assert mb.moe_check_proj_dims(pdims(**kw)) == code


def test_proj_sizes():
    d = pdims()
    assert mb.moe_packed_dense_bytes(d) == 512 * 8192 * 2
    assert mb.moe_packed_dense_bytes(pdims(N=10)) == 0
    ws = mb.moe_proj_workspace_bytes(d)
    assert ws >= 8 * 512 * 4 + 8 * 8192 * 2 and ws % 256 == 0
    assert mb.moe_proj_workspace_bytes(pdims(S=0)) == 0


def test_proj_calls_reject():
    d = pdims()
    pd = ctypes.byref(d)
    need = mb.moe_proj_workspace_bytes(d)
    # moe_pre_expert(dims, ffn_in, w, w_router, bias, logits, h_raw, ws, bytes, stream)
    ok = [FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE]
    pre = lambda dd, a, n=need: _rc("moe_pre_expert", dd, *a, n, None)  # noqa: E731
    assert pre(None, ok) == mb.MOE_ERR_NULL
    assert pre(ctypes.byref(pdims(K=100)), ok) == mb.MOE_ERR_SHAPE
    for i in (0, 1, 2, 4, 5, 6):
        a = list(ok)
        a[i] = None
        assert pre(pd, a) == mb.MOE_ERR_NULL, i
        a[i] = MIS
        assert pre(pd, a) == mb.MOE_ERR_ALIGN, i
    a = list(ok)
    a[2] = a[4] = None  # with router rows, their weights and logits are required
    assert pre(pd, a) == mb.MOE_ERR_NULL
    assert pre(pd, ok, need - 1) == mb.MOE_ERR_WORKSPACE
    # moe_latent_norm(dims, h_raw, gamma, h, stream)
    nd = ctypes.byref(pdims(N=4096))
    assert _rc("moe_latent_norm", nd, None, None, FAKE, None) == mb.MOE_ERR_NULL
    assert _rc("moe_latent_norm", nd, FAKE, MIS, FAKE, None) == mb.MOE_ERR_ALIGN
    assert _rc("moe_latent_norm", ctypes.byref(pdims(eps=float("nan"))), FAKE, None, FAKE, None) == mb.MOE_ERR_UNSUPPORTED
    # moe_post_expert(dims, partial, w, out, ws, bytes, stream)
    post = lambda a, n=need: _rc("moe_post_expert", pd, *a, n, None)  # noqa: E731
    for i in range(4):
        a = [FAKE] * 4
        a[i] = None
        assert post(a) == mb.MOE_ERR_NULL, i
        a[i] = MIS
        assert post(a) == mb.MOE_ERR_ALIGN, i
    assert post([FAKE] * 4, need - 1) == mb.MOE_ERR_WORKSPACE
    # moe_pack_dense(dims, w, packed, stream)
    assert _rc("moe_pack_dense", pd, None, FAKE, None) == mb.MOE_ERR_NULL
    assert _rc("moe_pack_dense", pd, FAKE, MIS, None) == mb.MOE_ERR_ALIGN
    # moe_topk(dims, logits, bias, ids, w, stream)
    bd = ctypes.byref(dims())
    assert _rc("moe_topk", bd, None, None, FAKE, FAKE, None) == mb.MOE_ERR_NULL
    assert _rc("moe_topk", bd, FAKE, MIS, FAKE, FAKE, None) == mb.MOE_ERR_ALIGN
    assert _rc("moe_topk", ctypes.byref(dims(S=0)), FAKE, None, FAKE, FAKE, None) == mb.MOE_ERR_SHAPE


def test_forward_rejects():
    d = dims()
    need = mb.moe_forward_workspace_bytes(d)
    assert need == mb.moe_ffn_workspace_bytes(d)
    # x, w_router, bias, w13, w2, ws13, ws2, gamma, logits, ids, w, counts,
    # offsets, rows, pick_pos, active, y, out, workspace
    ok = [FAKE, FAKE, None, FAKE, FAKE, None, None, None] + [FAKE] * 11
    call = lambda dd, a, n=need: _rc("moe_forward", ctypes.byref(dd), *a, n, None)  # noqa: E731
    assert call(dims(S=0), ok) == mb.MOE_ERR_SHAPE
    assert call(dims(bias_mode=3), ok) == mb.MOE_ERR_UNSUPPORTED
    for i in [0, 1, 3, 4] + list(range(8, 19)):
        a = list(ok)
        a[i] = None
        assert call(d, a) == mb.MOE_ERR_NULL, i
        a[i] = MIS
        assert call(d, a) == mb.MOE_ERR_ALIGN, i
    for i in (2, 5, 6, 7):  # optional pointers: misaligned is still an error
        a = list(ok)
        a[i] = MIS
        assert call(d, a) == mb.MOE_ERR_ALIGN, i
    assert call(d, ok, need - 1) == mb.MOE_ERR_WORKSPACE
    d4 = mb.dims_from(CONFIGS["s128_shared"])  # a shared expert needs its weights
    assert call(d4, ok, mb.moe_forward_workspace_bytes(d4)) == mb.MOE_ERR_NULL


def test_one_launch_rejects():
    """moe_forward_one_launch: moe_forward's checks, and MOE_ERR_UNSUPPORTED
    outside S <= 16, d <= 4096 without a shared expert (before anything is
    enqueued)."""
    d = dims(S=16, d=4096, shared_I=0)
    need = mb.moe_forward_workspace_bytes(d)
    # x, w_router, bias, w13, w2, gamma, logits, ids, w, counts, offsets,
    # rows, pick_pos, active, y, out, workspace
    ok = [FAKE, FAKE, None, FAKE, FAKE, None] + [FAKE] * 11
    call = lambda dd, a, n=need: _rc("moe_forward_one_launch", ctypes.byref(dd), *a, n, None)  # noqa: E731
    assert call(dims(S=0), ok) == mb.MOE_ERR_SHAPE
    for bad in (dims(S=17, d=4096, shared_I=0), dims(S=16, d=4224, shared_I=0),
                dims(S=8, d=1024, shared_I=256)):
        assert call(bad, ok, mb.moe_forward_workspace_bytes(bad)) == mb.MOE_ERR_UNSUPPORTED
    for i in [0, 1, 3, 4] + list(range(6, 17)):
        a = list(ok)
        a[i] = None
        assert call(d, a) == mb.MOE_ERR_NULL, i
        a[i] = MIS
        assert call(d, a) == mb.MOE_ERR_ALIGN, i
    for i in (2, 5):  # optional pointers: misaligned is still an error
        a = list(ok)
        a[i] = MIS
        assert call(d, a) == mb.MOE_ERR_ALIGN, i
    assert call(d, ok, need - 1) == mb.MOE_ERR_WORKSPACE


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback: with the library missing, the first call raises."""
    import subprocess
    import sys

    code = (
        "import moe_decode_layer_router_amd as mb\n"
        f"mb._LIB_PATH = {str(tmp_path / 'missing.so')!r}\n"
        "try:\n    mb.moe_abi_version()\nexcept RuntimeError as e:\n    print('raised:', e)\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert "raised:" in out.stdout and "is not built" in out.stdout, out.stdout + out.stderr


def test_bench_refuses_several_gpus():
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 2 and "one GPU" in out.stderr, out.stderr

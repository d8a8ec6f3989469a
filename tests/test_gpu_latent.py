"""GPU parity of the steps around the block against the CPU oracle, through
the C ABI: moe_pre_expert (router + this GPU's rows of the pre projection),
moe_latent_norm, moe_post_expert, and moe_topk chaining the pre step's logits
into the block.

Tolerances (tests/gpu_util.py derives the shared ones):

* router logits: the bound of check_logits (the same router kernels);
* projections: per output row, |d| <= 2^-7 |ref| + (K/32 + 64) 2^-24
  sum_k |x_k w_nk| (fp32 MFMA accumulation in K parts, one bf16 rounding that
  may land on the other side of a tie), and >= 99 % of values bit-identical
  (compare_y_step);
* norm: evaluated in fp64 on both sides, so at most one bf16 ulp apart (a
  different fp64 summation order of the squares) and >= 99.9 % identical;
* the whole latent chain (pre -> norm -> top-k -> bucket -> experts ->
  combine -> post): ids exact, and the final rows within 2e-2 of their RMS
  (the ratio is recorded as check_block records its own).
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import PROJ_CONFIGS, ProjConfig, get_config, make_inputs, make_proj_inputs  # noqa: E402
from tests._ref import bf16_val, nearest_bf16_bits  # noqa: E402
from tests.gpu_util import _record_ratio, compare_y_step, to_np  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _steps(inp):
    from moe_decode_layer_router_amd.block import ProjSteps

    st = ProjSteps(inp)
    st.pre()
    st.norm()
    st.post()
    torch.cuda.synchronize()
    return st


def _check_proj_rows(got, ref, x_bits, w_bits, what):
    w = bf16_val(w_bits)
    for t in range(got.shape[0]):
        compare_y_step(got[t], ref[t], x_bits[t], w, f"{what}, token {t}")


def _check_logits(got, x_bits, wr, bias, what):
    lo = oracle.router_logits(x_bits, wr, bias)
    mag = np.abs(bf16_val(x_bits)) @ np.abs(wr.astype(np.float64)).T
    u = 2.0**-24
    tol = (x_bits.shape[1] / 256 + 12) * u * mag + u * np.abs(lo) + 1e-30
    err = np.abs(got.astype(np.float64) - lo)
    assert np.all(err <= tol), f"{what}: logit error {err.max():.3g}"
    return lo


def _check_norm(got, h_raw, gamma, eps, what):
    ref = oracle.latent_norm(h_raw, gamma, eps)
    a = got.astype(np.int32)
    b = ref.astype(np.int32)
    same_sign = ((a ^ b) & 0x8000) == 0
    near = same_sign & (np.abs(a - b) <= 1)  # one ulp = one step of the bit pattern
    assert np.all(near | (a == b)), f"{what}: more than one ulp apart"
    assert np.mean(a == b) >= 0.999, f"{what}: only {np.mean(a == b):.5f} identical"


def _check_all(inp, st):
    pc = inp["cfg"]
    if pc.e_router:
        bias = inp.get("bias_pre") if pc.bias_mode == 0 else None
        _check_logits(to_np(st.logits), inp["ffn_in"], inp["wr_pre"], bias, pc.name)
    ref = oracle.dense_proj(inp["ffn_in"], inp["w_pre"])
    _check_proj_rows(to_np(st.h_raw), ref, inp["ffn_in"], inp["w_pre"], f"{pc.name} h_raw")
    _check_norm(to_np(st.h), inp["h_raw"], inp.get("gamma_l"), pc.eps, f"{pc.name} norm")
    ref = oracle.post_proj(inp["partial"], inp["w_post"])
    p16 = nearest_bf16_bits(inp["partial"].astype(np.float64))  # the post step's bf16 input
    _check_proj_rows(to_np(st.out), ref, p16, inp["w_post"], f"{pc.name} post")


@pytest.mark.parametrize("name", list(PROJ_CONFIGS))
def test_workloads(name):
    inp = make_proj_inputs(PROJ_CONFIGS[name], 0)
    _check_all(inp, _steps(inp))


def _small(**kw):
    base = ProjConfig(name="small", S=8, D=512, L=256, n_pre=128, e_router=16, n_post=192)
    return base.with_(**kw)


EDGE = {
    "S1": _small(S=1),
    "S17_ragged": _small(S=17),
    "S128": _small(S=128, D=1024, L=384, n_pre=320, n_post=64),
    "K128_N64": _small(D=128, L=128, n_pre=64, n_post=64),
    "no_router": _small(e_router=0),
    "K16384": _small(S=3, D=16384, L=256, n_pre=64, e_router=4),
    "sel_bias": _small(bias_mode=1),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name):
    pc = EDGE[name]
    inp = make_proj_inputs(pc, 7, gamma="ones" if name == "S1" else "random")
    rng = np.random.default_rng(1)
    inp["bias_pre"] = (rng.standard_normal(pc.e_router) * 0.3).astype(np.float32) if pc.e_router else None
    _check_all(inp, _steps(inp))


def test_repeated_calls_agree():
    """Back-to-back calls give the same bytes: the part counters return to
    zero within every call, and the partials' region may hold anything."""
    inp = make_proj_inputs(_small(S=20), 2)
    st = _steps(inp)
    first = [to_np(t).copy() for t in (st.logits, st.h_raw, st.h, st.out)]
    for ws, n_out in ((st.ws_pre, st.pc.n_pre), (st.ws_post, st.pc.n_post)):
        n_part = st.pc.S * n_out * 4  # the first part's partials at least
        ws[:n_part].fill_(0x7F)
    for _ in range(2):
        st.pre()
        st.norm()
        st.post()
    torch.cuda.synchronize()
    for a, t in zip(first, (st.logits, st.h_raw, st.h, st.out)):
        assert np.array_equal(a, to_np(t))


@pytest.mark.parametrize("bias_mode", [0, 1])
def test_latent_chain(bias_mode):
    """The latent MoE end to end on one GPU: ffn_in -> router + pre projection
    (all latent rows) -> norm -> moe_topk -> bucket -> expert FFN -> combine ->
    post projection, against the oracle's chain on its own intermediates."""
    from moe_decode_layer_router_amd import moe_latent_norm, moe_topk
    from moe_decode_layer_router_amd.block import MoeBlock, ProjSteps

    cfg = get_config("tiny").with_(S=12, E=8, n_local=8, topk=2, bias_mode=bias_mode)  # experts at d = 256
    pc = ProjConfig(name="chain", S=cfg.S, D=512, L=cfg.d, n_pre=cfg.d, e_router=cfg.E, n_post=384,
                    bias_mode=bias_mode)
    pin = make_proj_inputs(pc, 5)
    bin_ = make_inputs(cfg, 5, gamma="random")
    rng = np.random.default_rng(9)
    pin["bias_pre"] = (rng.standard_normal(cfg.E) * 0.3).astype(np.float32)

    st = ProjSteps(pin)
    blk = MoeBlock(bin_)
    st.pre()
    moe_latent_norm(st.norm_dims, st.h_raw, st.gamma, blk.x)  # the experts' input
    moe_topk(blk.dims, st.logits, st.bias, blk.ids, blk.w)
    blk.bucket()
    blk.expert_ffn()
    blk.combine()
    st.partial.copy_(blk.out)
    st.post()
    torch.cuda.synchronize()
    assert blk.ffn_error() == 0

    # the oracle's chain
    bias = pin["bias_pre"]
    lo = oracle.router_logits(pin["ffn_in"], pin["wr_pre"], bias if bias_mode == 0 else None)
    if bias_mode == 0:
        ids, w = oracle.topk(lo, cfg.topk, cfg.renorm)
    else:
        ids, w = oracle.topk_sel(lo, bias, cfg.topk, cfg.renorm)
    assert np.array_equal(to_np(blk.ids), ids)
    np.testing.assert_allclose(to_np(blk.w), w, rtol=1e-6)
    h = oracle.latent_norm(oracle.dense_proj(pin["ffn_in"], pin["w_pre"]), pin["gamma_l"], pc.eps)
    binp = dict(bin_)
    binp["x"] = h
    bk = oracle.bucket(ids, cfg.n_local, cfg.local_base)
    y = oracle.expert_ffn(binp, bk)
    part = oracle.combine(cfg, y, w, bk["pick_pos"], bin_.get("gamma"))
    ref = bf16_val(oracle.post_proj(part, pin["w_post"]))
    got = bf16_val(to_np(st.out))
    rms = np.sqrt(np.mean(ref * ref))
    ratio = float(np.abs(got - ref).max() / (2e-2 * rms))
    _record_ratio(ratio, int((np.abs(got - ref) > 2e-2 * rms).sum()))
    assert ratio <= 1.0, f"max error {np.abs(got - ref).max():.3g}, rms {rms:.3g}"


def _random_proj(seed):
    """Seeded random sizes inside the supported ranges (small enough for the
    oracle): S, the input and latent widths, the rows held, router rows, bias
    mode."""
    r = np.random.default_rng([seed, 91])
    return _small(
        name=f"random{seed}",
        S=int(r.integers(1, 129)),
        D=128 * int(r.integers(1, 25)),
        L=128 * int(r.integers(1, 9)),
        n_pre=64 * int(r.integers(1, 9)),
        e_router=int(r.integers(0, 65)),
        n_post=64 * int(r.integers(1, 9)),
        bias_mode=int(r.integers(0, 2)),
    )


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes(seed):
    pc = _random_proj(seed)
    inp = make_proj_inputs(pc, 20 + seed)
    rng = np.random.default_rng(seed)
    inp["bias_pre"] = (rng.standard_normal(pc.e_router) * 0.3).astype(np.float32) if pc.e_router else None
    _check_all(inp, _steps(inp))

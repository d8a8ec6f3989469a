"""GPU parity of the HIP block against the CPU oracle, through the C ABI.

Every case draws seeded synthetic inputs, runs route -> bucket -> expert FFN ->
combine on the GPU and checks each step against the oracle on the same bytes
(tests/gpu_util.py states the tolerances). The four named workloads are
compared on every token at full size in the launch configuration the
benchmark times; the other full-size runs (more row counts, moe_forward, the
selection-only bias) compare routing and bucketing everywhere and the expert
chain on sampled tokens, and the one-call path bit for bit against the four
calls."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import get_config, make_inputs  # noqa: E402
from tests._ref import bf16_val  # noqa: E402
from tests.gpu_util import check_block, run_gpu, to_np  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tiny(**kw):
    return get_config("tiny").with_(**kw)


def _unpack_mx(packed, n_loc, N, K, which):
    """Invert the documented packed MXFP4 tile order on the host."""
    RB, NC = N // 64, K // 128
    p = packed.reshape(n_loc, RB, NC, 4352)
    q = np.zeros((n_loc, N, K // 2), np.uint8)
    s = np.zeros((n_loc, N, K // 32), np.uint8)
    half = N // 2
    for rb in range(RB):
        for r in range(4):
            for m in range(16):
                if which == 1:
                    n = 64 * rb + 16 * r + m
                else:
                    i = 32 * rb + 8 * r + 2 * (m // 4) + (m % 2)
                    n = half + i if (m & 2) else i
                for g in range(4):
                    lane = 16 * g + m
                    for c in range(NC):
                        k0 = 128 * c + 32 * g
                        q[:, n, k0 // 2 : k0 // 2 + 16] = p[:, rb, c, r * 1024 + lane * 16 : r * 1024 + lane * 16 + 16]
                        s[:, n, k0 // 32] = p[:, rb, c, 4096 + lane * 4 + r]
    return q, s


def test_pack_mxfp4_is_a_permutation():
    cfg = _tiny()
    inp = make_inputs(cfg, 3)
    from moe_decode_layer_router_amd.block import MoeBlock

    blk = MoeBlock(inp)
    torch.cuda.synchronize()
    q, s = _unpack_mx(to_np(blk.sets[0]["w13"]), cfg.n_local, 2 * cfg.I, cfg.d, 0)
    assert np.array_equal(q, inp["w13q"]) and np.array_equal(s, inp["w13s"])
    q, s = _unpack_mx(to_np(blk.sets[0]["w2"]), cfg.n_local, cfg.d, cfg.I, 1)
    assert np.array_equal(q, inp["w2q"]) and np.array_equal(s, inp["w2s"])


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("gamma", ["ones", "random"])
def test_tiny_block(seed, gamma):
    inp = make_inputs(get_config("tiny"), seed, gamma=gamma)
    check_block(inp, run_gpu(inp))


EDGE = {
    "S1": _tiny(S=1),
    "S13_ragged": _tiny(S=13),
    "S37_k1": _tiny(S=37, topk=1),
    "k_eq_E": _tiny(S=5, E=4, n_local=4, topk=4),
    "eight_local_picks": _tiny(S=12, E=8, n_local=8, topk=8, d=1024),
    "d384_I384": _tiny(S=9, d=384, I=384),
    "d640_I256": _tiny(S=6, d=640, I=256, E=16, n_local=4, local_base=4, topk=3),
    "n_local1": _tiny(S=16, E=8, n_local=1, local_base=3, topk=4),
    "renorm0": _tiny(S=8, renorm=0),
    "E256_uniform_small": _tiny(S=16, d=512, E=256, n_local=32, local_base=32, topk=8, I=256),
    "buckets_gt32": _tiny(S=64, E=8, n_local=8, topk=4),
    "buckets_gt48": _tiny(S=128, E=4, n_local=4, topk=3, d=512, I=256),
    "every_token_both": _tiny(S=128, E=2, n_local=2, topk=2, d=384, I=384),
    "popular_expert_63": _tiny(S=80, E=64, n_local=16, topk=4, bias_kind="zipf", zipf_s=1.5, d=1024),
    "S128_buckets_gt64": _tiny(S=128, E=4, n_local=4, topk=2),
    "shared_small": _tiny(S=20, shared_I=128),
    "shared_S128": _tiny(S=128, E=16, n_local=4, topk=2, shared_I=256, d=256),
    "scales_wide": _tiny(S=8, e8m0_lo=100, e8m0_hi=150),
    "zipf": _tiny(S=48, E=64, n_local=8, local_base=8, topk=8, bias_kind="zipf", zipf_s=1.1),
    "d_max16384": _tiny(S=4, d=16384, I=128),
    "d7168_S33": _tiny(S=33, d=7168, I=128, E=32, n_local=8, topk=8),
    "sel_bias_zipf": _tiny(S=48, E=64, n_local=8, local_base=8, topk=8, bias_kind="zipf", zipf_s=1.1,
                           bias_mode=1),
    "sel_bias_strong": _tiny(S=24, E=16, n_local=4, local_base=4, topk=4, bias_kind="local", beta=3.0,
                             bias_mode=1),
}


@pytest.mark.parametrize("S", [33, 64, 128])
def test_split_router_wide_weights(S):
    """The split router (S > 32) splits each fp32 weight into three bf16 for
    the bf16 MFMA; router weights spread over 44 binades, both signs and exact
    zeros, hold its logits to the same fp32 bound and its top-k to the
    oracle's (check_block)."""
    cfg = _tiny(S=S, d=1024, E=64, n_local=8, local_base=8, topk=4, wr_kind="wide")
    inp = make_inputs(cfg, 21, gamma="random")
    check_block(inp, run_gpu(inp))


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name):
    inp = make_inputs(EDGE[name], 11, gamma="random")
    check_block(inp, run_gpu(inp))


def test_no_local_picks_gives_zero():
    cfg = _tiny(S=12, E=16, n_local=4, local_base=8, topk=2, bias_kind="local", beta=-50.0)
    inp = make_inputs(cfg, 5)
    g = run_gpu(inp)
    assert g["active"][0] == 0 and np.all(g["counts"] == 0)
    assert np.all(g["out"] == 0)
    check_block(inp, g)


def test_deterministic():
    inp = make_inputs(_tiny(S=64, E=8, n_local=8, topk=4), 2)
    g1 = run_gpu(inp)
    g2 = run_gpu(inp, g1["blk"])
    for k in ("logits", "ids", "w", "rows", "y", "out"):
        assert np.array_equal(g1[k], g2[k]), k


def _random_dims(seed):
    """Seeded random problem sizes inside the supported ranges (small d and I,
    so the oracle stays quick)."""
    r = np.random.default_rng([seed, 77])
    E = int(r.integers(1, 65))
    topk = int(r.integers(1, min(8, E) + 1))
    n_local = int(r.integers(1, min(32, E) + 1))
    return dict(
        S=int(r.integers(1, 129)),
        d=128 * int(r.integers(1, 9)),
        E=E,
        topk=topk,
        n_local=n_local,
        local_base=int(r.integers(0, E - n_local + 1)),
        I=128 * int(r.integers(1, 5)),
        renorm=int(r.integers(0, 2)),
        shared_I=[0, 0, 128, 256][int(r.integers(0, 4))],
        bias_kind=["none", "local"][int(r.integers(0, 2))],
        beta=float(r.uniform(-0.5, 0.5)),
        bias_mode=int(r.integers(0, 2)),
    )


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    """Random sizes within the supported ranges: the four calls against the
    oracle, and moe_forward against the four calls bit for bit."""
    kw = _random_dims(seed)
    inp = make_inputs(_tiny(**kw), 100 + seed, gamma="random")
    g = run_gpu(inp)
    check_block(inp, g)
    g1 = run_gpu(inp, g["blk"], fused=True)
    for k in ("logits", "ids", "w", "counts", "offsets", "rows", "pick_pos", "active", "out"):
        assert np.array_equal(g1[k], g[k]), (k, kw)


# ------------------------------------------------------------ full workloads


def _sample_tokens(g, cfg, n):
    """Tokens with local picks first (largest bucket's tokens included)."""
    pp = g["pick_pos"]
    has = [t for t in range(cfg.S) if (pp[t] >= 0).any()]
    big = int(np.argmax(g["counts"]))
    rows = g["rows"][g["offsets"][big] : g["offsets"][big + 1]]
    pick = [int(rows[0]), int(rows[-1])] if len(rows) else []
    for t in has:
        if len(pick) >= n:
            break
        if t not in pick:
            pick.append(t)
    none = [t for t in range(cfg.S) if t not in has]
    return sorted(set(pick + none[:1]))


@pytest.mark.parametrize("name", ["s8_uniform", "s16_local25", "s64_zipf", "s128_shared"])
def test_full_workload(name):
    """Each full workload in the launch configuration the benchmark times,
    every token and every bucket row checked step by step against the oracle,
    end to end within the plain bound."""
    cfg = get_config(name)
    inp = make_inputs(cfg, 0, gamma="random")
    g = run_gpu(inp)
    check_block(inp, g)


@pytest.mark.parametrize("S", [32, 96])
def test_more_row_counts(S):
    """The K5 page's other row counts (S = 32, 96) on the S = 8 workload's
    shapes and routing, through both entry points."""
    cfg = get_config(f"s{S}_uniform")
    inp = make_inputs(cfg, 1, gamma="random")
    g = run_gpu(inp)
    check_block(inp, g, tokens=_sample_tokens(g, cfg, 3))
    g1 = run_gpu(inp, g["blk"], fused=True)
    for k in ("ids", "w", "counts", "rows", "pick_pos", "out"):
        assert np.array_equal(g1[k], g[k]), k


MAX_SIZES = {
    # both intermediate sizes at their limit, S > 32 (split router, 32-row items, the
    # shared expert's 64-token down groups)
    "I8192_shared8192_S33": _tiny(S=33, d=1024, E=64, n_local=8, topk=4, I=8192, shared_I=8192),
    # d at its limit with the shared expert at S > 32 (the combine's register path with
    # the shared row)
    "d16384_shared_S33": _tiny(S=33, d=16384, E=64, n_local=8, topk=4, I=128, shared_I=256),
    # S, d and E at their limits (split router over d = 16384, 128 tokens)
    "S128_d16384_E256": _tiny(S=128, d=16384, E=256, n_local=8, local_base=64, topk=8, I=128),
}


@pytest.mark.parametrize("name", list(MAX_SIZES))
def test_max_sizes(name):
    """The largest sizes moe_check_dims accepts, through the four calls against
    the oracle (every token) and through moe_forward bit for bit."""
    inp = make_inputs(MAX_SIZES[name], 31, gamma="random")
    g = run_gpu(inp)
    check_block(inp, g)
    g1 = run_gpu(inp, g["blk"], fused=True)
    for k in ("logits", "ids", "w", "counts", "offsets", "rows", "pick_pos", "active", "out"):
        assert np.array_equal(g1[k], g[k]), k


# ------------------------------------------------------------ moe_forward

FUSED = {
    "tiny": get_config("tiny"),
    "S13_ragged": _tiny(S=13),
    "buckets_gt32": _tiny(S=64, E=8, n_local=8, topk=4),
    "buckets_gt48": _tiny(S=128, E=4, n_local=4, topk=3, d=512, I=256),
    "every_token_both": _tiny(S=128, E=2, n_local=2, topk=2, d=384, I=384),
    "popular_expert_63": _tiny(S=80, E=64, n_local=16, topk=4, bias_kind="zipf", zipf_s=1.5, d=1024),
    "shared_S128": _tiny(S=128, E=16, n_local=4, topk=2, shared_I=256, d=256),
    "d640_I256": _tiny(S=6, d=640, I=256, E=16, n_local=4, local_base=4, topk=3),
    "d7168_S33": _tiny(S=33, d=7168, I=128, E=32, n_local=8, topk=8),
    "no_local": _tiny(S=12, E=16, n_local=4, local_base=8, topk=2, bias_kind="local", beta=-50.0),
    "S1": _tiny(S=1),
    "some_local": _tiny(S=16, E=32, n_local=4, local_base=8, topk=2),
    "d4096_S16": _tiny(S=16, d=4096, I=256, E=16, n_local=8, topk=4),
    "sel_bias_S16": _tiny(S=16, E=32, n_local=8, topk=4, bias_kind="local", beta=0.5, bias_mode=1),
    "sel_bias_S40": _tiny(S=40, E=64, n_local=8, topk=6, bias_kind="zipf", zipf_s=1.1, bias_mode=1),
}

KEYS = ("logits", "ids", "w", "counts", "offsets", "rows", "pick_pos", "active", "out")


@pytest.mark.parametrize("name", list(FUSED))
def test_fused_equals_four_calls(name):
    """moe_forward computes every value with the same device code as the four
    calls: every output is bit-identical, and both match the oracle. The out
    rows are poisoned in between, so every row must be written again (also
    the zero rows of tokens without a local pick)."""
    inp = make_inputs(FUSED[name], 11, gamma="random")
    g4 = run_gpu(inp)
    g4["blk"].out.fill_(float("nan"))
    g1 = run_gpu(inp, g4["blk"], fused=True)
    for k in KEYS:
        assert np.array_equal(g1[k], g4[k]), k
    R = g4["blk"].dims.r_max
    n = int(g4["offsets"][-1])
    assert np.array_equal(g1["y"][:n], g4["y"][:n])
    if FUSED[name].shared_I:
        assert np.array_equal(g1["y"][R:], g4["y"][R:])
    check_block(inp, g1)


@pytest.mark.parametrize(
    "name,n_tok", [("s8_uniform", 8), ("s16_local25", 4), ("s64_zipf", 3), ("s128_shared", 2)]
)
def test_fused_full_workload(name, n_tok):
    cfg = get_config(name)
    inp = make_inputs(cfg, 0, gamma="random")
    g1 = run_gpu(inp, fused=True)
    check_block(inp, g1, tokens=_sample_tokens(g1, cfg, n_tok))
    g4 = run_gpu(inp, g1["blk"])
    for k in KEYS:
        assert np.array_equal(g1[k], g4[k]), k


@pytest.mark.parametrize("name,n_tok", [("s16_local25", 4), ("s64_zipf", 3)])
def test_selection_bias_workload(name, n_tok):
    """The biased workloads with the bias steering the selection only (the
    other reading of the router bias), through both entry points."""
    cfg = get_config(name).with_(bias_mode=1)
    inp = make_inputs(cfg, 0, gamma="random")
    g1 = run_gpu(inp, fused=True)
    check_block(inp, g1, tokens=_sample_tokens(g1, cfg, n_tok))
    g4 = run_gpu(inp, g1["blk"])
    for k in KEYS:
        assert np.array_equal(g1[k], g4[k]), k


def test_fused_repeated_calls_agree():
    """Back-to-back calls through both entry points agree: the single-launch
    FFN's counters return to zero within every call (S <= 16, no shared
    expert), and the rest of a workspace may hold anything."""
    inp = make_inputs(_tiny(S=16, E=8, n_local=8, topk=4), 3)
    from moe_decode_layer_router_amd.block import MoeBlock
    from moe_decode_layer_router_amd import moe_ffn_workspace_bytes

    blk = MoeBlock(inp)
    # garbage in the SwiGLU rows (the first R_max * I * 2 bytes)
    n_h = blk.dims.r_max * inp["cfg"].I * 2
    assert n_h < moe_ffn_workspace_bytes(blk.dims) - 256
    blk.ws[:n_h].fill_(0xA5)
    blk.fws[:n_h].fill_(0x5A)
    outs = []
    for i in range(6):
        if i % 2:
            blk.forward()
        else:
            blk.step()
        torch.cuda.synchronize()
        assert blk.forward_error() == 0 and blk.ffn_error() == 0
        outs.append(to_np(blk.out))
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


# ------------------------------------------------- moe_forward_one_launch

# S <= 16, d <= 4096, no shared expert: ragged S, one token, tokens without a
# local pick, a token with all 8 picks local (two staged batches in the
# combine), few router rows (E = 8), d = 640 and 4096, the selection-only bias
ONE = {k: FUSED[k] for k in ("tiny", "S13_ragged", "d640_I256", "no_local", "S1", "some_local",
                             "d4096_S16", "sel_bias_S16")}
ONE["eight_local_picks"] = EDGE["eight_local_picks"]
ONE["E8_S16"] = _tiny(S=16, E=8, n_local=8, topk=4)


@pytest.mark.parametrize("name", list(ONE))
def test_one_launch_equals_forward(name):
    """The block as one launch gives moe_forward's outputs bit for bit (the
    same device code computes every value), twice in a row on one workspace
    (its last combine workgroup leaves the control words at zero), and
    matches the oracle."""
    inp = make_inputs(ONE[name], 17, gamma="random")
    gf = run_gpu(inp, fused=True)
    blk = gf["blk"]
    for rep in range(2):
        blk.out.fill_(float("nan"))
        g1 = run_gpu(inp, blk, fused="one")
        for k in KEYS:
            assert np.array_equal(g1[k], gf[k]), (rep, k)
        n = int(gf["offsets"][-1])
        assert np.array_equal(g1["y"][:n], gf["y"][:n]), rep
    check_block(inp, g1)


@pytest.mark.parametrize("name", ["s8_uniform", "s16_local25"])
def test_one_launch_full_workload(name):
    """The S = 8 and S = 16 workloads at full size, one launch against
    moe_forward (itself checked against the oracle at full size), every
    output compared, three calls in a row with moe_forward in between."""
    inp = make_inputs(get_config(name), 0, gamma="random")
    gf = run_gpu(inp, fused=True)
    blk = gf["blk"]
    for rep in range(3):
        g1 = run_gpu(inp, blk, fused="one")
        for k in KEYS:
            assert np.array_equal(g1[k], gf[k]), (rep, k)
        n = int(gf["offsets"][-1])
        assert np.array_equal(g1["y"][:n], gf["y"][:n]), rep
        if rep == 1:  # moe_forward on the workspace the one launch left behind
            g2 = run_gpu(inp, blk, fused=True)
            assert np.array_equal(g2["out"], gf["out"])


# Bucket sizes on both sides of the limits of the routed tasks that stage their
# rows in LDS, in the launches with a shared expert (at most 16 rows, and
# rows x K x 2 bytes at most 64 KiB; at S > 16 48 KiB in gate_up and 32 KiB in
# down), and of the one-token-tile tasks (at most 16 rows): (config, seed,
# the limit). The seeds give buckets on both sides (checked below).
LDSB = {
    # gate_up K = 7168 at S > 16: 3 rows stage, 4 .. 7 do not
    "pair_gate_up_d7168": (_tiny(S=40, d=7168, I=256, E=16, n_local=8, topk=2, shared_I=128), 0, 3),
    # down K = 2048 at S > 16: 8 rows (exactly 32 KiB) stage, 9 .. 13 do not
    "pair_down_I2048_lds": (_tiny(S=36, d=256, I=2048, E=8, n_local=8, topk=2, shared_I=128), 0, 8),
    # down K = 2048: items of 10 .. 16 rows run one token tile, 17 .. 21 two
    "pair_down_I2048": (_tiny(S=64, d=256, I=2048, E=8, n_local=8, topk=2, shared_I=128), 0, 16),
    # 16-row items (S <= 16)
    "pair_S16_d7168": (_tiny(S=16, d=7168, I=256, E=8, n_local=8, topk=2, shared_I=128), 0, 4),
}


@pytest.mark.parametrize("name", list(LDSB))
def test_lds_staged_task_limits(name):
    cfg, seed, lim = LDSB[name]
    inp = make_inputs(cfg, seed, gamma="random")
    g = run_gpu(inp)
    c = g["counts"][g["counts"] > 0]
    assert c.min() <= lim < c.max(), sorted(c.tolist())
    check_block(inp, g)
    # the one-call path takes the same tasks: bit-identical results
    g["blk"].out.fill_(float("nan"))
    gf = run_gpu(inp, g["blk"], fused=True)
    n, R = int(g["offsets"][-1]), g["blk"].dims.r_max
    for k in ("ids", "w", "out"):
        assert np.array_equal(g[k], gf[k]), k
    assert np.array_equal(g["y"][:n], gf["y"][:n])
    if cfg.shared_I:
        assert np.array_equal(g["y"][R:], gf["y"][R:])


# The shared expert's 32-token groups at ragged S (33: a 1-token last group;
# 100: a 4-token one), S = 32 (one group), S = 128 with d = 128 (one K chunk),
# d = 1152 (an odd chunk count) and d = 7168; a second call on the same
# workspace gives the same bits, and so does the one-call path.
SG_GROUPS = {
    "S33_d1152": _tiny(S=33, d=1152, I=128, E=8, n_local=4, topk=2, shared_I=256),
    "S128_d128": _tiny(S=128, d=128, I=128, E=8, n_local=8, topk=2, shared_I=384),
    "S100_d2048": _tiny(S=100, d=2048, I=256, E=16, n_local=4, topk=2, shared_I=128),
    "S64_d7168": _tiny(S=64, d=7168, I=128, E=16, n_local=2, topk=1, shared_I=256),
    "S32_d640": _tiny(S=32, d=640, I=128, E=8, n_local=4, topk=2, shared_I=128),
}


@pytest.mark.parametrize("name", list(SG_GROUPS))
def test_shared_token_groups(name):
    cfg = SG_GROUPS[name]
    inp = make_inputs(cfg, 5, gamma="random")
    g = run_gpu(inp)
    check_block(inp, g)
    R = g["blk"].dims.r_max
    # a second call on the same workspace
    g["blk"].y.fill_(0)
    g2 = run_gpu(inp, g["blk"])
    assert np.array_equal(g["y"][R:], g2["y"][R:])
    assert np.array_equal(g["out"], g2["out"])
    # the one-call path: bit-identical
    g["blk"].out.fill_(float("nan"))
    gf = run_gpu(inp, g["blk"], fused=True)
    assert np.array_equal(g["y"][R:], gf["y"][R:])
    assert np.array_equal(g["out"], gf["out"])


# ------------------------------------------------------------ e8m0 range ends
#
# The decode (v_cvt_scalef32_pk_bf16_fp4) takes the exponent field of its fp32
# scale operand as the e8m0 byte: byte 0 scales by 2^-127 (values down to
# 2^-128, bf16 subnormals), 255 is NaN, and at 253 / 254 the magnitudes from
# 2^128 on become infinite, as the oracle's decode states. The cases put
# every part of the byte range into the expert weights, with activations
# scaled so that the sums stay in range where the case wants finite results.


def _edge_bytes(kind: str, seed: int) -> dict:
    two = 2.0**-8
    base = dict(S=8, d=256, E=8, n_local=8, topk=2, I=128)
    if kind in ("low_gate_high_up", "high_gate_low_up"):
        cfg = _tiny(**base, x_std=two, wr_std=0.02 / two, eps=0.0)
    elif kind == "top_finite":
        cfg = _tiny(**base, x_std=2.0**-20, wr_std=0.02 * 2.0**20)
    else:  # 16 experts, 8 of them local: some tokens avoid the special ones
        cfg = _tiny(**dict(base, S=16, E=16))
    inp = make_inputs(cfg, seed, gamma="random")
    r = np.random.default_rng([seed, 991])
    n, I, d = cfg.n_local, cfg.I, cfg.d
    w13s, w2s = inp["w13s"].copy(), inp["w2s"].copy()
    w13q, w2q = inp["w13q"].copy(), inp["w2q"].copy()
    if kind == "low_gate_high_up":  # tiny gates times huge ups
        w13s[:, :I] = r.integers(0, 4, (n, I, d // 32))
        w13s[:, I:] = r.integers(249, 253, (n, I, d // 32))
        w2s[:] = r.integers(0, 4, w2s.shape)  # y on the bf16 subnormal grid
    elif kind == "high_gate_low_up":
        w13s[:, :I] = r.integers(249, 253, (n, I, d // 32))
        w13s[:, I:] = r.integers(0, 4, (n, I, d // 32))
        w2s[:] = r.integers(0, 4, w2s.shape)
    elif kind == "top_finite":  # 250..254 in down; codes kept below 2^128
        w2s[:] = r.integers(250, 255, w2s.shape)
        blk = np.repeat(w2s, 16, axis=-1)  # the scale byte of every code byte
        for lim, byte in ((5, 253), (3, 254)):  # largest e2m1 magnitude index
            for sh in (0, 4):
                nib = (w2q >> sh) & 0xF
                mag = np.minimum(nib & 7, lim)
                nib2 = (nib & 8) | mag
                keep = blk != byte
                w2q = np.where(keep, w2q, (w2q & ~np.uint8(0xF << sh)) | (nib2 << sh).astype(np.uint8))
    elif kind == "inf_nan":
        w2s[0, 5, 0] = 255  # NaN block in expert 0's output column 5
        w2s[1, 9, 1] = 254  # one infinite weight in expert 1's column 9: y = +-inf there
        w2q[1, 9, 16:32] = 0
        w2q[1, 9, 16] = 0x06  # element 32: 4 x 2^127
        w13s[2, 3, 0] = 255  # NaN gate of expert 2, intermediate 3
        w13s[3, I + 7, 2] = 253  # infinite up weights of expert 3, intermediate 7
    else:
        raise ValueError(kind)
    inp.update(w13s=w13s.astype(np.uint8), w2s=w2s.astype(np.uint8), w13q=w13q, w2q=w2q)
    return inp


def _same_class(a, b, what):
    """NaN where the other is NaN, the same infinities; returns the finite mask."""
    assert np.array_equal(np.isnan(a), np.isnan(b)), f"{what}: NaN positions differ"
    ia, ib = np.isinf(a), np.isinf(b)
    assert np.array_equal(ia, ib) and np.array_equal(a[ia], b[ib]), f"{what}: infinities differ"
    return np.isfinite(b)


@pytest.mark.parametrize("kind", ["low_gate_high_up", "high_gate_low_up", "top_finite"])
def test_scale_bytes_range_ends_finite(kind):
    """Bytes 0..3 and 249..254 in the expert weights with finite results: the
    whole block against the oracle (both entry points)."""
    inp = _edge_bytes(kind, 21)
    g = run_gpu(inp)
    check_block(inp, g)
    g1 = run_gpu(inp, g["blk"], fused=True)
    for k in ("ids", "w", "counts", "rows", "pick_pos", "out"):
        assert np.array_equal(g1[k], g[k]), k


def test_scale_bytes_nan_and_inf():
    """Byte 255 (NaN) and bytes 253 / 254 with codes of magnitude >= 2^128 in
    the expert weights: NaNs and infinities land where the oracle puts them,
    step by step, and the finite values agree as usual."""
    from tests._ref import decode_mx
    from tests.gpu_util import check_bucket, check_logits, check_topk, gpu_h

    inp = _edge_bytes("inf_nan", 22)
    cfg = inp["cfg"]
    g = run_gpu(inp)
    lo = check_logits(inp, g)
    check_topk(inp, g, lo)
    bk = check_bucket(inp, g)
    h_all, _ = gpu_h(g, cfg)
    n_special = 0
    for r in range(int(bk["offsets"][-1])):
        el = int(np.searchsorted(bk["offsets"], r, side="right") - 1)
        t = int(bk["rows"][r])
        _, h_o = oracle.mx_gate_up(inp["x"][t], inp["w13q"][el], inp["w13s"][el])
        a, b = bf16_val(h_all[r]), bf16_val(h_o)
        fin = _same_class(a, b, f"h of row {r}")
        n_special += int((~fin).sum())
        rms = np.sqrt(np.mean(b[fin] ** 2))
        assert np.all(np.abs(a - b)[fin] <= 2.0**-6 * np.abs(b[fin]) + 2.0**-10 * rms + 2.0**-133)
        y_ref = oracle.mx_down(h_all[r], inp["w2q"][el], inp["w2s"][el])
        a, b = bf16_val(g["y"][r]), bf16_val(y_ref)
        fin = _same_class(a, b, f"y of row {r}")
        n_special += int((~fin).sum())
        w = decode_mx(inp["w2q"][el], inp["w2s"][el])
        hv = bf16_val(h_all[r])
        with np.errstate(invalid="ignore"):
            mag = np.abs(w) @ np.abs(np.where(np.isfinite(hv), hv, 0.0))
        tol = 2.0**-7 * np.abs(b) + (cfg.I / 32 + 64) * 2.0**-24 * mag + 2.0**-133
        assert np.all(np.abs(a - b)[fin] <= tol[fin]), f"y of row {r}"
    assert n_special > 0, "the case must produce NaNs and infinities"
    out_c = oracle.combine(cfg, g["y"], g["w"], g["pick_pos"], inp.get("gamma"))
    fin = _same_class(g["out"].astype(np.float64), out_c.astype(np.float64), "out (combine)")
    rms = np.sqrt(np.mean(out_c[fin].astype(np.float64) ** 2))
    assert np.all(np.abs(g["out"] - out_c)[fin] <= 1e-5 * rms)
    ref = oracle.forward(inp)
    fin = _same_class(g["out"].astype(np.float64), ref["out"].astype(np.float64), "out (end to end)")
    rms = np.sqrt(np.mean(ref["out"][fin].astype(np.float64) ** 2))
    assert np.all(np.abs(g["out"] - ref["out"])[fin] <= 2e-2 * rms)

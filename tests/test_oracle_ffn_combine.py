"""Pins of the oracle's expert FFN, per-pick norm and weighted sum.

* the whole tiny block against a dense brute force over every (token, expert)
  pair (tests/_ref.py: numpy matmuls, table decode, nearest-search rounding,
  mpmath sigmoid);
* closed forms: all-ones weights, one-hot rows (gate/up order, nibble order,
  down row selection), scale-byte shifts multiply by exact powers of two;
* norm: constant rows, power-of-two scale invariance with eps = 0;
* combine: k = 1 and w = 1 returns the normalised row; slot order; the shared
  expert's row is added unnormalised; tokens without a local pick are zero.
"""

import math

import numpy as np
import pytest

import oracle
from synth import get_config, make_inputs, f32_to_bf16_bits
from tests._ref import bf16_val, dense_block, nearest_bf16_bits, silu_hp


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("gamma", ["ones", "random"])
def test_tiny_block_equals_dense_brute_force(seed, gamma):
    cfg = get_config("tiny")
    inp = make_inputs(cfg, seed, gamma=gamma)
    got = oracle.forward(inp)
    ref = dense_block(inp)
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.array_equal(got["w"], ref["w"])
    # every bucket row's y equals the dense evaluation of that (token, expert)
    for el in range(cfg.n_local):
        o, c = got["offsets"][el], got["counts"][el]
        for r in range(o, o + c):
            t = got["rows"][r]
            assert np.array_equal(got["y"][r], ref["y_all"][t, el]), (el, t)
    np.testing.assert_allclose(got["out"], ref["out"], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize(
    "kw",
    [
        dict(S=6, E=16, n_local=4, local_base=8, topk=3, renorm=0),
        dict(S=5, E=12, n_local=3, local_base=3, topk=4, bias_kind="local", beta=0.3),
        dict(S=4, E=8, n_local=8, topk=2, shared_I=128),
        dict(S=7, E=16, n_local=4, local_base=12, topk=2, shared_I=256),
        dict(S=6, E=16, n_local=8, topk=4, bias_kind="local", beta=0.3, bias_mode=1),
        dict(S=8, E=32, n_local=8, local_base=8, topk=3, bias_kind="zipf", zipf_s=1.1, bias_mode=1),
    ],
)
def test_block_equals_dense_brute_force_general(kw):
    """Non-local picks, a local range not at 0, renorm off, a routing bias (in
    the logit, or steering the selection only) and the shared expert, against
    the independent dense evaluation."""
    cfg = get_config("tiny").with_(**kw)
    inp = make_inputs(cfg, 4, gamma="random")
    got = oracle.forward(inp)
    ref = dense_block(inp)
    assert np.array_equal(got["ids"], ref["ids"])
    assert np.array_equal(got["w"], ref["w"])
    np.testing.assert_allclose(got["out"], ref["out"], rtol=1e-6, atol=1e-6)


def _one_expert(d=256, I=128, seed=0):  # noqa: E741
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal(d, dtype=np.float32))
    w13q = np.zeros((2 * I, d // 2), np.uint8)
    w13s = np.full((2 * I, d // 32), 127, np.uint8)
    w2q = np.zeros((d, I // 2), np.uint8)
    w2s = np.full((d, I // 32), 127, np.uint8)
    return x, w13q, w13s, w2q, w2s


def _set_nib(q, row, k, nib):
    b = q[row, k // 2]
    q[row, k // 2] = (b & 0xF0) | nib if k % 2 == 0 else (b & 0x0F) | (nib << 4)


def test_all_ones_weights_closed_form():
    d, I = 256, 128  # noqa: E741
    x, w13q, w13s, w2q, w2s = _one_expert(d, I)
    w13q[:] = 0x22  # every element 1.0
    w2q[:] = 0x22
    gu, h, y = oracle.expert_row(x, w13q, w13s, w2q, w2s)
    sx = math.fsum(bf16_val(x))
    g = nearest_bf16_bits(sx)
    assert np.all(gu == g)
    gv = bf16_val(g)
    hh = nearest_bf16_bits(silu_hp(gv) * gv)
    assert np.all(h == hh)
    assert np.all(y == nearest_bf16_bits(I * bf16_val(hh)))


def test_one_hot_rows_pin_gate_up_order_and_indexing():
    d, I = 256, 128  # noqa: E741
    x, w13q, w13s, w2q, w2s = _one_expert(d, I, seed=5)
    rng = np.random.default_rng(11)
    ja = rng.integers(0, d, I)  # gate row i reads x[ja[i]]
    jb = rng.integers(0, d, I)  # up row I+i reads x[jb[i]]
    for i in range(I):
        _set_nib(w13q, i, int(ja[i]), 0x2)
        _set_nib(w13q, I + i, int(jb[i]), 0x2)
    ic = rng.integers(0, I, d)  # down row c reads h[ic[c]], scaled by -2
    for c in range(d):
        _set_nib(w2q, c, int(ic[c]), 0xC)
    gu, h, y = oracle.expert_row(x, w13q, w13s, w2q, w2s)
    assert np.array_equal(gu[:I], x[ja]) and np.array_equal(gu[I:], x[jb])
    want_h = nearest_bf16_bits(silu_hp(bf16_val(x[ja])) * bf16_val(x[jb]))
    assert np.array_equal(h, want_h)
    assert np.array_equal(y, nearest_bf16_bits(-2.0 * bf16_val(h[ic])))


@pytest.mark.parametrize("m", [1, 3, -4])
def test_scale_shift_is_exact_power_of_two(m):
    cfg = get_config("tiny")
    inp = make_inputs(cfg, 4)
    e = 2
    x = inp["x"][0]
    args = [inp[k][e] for k in ("w13q", "w13s", "w2q", "w2s")]
    gu0, _, _ = oracle.expert_row(x, *args)
    s2 = (args[1].astype(np.int64) + m).astype(np.uint8)
    gu1, _, _ = oracle.expert_row(x, args[0], s2, args[2], args[3])
    v0, v1 = bf16_val(gu0), bf16_val(gu1)
    assert np.array_equal(v1, v0 * 2.0**m)


def test_norm_constant_row_closed_form():
    d = 512
    c = 3.0
    y = np.full(d, f32_to_bf16_bits(np.float32(c)), np.uint16)
    z = oracle.norm_row(y, None, 1e-6)
    assert np.allclose(z, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    g = f32_to_bf16_bits(np.linspace(0.5, 1.5, d, dtype=np.float32))
    zg = oracle.norm_row(y, g, 1e-6)
    assert np.allclose(zg, c / math.sqrt(c * c + 1e-6) * bf16_val(g), rtol=1e-15)


def test_norm_scale_invariance_without_eps():
    rng = np.random.default_rng(2)
    y = f32_to_bf16_bits(rng.standard_normal(256, dtype=np.float32))
    y8 = f32_to_bf16_bits(bf16_val(y).astype(np.float32) * 8)
    z1 = oracle.norm_row(y, None, 0.0)
    z8 = oracle.norm_row(y8, None, 0.0)
    assert np.array_equal(z1, z8)
    assert abs(np.mean(z1 * z1) - 1.0) < 1e-12


def test_combine_slot_order_shared_and_empty_tokens():
    cfg = get_config("tiny").with_(S=3, topk=2, n_local=4, shared_I=128)
    d = cfg.d
    R_max = cfg.S * min(cfg.topk, cfg.n_local)
    rng = np.random.default_rng(9)
    y = f32_to_bf16_bits(rng.standard_normal((R_max + cfg.S, d), dtype=np.float32))
    w = np.array([[0.75, 0.25], [1.0, 0.5], [0.3, 0.7]], np.float32)
    pick_pos = np.array([[2, 0], [-1, 5], [-1, -1]], np.int32)
    out = oracle.combine(cfg, y, w, pick_pos)
    z = [oracle.norm_row(y[r], None, float(np.float32(cfg.eps))) for r in range(R_max)]
    sh = bf16_val(y[R_max:])
    want0 = (0.75 * z[2] + 0.25 * z[0] + sh[0]).astype(np.float32)
    want1 = (0.5 * z[5] + sh[1]).astype(np.float32)
    assert np.array_equal(out[0], want0)
    assert np.array_equal(out[1], want1)
    assert np.array_equal(out[2], sh[2].astype(np.float32))
    cfg0 = cfg.with_(shared_I=0)
    out0 = oracle.combine(cfg0, y[:R_max], w, pick_pos)
    assert np.all(out0[2] == 0)
    assert np.array_equal(out0[1], (0.5 * z[5]).astype(np.float32))


def test_combine_k1_returns_normalised_row():
    cfg = get_config("tiny").with_(S=2, topk=1, n_local=8)
    rng = np.random.default_rng(1)
    y = f32_to_bf16_bits(rng.standard_normal((2, cfg.d), dtype=np.float32))
    out = oracle.combine(cfg, y, np.ones((2, 1), np.float32), np.array([[1], [0]], np.int32))
    assert np.array_equal(out[0], oracle.norm_row(y[1], None, float(np.float32(cfg.eps))).astype(np.float32))


def test_shared_row_matches_dense_numpy():
    rng = np.random.default_rng(4)
    d, Is = 256, 128
    x = f32_to_bf16_bits(rng.standard_normal(d, dtype=np.float32))
    ws13 = f32_to_bf16_bits(rng.standard_normal((2 * Is, d), dtype=np.float32) * 0.05)
    ws2 = f32_to_bf16_bits(rng.standard_normal((d, Is), dtype=np.float32) * 0.05)
    gu, h, y = oracle.shared_row(x, ws13, ws2)
    g = nearest_bf16_bits(bf16_val(ws13) @ bf16_val(x))
    assert np.array_equal(gu, g)
    hh = nearest_bf16_bits(silu_hp(bf16_val(g[:Is])) * bf16_val(g[Is:]))
    assert np.array_equal(h, hh)
    assert np.array_equal(y, nearest_bf16_bits(bf16_val(ws2) @ bf16_val(hh)))


def test_thread_count_does_not_change_results():
    """The batch functions split independent outputs over threads; each value
    is computed by one thread in the written order, so 1 thread and many
    threads give the same bits."""
    from synth import get_config, make_inputs

    inp = make_inputs(get_config("tiny").with_(S=24, E=16, n_local=8, topk=4, shared_I=128), 4,
                      gamma="random")
    n = oracle.max_threads()
    try:
        oracle.set_threads(1)
        a = oracle.forward(inp)
        oracle.set_threads(max(n, 4))
        b = oracle.forward(inp)
    finally:
        oracle.set_threads(n)
    for k in ("logits", "ids", "w", "rows", "y", "out"):
        assert np.array_equal(a[k], b[k]), k

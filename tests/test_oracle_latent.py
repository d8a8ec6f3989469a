"""Pins of the oracle's steps around the block: the dense latent projections
(pre_expert_proj, post_expert_proj) and the latent norm (pre_expert_norm).

* projections against numpy's fp64 matmul rounded by nearest search
  (tests/_ref.py), and closed forms: one-hot weight rows return input
  elements, all-ones rows return row sums;
* the post projection's bf16 hand-off: hand-picked fp32 inputs at and
  between bf16 ties, through one-hot rows;
* the norm against 50-digit mpmath, a constant-row closed form and exact
  scale invariance without eps.
"""

import mpmath
import numpy as np
import pytest

import oracle
from synth import PROJ_CONFIGS, f32_to_bf16_bits, make_proj_inputs
from tests._ref import bf16_val, nearest_bf16_bits


def _bf16(rng, shape, std=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


@pytest.mark.parametrize("S,K,N", [(1, 128, 64), (5, 384, 128), (16, 1024, 192)])
def test_dense_proj_against_numpy(S, K, N):
    rng = np.random.default_rng([S, K, N])
    x = _bf16(rng, (S, K))
    w = _bf16(rng, (N, K), 0.05)
    got = oracle.dense_proj(x, w)
    want = nearest_bf16_bits(bf16_val(x) @ bf16_val(w).T)
    assert np.array_equal(got, want)


def test_dense_proj_one_hot_and_ones():
    rng = np.random.default_rng(7)
    S, K = 4, 256
    x = _bf16(rng, (S, K))
    sel = [0, 5, 255, 17]
    w = np.zeros((len(sel), K), np.uint16)
    for n, k in enumerate(sel):
        w[n, k] = 0x3F80  # 1.0
    assert np.array_equal(oracle.dense_proj(x, w), x[:, sel])
    ones = np.full((2, K), 0x3F80, np.uint16)
    got = oracle.dense_proj(x, ones)
    want = nearest_bf16_bits(bf16_val(x).sum(axis=1))
    assert np.array_equal(got, np.stack([want, want], axis=1))


def test_post_proj_rounds_the_partial_to_bf16():
    """fp32 partials at bf16 ties and between them, picked out by one-hot rows:
    1 + 2^-8 ties between 1 and 1 + 2^-7 and goes to even (1.0);
    1 + 3 * 2^-8 ties between 1 + 2^-7 and 1 + 2^-6 and goes to 1 + 2^-6;
    1 + 2^-8 + 2^-20 is past the tie and goes up to 1 + 2^-7."""
    vals = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, 1 + 2.0**-8 + 2.0**-20, -(1 + 2.0**-8)], np.float32)
    K = 128
    partial = np.zeros((1, K), np.float32)
    partial[0, : len(vals)] = vals
    w = np.zeros((len(vals), K), np.uint16)
    for n in range(len(vals)):
        w[n, n] = 0x3F80
    got = bf16_val(oracle.post_proj(partial, w))[0]
    assert got.tolist() == [1.0, 1 + 2.0**-6, 1 + 2.0**-7, -1.0]


def test_post_proj_equals_dense_proj_of_rounded_input():
    rng = np.random.default_rng(3)
    partial = rng.standard_normal((6, 256)).astype(np.float32)
    w = _bf16(rng, (128, 256), 0.05)
    x16 = nearest_bf16_bits(partial.astype(np.float64))
    assert np.array_equal(oracle.post_proj(partial, w), oracle.dense_proj(x16, w))
    want = nearest_bf16_bits(bf16_val(x16) @ bf16_val(w).T)
    assert np.array_equal(oracle.post_proj(partial, w), want)


def test_latent_norm_against_mpmath():
    rng = np.random.default_rng(11)
    S, L, eps = 3, 192, 1e-6
    h = _bf16(rng, (S, L), 1.8)
    g = f32_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(L).astype(np.float32))
    got = oracle.latent_norm(h, g, eps)
    mpmath.mp.dps = 50
    hv, gv = bf16_val(h), bf16_val(g)
    for t in range(S):
        ss = mpmath.fsum(mpmath.mpf(float(v)) ** 2 for v in hv[t])
        r = 1 / mpmath.sqrt(ss / L + mpmath.mpf(eps))
        want = nearest_bf16_bits(np.array([float(mpmath.mpf(float(a)) * r * mpmath.mpf(float(b))) for a, b in zip(hv[t], gv)]))
        assert np.array_equal(got[t], want), t


def test_latent_norm_constant_row_and_scale_invariance():
    L = 256
    c = 0x4040  # 3.0
    h = np.full((1, L), c, np.uint16)
    got = bf16_val(oracle.latent_norm(h, None, 1e-6))[0]
    want = bf16_val(nearest_bf16_bits(np.array([3.0 / np.sqrt(9.0 + 1e-6)])))[0]
    assert np.all(got == want)
    rng = np.random.default_rng(5)
    h = _bf16(rng, (4, L))
    scaled = f32_to_bf16_bits(bf16_val(h).astype(np.float32) * np.float32(8.0))  # exact: power of two
    assert np.array_equal(oracle.latent_norm(h, None, 0.0), oracle.latent_norm(scaled, None, 0.0))


def test_workload_shapes():
    inp = make_proj_inputs(PROJ_CONFIGS["latent_s8"], 0)
    pc = inp["cfg"]
    assert inp["ffn_in"].shape == (pc.S, pc.D) and inp["w_pre"].shape == (512, 8192)
    assert inp["wr_pre"].shape == (32, 8192) and inp["w_post"].shape == (1024, 4096)

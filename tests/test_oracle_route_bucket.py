"""Pins of the oracle's routing (logits, top-k, weights) and bucketing.

Logits against numpy's fp64 matmul; top-k against a stable full sort; weights
against mpmath's sigmoid; ties and k = E as special cases; bucketing against a
dictionary-based brute force."""

import math

import mpmath
import numpy as np
import pytest

import oracle
from synth import get_config, make_inputs
from tests._ref import bf16_val


def _routing_inputs(S=16, d=256, E=64, seed=3, bias=False):
    rng = np.random.default_rng(seed)
    from synth import f32_to_bf16_bits

    x = f32_to_bf16_bits(rng.standard_normal((S, d), dtype=np.float32))
    wr = (rng.standard_normal((E, d), dtype=np.float32) * 0.02).astype(np.float32)
    b = (rng.standard_normal(E, dtype=np.float32) * 0.3).astype(np.float32) if bias else None
    return x, wr, b


@pytest.mark.parametrize("bias", [False, True])
def test_logits_match_numpy_matmul(bias):
    x, wr, b = _routing_inputs(bias=bias)
    got = oracle.router_logits(x, wr, b)
    want = bf16_val(x) @ wr.astype(np.float64).T
    if b is not None:
        want = want + b.astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("k", [1, 2, 8])
def test_topk_equals_stable_full_sort(k):
    x, wr, b = _routing_inputs(bias=True)
    logits = oracle.router_logits(x, wr, b)
    ids, w = oracle.topk(logits, k)
    want = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, want)
    for t in range(logits.shape[0]):
        sel = logits[t, ids[t]]
        rest = np.delete(logits[t], ids[t])
        assert sel.min() >= rest.max()
        assert np.all(np.diff(sel) <= 0)


def test_weights_against_mpmath_sigmoid():
    x, wr, b = _routing_inputs(bias=True)
    logits = oracle.router_logits(x, wr, b)
    for renorm in (0, 1):
        ids, w = oracle.topk(logits, 8, renorm=renorm)
        mpmath.mp.dps = 40
        for t in range(logits.shape[0]):
            s = [1 / (1 + mpmath.exp(-mpmath.mpf(float(logits[t, e])))) for e in ids[t]]
            tot = sum(s) if renorm else 1
            want = np.array([float(si / tot) for si in s], np.float32)
            assert np.array_equal(w[t], want), (renorm, t)
        if renorm:
            np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)


def test_ties_go_to_lower_id():
    x, wr, _ = _routing_inputs(S=4, E=32)
    wr[9] = wr[5]
    wr[5] *= 0  # rows 5 and 9 made equal below
    wr[5] += 1.0
    wr[9] = wr[5]
    logits = oracle.router_logits(x, wr)
    ids, _ = oracle.topk(logits, 4)
    for t in range(4):
        row = list(ids[t])
        if logits[t, 5] > np.delete(logits[t], [5, 9]).max():
            assert row[:2] == [5, 9]


def test_all_equal_logits_closed_form():
    S, E, k = 3, 16, 4
    logits = np.zeros((S, E))
    ids, w = oracle.topk(logits, k)
    assert np.array_equal(ids, np.tile(np.arange(k), (S, 1)))
    assert np.all(w == np.float32(0.25))  # sigmoid(0)=1/2, renormalised over 4
    _, w0 = oracle.topk(logits, k, renorm=0)
    assert np.all(w0 == np.float32(0.5))


def test_k_equals_e_selects_all_in_order():
    x, wr, b = _routing_inputs(S=5, E=16, bias=True)
    logits = oracle.router_logits(x, wr, b)
    ids, w = oracle.topk(logits, 16)
    for t in range(5):
        assert sorted(ids[t]) == list(range(16))
        assert np.all(np.diff(logits[t, ids[t]]) <= 0)


@pytest.mark.parametrize("k", [1, 4, 8])
def test_topk_sel_against_sort_and_mpmath(k):
    """Selection-only bias: picks = stable sort of -(logits + bias), weights =
    mpmath sigmoid of the unbiased logits, renormalised over the picks."""
    x, wr, b = _routing_inputs(bias=True)
    logits = oracle.router_logits(x, wr)
    for renorm in (0, 1):
        ids, w = oracle.topk_sel(logits, b, k, renorm)
        key = logits + b.astype(np.float64)
        assert np.array_equal(ids, np.argsort(-key, axis=1, kind="stable")[:, :k])
        mpmath.mp.dps = 40
        for t in range(logits.shape[0]):
            s = [1 / (1 + mpmath.exp(-mpmath.mpf(float(logits[t, e])))) for e in ids[t]]
            tot = sum(s) if renorm else 1
            assert np.array_equal(w[t], np.array([float(si / tot) for si in s], np.float32))


def test_topk_sel_hand_example():
    """logits (1, 2, 3, 0), bias (5, 0, 0, 0), k = 2: the bias lifts expert 0
    to the top (score 6), expert 2 (score 3) is second; the weights are
    sigmoid(1) and sigmoid(3) over their sum, not sigmoid(6) and sigmoid(3)."""
    logits = np.array([[1.0, 2.0, 3.0, 0.0]])
    bias = np.array([5.0, 0.0, 0.0, 0.0], np.float32)
    ids, w = oracle.topk_sel(logits, bias, 2)
    assert ids.tolist() == [[0, 2]]
    s1, s3 = 1 / (1 + math.exp(-1.0)), 1 / (1 + math.exp(-3.0))
    assert np.array_equal(w[0], np.array([s1 / (s1 + s3), s3 / (s1 + s3)], np.float32))
    ids_b, w_b = oracle.topk(logits + bias, 2)  # bias in the logit: same picks
    assert ids_b.tolist() == [[0, 2]] and not np.array_equal(w_b, w)


def test_topk_sel_zero_bias_is_topk():
    x, wr, _ = _routing_inputs()
    logits = oracle.router_logits(x, wr)
    ids, w = oracle.topk_sel(logits, np.zeros(logits.shape[1], np.float32), 8)
    ids0, w0 = oracle.topk(logits, 8)
    assert np.array_equal(ids, ids0) and np.array_equal(w, w0)


def test_forward_bias_mode_1_writes_unbiased_logits():
    cfg = get_config("tiny").with_(E=16, n_local=8, topk=4, bias_kind="local", beta=0.3, bias_mode=1)
    inp = make_inputs(cfg, 2)
    got = oracle.forward(inp)
    assert np.array_equal(got["logits"], oracle.router_logits(inp["x"], inp["wr"]))
    ids, w = oracle.topk_sel(got["logits"], inp["bias"], cfg.topk)
    assert np.array_equal(got["ids"], ids) and np.array_equal(got["w"], w)


def _brute_bucket(ids, n_loc, base):
    S, k = ids.shape
    buckets = {el: [] for el in range(n_loc)}
    for t in range(S):
        for s in range(k):
            el = int(ids[t, s]) - base
            if 0 <= el < n_loc:
                buckets[el].append((t, s))
    return buckets


@pytest.mark.parametrize(
    "S,k,n_loc,base,E,seed",
    [(8, 2, 8, 0, 8, 0), (16, 8, 32, 0, 256, 1), (64, 8, 32, 64, 256, 2), (128, 8, 32, 224, 256, 3), (5, 3, 4, 2, 9, 4)],
)
def test_bucket_against_brute_force(S, k, n_loc, base, E, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(S)]).astype(np.int32)
    bk = oracle.bucket(ids, n_loc, base)
    brute = _brute_bucket(ids, n_loc, base)
    pos = 0
    nv = 0
    for el in range(n_loc):
        assert bk["offsets"][el] == pos
        assert bk["counts"][el] == len(brute[el])
        for j, (t, s) in enumerate(brute[el]):
            assert bk["rows"][pos + j] == t
            assert bk["pick_pos"][t, s] == pos + j
        pos += len(brute[el])
        if brute[el]:
            assert bk["active"][1 + nv] == el
            nv += 1
    assert bk["offsets"][n_loc] == pos
    assert bk["active"][0] == nv
    assert np.all(bk["active"][1 + nv :] == -1)
    assert np.all(bk["rows"][pos:] == -1)
    local = (ids >= base) & (ids < base + n_loc)
    assert np.all(bk["pick_pos"][~local] == -1)
    assert np.all(bk["pick_pos"][local] >= 0)


def test_bucket_no_local_picks():
    ids = np.array([[40, 41], [50, 60]], np.int32)
    bk = oracle.bucket(ids, 8, 0)
    assert bk["active"][0] == 0 and np.all(bk["counts"] == 0) and np.all(bk["pick_pos"] == -1)


def test_bucket_rejects_duplicate_ids():
    with pytest.raises(ValueError):
        oracle.bucket(np.array([[3, 3]], np.int32), 8, 0)


def test_workload_routing_shapes():
    """The workload recipes give the routing structure their names promise."""
    cfg = get_config("s16_local25")
    inp = make_inputs(cfg, 0, parts=("x", "wr", "bias"))
    logits = oracle.router_logits(inp["x"], inp["wr"], inp["bias"])
    ids, _ = oracle.topk(logits, cfg.topk)
    frac = np.mean(ids < cfg.n_local)
    assert 0.15 < frac < 0.35

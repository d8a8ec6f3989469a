"""Helpers of the GPU parity tests: run the HIP block, run the oracle on the
same inputs, compare step by step.

Tolerances (derived from the arithmetic; every comparison states its own):

* router logits: the GPU sums fp32 products in a per-lane loop of d / 64 terms
  and a 6-level shuffle tree; with u = 2^-24 the error is at most
  (d / 64 + 8) u sum_j |x_j w_ej| (+ one rounding of the bias add);
* top-k: ids bit-exact, except where the oracle's logits of the two
  experts that trade places differ by < 1e-5 (several answers are then
  correct); weights within 1e-6 relative of the oracle's weights computed
  from the GPU's own logits;
* buckets: bit-exact;
* expert outputs y: the GPU accumulates in fp32 before each bf16 rounding,
  the oracle in fp64, so a value sitting on a bf16 rounding boundary can land
  one ulp apart and move later sums slightly: per row, max |dy| <= 1e-2 RMS(y)
  and at least 90 % of the bf16 values identical;
* combine alone (same y): fp32 against fp64, max |d out| <= 1e-5 RMS(out);
* end to end: max |d out| <= 2e-2 RMS(out_oracle) over the compared rows;
  rows the oracle gives exactly zero must be exactly zero.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from moe_decode_layer_router_amd.block import MoeBlock
from tests._ref import bf16_val


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run_gpu(inp: dict, blk: MoeBlock | None = None) -> dict:
    blk = blk or MoeBlock(inp)
    blk.step()
    torch.cuda.synchronize()
    return dict(
        blk=blk, logits=to_np(blk.logits), ids=to_np(blk.ids), w=to_np(blk.w), counts=to_np(blk.counts),
        offsets=to_np(blk.offsets), rows=to_np(blk.rows), pick_pos=to_np(blk.pick_pos),
        active=to_np(blk.active), y=to_np(blk.y), out=to_np(blk.out),
    )


def check_logits(inp, g) -> np.ndarray:
    """GPU fp32 logits against the fp64 oracle; returns the oracle's logits."""
    cfg = inp["cfg"]
    lo = oracle.router_logits(inp["x"], inp["wr"], inp.get("bias"))
    mag = np.abs(bf16_val(inp["x"])) @ np.abs(inp["wr"].astype(np.float64)).T
    u = 2.0**-24
    tol = (cfg.d / 64 + 8) * u * mag + u * np.abs(lo) + 1e-30
    err = np.abs(g["logits"].astype(np.float64) - lo)
    assert np.all(err <= tol), f"logit error {err.max():.3g} > bound {tol[np.argmax(err / tol)]:.3g}"
    return lo


def check_topk(inp, g, lo) -> None:
    """ids against the oracle's top-k (near-ties excepted), weights against the
    oracle's weights of the GPU's logits and ids."""
    cfg = inp["cfg"]
    ids_o, _ = oracle.topk(lo, cfg.topk, cfg.renorm)
    ids_g = g["ids"]
    for t in range(cfg.S):
        if np.array_equal(ids_o[t], ids_g[t]):
            continue
        gap = np.abs(lo[t, ids_o[t]] - lo[t, ids_g[t]])
        assert np.all(gap < 1e-5), f"token {t}: ids {ids_g[t]} vs oracle {ids_o[t]} (logit gaps {gap})"
        assert len(set(ids_g[t])) == cfg.topk
    w_ref = oracle.route_weights(g["logits"].astype(np.float64), ids_g, cfg.renorm)
    np.testing.assert_allclose(g["w"], w_ref, rtol=1e-6, atol=0)


def check_bucket(inp, g) -> dict:
    cfg = inp["cfg"]
    bk = oracle.bucket(g["ids"], cfg.n_local, cfg.local_base)
    for k in ("counts", "offsets", "pick_pos", "active"):
        assert np.array_equal(g[k], bk[k]), k
    R = cfg.S * min(cfg.topk, cfg.n_local)
    assert np.array_equal(g["rows"][:R], bk["rows"]), "rows"
    return bk


def oracle_y_rows(inp, bk, rows_sel) -> dict:
    """Oracle expert outputs of the chosen bucket rows: {row: y bf16 bits}."""
    cfg = inp["cfg"]
    out = {}
    for r in rows_sel:
        el = int(np.searchsorted(bk["offsets"], r, side="right") - 1)
        t = int(bk["rows"][r])
        _, _, y = oracle.expert_row(
            inp["x"][t], inp["w13q"][el], inp["w13s"][el], inp["w2q"][el], inp["w2s"][el]
        )
        out[int(r)] = y
    return out


def compare_y(y_gpu_row, y_orc_row, what=""):
    a = bf16_val(y_gpu_row)
    b = bf16_val(y_orc_row)
    rms = np.sqrt(np.mean(b * b))
    err = np.abs(a - b).max()
    same = np.mean(y_gpu_row == y_orc_row)
    assert err <= 1e-2 * rms + 1e-30, f"{what}: max |dy| {err:.3g} > 1e-2 rms {rms:.3g}"
    assert same >= 0.9, f"{what}: only {same:.3f} of bf16 values identical"


def check_block(inp, g, tokens=None, max_rows=None) -> None:
    """Everything, step by step, on all tokens or on ``tokens`` only."""
    cfg = inp["cfg"]
    lo = check_logits(inp, g)
    check_topk(inp, g, lo)
    bk = check_bucket(inp, g)
    S = cfg.S
    tokens = list(range(S)) if tokens is None else list(tokens)
    R = cfg.S * min(cfg.topk, cfg.n_local)
    # expert outputs of the picks of the chosen tokens
    sel = sorted({int(p) for t in tokens for p in bk["pick_pos"][t] if p >= 0})
    if max_rows is not None:
        sel = sel[:max_rows]
    yo = oracle_y_rows(inp, bk, sel)
    for r, y in yo.items():
        compare_y(g["y"][r], y, f"bucket row {r}")
    y_full = g["y"].copy()
    if cfg.shared_I:
        for t in tokens:
            _, _, ys = oracle.shared_row(inp["x"][t], inp["ws13"], inp["ws2"])
            compare_y(g["y"][R + t], ys, f"shared row {t}")
    # combine alone: oracle on the GPU's y and weights
    out_c = oracle.combine(cfg, y_full, g["w"], g["pick_pos"], inp.get("gamma"))
    for t in tokens:
        rms = np.sqrt(np.mean(out_c[t].astype(np.float64) ** 2))
        err = np.abs(g["out"][t] - out_c[t]).max()
        assert err <= 1e-5 * rms + 1e-30, f"combine token {t}: {err:.3g} vs rms {rms:.3g}"
    # end to end on the selected tokens: oracle y and weights from its logits
    y_o = np.zeros_like(g["y"])
    for r, y in yo.items():
        y_o[r] = y
    if cfg.shared_I:
        for t in tokens:
            y_o[R + t] = oracle.shared_row(inp["x"][t], inp["ws13"], inp["ws2"])[2]
    w_o = oracle.route_weights(lo, g["ids"], cfg.renorm)
    out_o = oracle.combine(cfg, y_o, w_o, g["pick_pos"], inp.get("gamma"))
    ref = out_o[tokens].astype(np.float64)
    got = g["out"][tokens].astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    if max_rows is None:
        err = np.abs(got - ref).max() if ref.size else 0.0
        assert err <= 2e-2 * rms + 1e-30, f"end to end: max |d out| {err:.3g} > 2e-2 RMS {rms:.3g}"
        zero = np.all(ref == 0, axis=1)
        assert np.all(got[zero] == 0), "tokens without a local pick must be exactly zero"

"""Helpers of the GPU parity tests: run the HIP block, run the oracle on the
same inputs, compare step by step.

Tolerances (derived from the arithmetic; every comparison states its own):

* router logits, with u = 2^-24, checked against n u sum_j |x_j w_ej| + u |logit|
  where n bounds the roundings on any path of the GPU's summation order
  (logit_roundings): for S <= 16 a per-lane loop of at most d / 256 terms, a
  6-level shuffle tree, 4 levels over the 16 K slices and the bias add,
  n = d / 256 + 12 (S <= 32); beyond, the MFMA chains of a K part, the parts
  and the bias;
* top-k: ids bit-exact, except where the oracle's ranking keys (the logits,
  or logit + bias under the selection-only bias) of the two experts that
  trade places differ by < 1e-5 (several answers are then correct); weights within 1e-6 relative of the oracle's weights computed
  from the GPU's own logits;
* buckets: bit-exact;
* expert FFN, step by step: the GPU's SwiGLU rows h against the oracle's
  gate_up + SwiGLU (compare_h), then the GPU's y against the oracle's down GEMM
  applied to the GPU's own h (compare_y_step); the bounds are stated there;
* combine alone (same y): fp32 against fp64, max |d out| <= 1e-5 RMS(out);
* end to end: max |d out| <= 2e-2 RMS(out_oracle) at every compared element,
  in every case; each check records its ratio max |d out| / (2e-2 RMS)
  (PARITY_RATIO_LOG names a file that collects them); rows the oracle gives
  exactly zero must be exactly zero.
"""

from __future__ import annotations

import numpy as np
import torch

import moe_decode_layer_router_amd as mb
import oracle
from moe_decode_layer_router_amd.block import MoeBlock
from tests._ref import bf16_val


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run_gpu(inp: dict, blk: MoeBlock | None = None, fused: bool | str = False) -> dict:
    """One step of the block on the GPU: the four calls, or (fused) through
    moe_forward, or (fused="one") through moe_forward_one_launch. The SwiGLU
    rows are read from the call's workspace."""
    blk = blk or MoeBlock(inp)
    if fused == "one":
        blk.forward_one_launch()
    elif fused:
        blk.forward()
    else:
        blk.step()
    torch.cuda.synchronize()
    err = blk.forward_error() if fused else blk.ffn_error()
    assert err == 0, "a wait in the expert-FFN launch hit its bound"
    return dict(
        blk=blk, fused=fused, logits=to_np(blk.logits), ids=to_np(blk.ids), w=to_np(blk.w), counts=to_np(blk.counts),
        offsets=to_np(blk.offsets), rows=to_np(blk.rows), pick_pos=to_np(blk.pick_pos),
        active=to_np(blk.active), y=to_np(blk.y), out=to_np(blk.out),
    )


def logit_roundings(cfg, dims) -> float:
    """Worst-case number of fp32 roundings on the way to one GPU logit, from the
    summation order moe_route documents (the pages fix fp32 accumulation, not
    an order). Without scratch (S <= 32): a thread sums d / 1024 products (d / 256 roundings
    counting each product and each add, generously), then a tree of 12 levels
    (64 lanes, 16 waves) and the bias. With scratch: every product of a bf16
    token value with one of the three bf16 pieces of a weight is exact in fp32;
    in a K part of Kp, each of 4 chains takes ceil(Kp / 128) blocks of 3 MFMAs,
    each adding 32 products to its accumulator (at most 32 roundings, counting
    every add), the chains are added pairwise (2), each of 4 waves adds P / 4
    parts, the waves pairwise (2), then the bias (1); P from the scratch size
    moe_route asks for."""
    P = mb.moe_route_workspace_bytes(dims) // (cfg.S * cfg.E * 4)
    if P == 0:
        return cfg.d / 256 + 12
    return 3 * 32 * -(-(cfg.d // P) // 128) + 2 + P / 4 + 2 + 1


def check_logits(inp, g) -> np.ndarray:
    """GPU fp32 logits against the fp64 oracle; returns the oracle's logits."""
    cfg = inp["cfg"]
    lo = oracle.router_logits(inp["x"], inp["wr"], inp.get("bias") if cfg.bias_mode == 0 else None)
    mag = np.abs(bf16_val(inp["x"])) @ np.abs(inp["wr"].astype(np.float64)).T
    u = 2.0**-24
    n = logit_roundings(cfg, g["blk"].dims)
    tol = n * u * mag + u * np.abs(lo) + 1e-30
    err = np.abs(g["logits"].astype(np.float64) - lo)
    assert np.all(err <= tol), f"logit error {err.max():.3g} > bound {tol[np.argmax(err / tol)]:.3g}"
    return lo


def check_topk(inp, g, lo) -> None:
    """ids against the oracle's top-k (near-ties of the ranking key excepted),
    weights against the oracle's weights of the GPU's logits and ids. With the
    selection-only bias the key is logit + bias and the logits are unbiased."""
    cfg = inp["cfg"]
    bias = inp.get("bias")
    if cfg.bias_mode == 1 and bias is not None:
        ids_o, _ = oracle.topk_sel(lo, bias, cfg.topk, cfg.renorm)
        key = lo + bias.astype(np.float64)
    else:
        ids_o, _ = oracle.topk(lo, cfg.topk, cfg.renorm)
        key = lo
    ids_g = g["ids"]
    for t in range(cfg.S):
        if np.array_equal(ids_o[t], ids_g[t]):
            continue
        gap = np.abs(key[t, ids_o[t]] - key[t, ids_g[t]])
        assert np.all(gap < 1e-5), f"token {t}: ids {ids_g[t]} vs oracle {ids_o[t]} (key gaps {gap})"
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


def gpu_h(g, cfg) -> tuple[np.ndarray, np.ndarray | None]:
    """The SwiGLU rows the FFN left in its workspace: routed [R_max][I] and,
    with a shared expert, [S][I_s]. moe_forward's workspace holds moe_route's
    scratch first, then the FFN's."""
    ws = to_np(g["blk"].fws if g.get("fused") else g["blk"].ws)
    if g.get("fused"):
        ws = ws[mb.moe_route_workspace_bytes(g["blk"].dims):]
    R = cfg.S * min(cfg.topk, cfg.n_local)
    nb = R * cfg.I * 2
    h = ws[:nb].view(np.uint16).reshape(R, cfg.I)
    hs = None
    if cfg.shared_I:
        off = (nb + 255) // 256 * 256
        hs = ws[off : off + cfg.S * cfg.shared_I * 2].view(np.uint16).reshape(cfg.S, cfg.shared_I)
    return h, hs


def compare_h(h_gpu, h_orc, what=""):
    """SwiGLU rows. Both sides evaluate silu(g) * u in fp64 and round once to
    bf16, so they differ only where a gate_up value itself landed one bf16 ulp
    apart (the GPU rounds an fp32 sum, the oracle an fp64 sum; measured ~0.1 %
    of values); silu then moves the SwiGLU value by up to a few percent for a
    large negative gate, where it is tiny. So: per element
    |dh| <= 2^-6 |h| + 2^-10 RMS(h) + 2^-133 (one step of the bf16 subnormal
    grid, where a relative bound says nothing), and >= 98 % bit-identical
    among the values with |h| >= 2^-24 RMS(h) (the rest are numerically zero
    next to the row)."""
    a, b = bf16_val(h_gpu), bf16_val(h_orc)
    rms = np.sqrt(np.mean(b * b))
    err = np.abs(a - b)
    tol = 2.0**-6 * np.abs(b) + 2.0**-10 * rms + 2.0**-133
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, f"{what}: {bad.size} values off, e.g. [{bad[0]}] {a[bad[0]]} vs {b[bad[0]]}"
    sig = np.abs(b) >= 2.0**-24 * rms
    same = np.mean(h_gpu[sig] == h_orc[sig]) if sig.any() else 1.0
    assert same >= 0.98, f"{what}: only {same:.4f} of bf16 values identical"


def compare_y_step(y_gpu, y_ref, h_gpu, w_dense, what=""):
    """Down GEMM on the same (GPU) SwiGLU row: the only differences are the fp32
    accumulation order and a bf16 rounding flip it can cause:
    |dy| <= 2^-7 |y| + (K/32 + 64) 2^-24 sum_i |h_i w_ci| + 2^-133 (a step of
    the subnormal grid), >= 99 % identical."""
    a, b = bf16_val(y_gpu), bf16_val(y_ref)
    hv = bf16_val(h_gpu)
    mag = np.abs(w_dense) @ np.abs(hv)
    K = hv.shape[0]
    tol = 2.0**-7 * np.abs(b) + (K / 32 + 64) * 2.0**-24 * mag + 2.0**-133
    err = np.abs(a - b)
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, f"{what}: {bad.size} values off, e.g. [{bad[0]}] {a[bad[0]]} vs {b[bad[0]]}"
    same = np.mean(y_gpu == y_ref)
    assert same >= 0.99, f"{what}: only {same:.4f} of bf16 values identical"


def check_ffn_rows(inp, g, bk, rows_sel) -> dict:
    """Step-wise parity of the chosen bucket rows; returns the oracle's own
    end-to-end y rows {row: y}. Rows are taken expert by expert, so that only
    one expert's decoded down matrix is held at a time."""
    from tests._ref import decode_mx

    cfg = inp["cfg"]
    h_all, _ = gpu_h(g, cfg)
    y_o = {}
    by_el: dict = {}
    for r in rows_sel:
        el = int(np.searchsorted(bk["offsets"], r, side="right") - 1)
        by_el.setdefault(el, []).append(int(r))
    for el, rows in sorted(by_el.items()):
        dense = decode_mx(inp["w2q"][el], inp["w2s"][el])
        for r in rows:
            t = int(bk["rows"][r])
            _, h_o = oracle.mx_gate_up(inp["x"][t], inp["w13q"][el], inp["w13s"][el])
            compare_h(h_all[r], h_o, f"h of bucket row {r} (expert {el}, token {t})")
            y_ref = oracle.mx_down(h_all[r], inp["w2q"][el], inp["w2s"][el])
            compare_y_step(g["y"][r], y_ref, h_all[r], dense, f"y of bucket row {r}")
            y_o[r] = oracle.mx_down(h_o, inp["w2q"][el], inp["w2s"][el])
        del dense
    return y_o


def check_shared_rows(inp, g, tokens) -> dict:
    cfg = inp["cfg"]
    R = cfg.S * min(cfg.topk, cfg.n_local)
    _, hs = gpu_h(g, cfg)
    w2 = bf16_val(inp["ws2"])
    y_o = {}
    for t in tokens:
        _, h_o = oracle.bf_gate_up(inp["x"][t], inp["ws13"])
        compare_h(hs[t], h_o, f"shared h of token {t}")
        y_ref = oracle.bf_down(hs[t], inp["ws2"])
        compare_y_step(g["y"][R + t], y_ref, hs[t], w2, f"shared y of token {t}")
        y_o[t] = oracle.bf_down(h_o, inp["ws2"])
    return y_o


# max |d out| / (2e-2 RMS(out)) of every end-to-end check in this process,
# as (test id, ratio, elements over the plain bound); PARITY_RATIO_LOG names a
# file that each check also appends its line to
RATIOS: list = []


def _record_ratio(ratio: float, n_over: int, note: str = "") -> None:
    """Print and (PARITY_RATIO_LOG) append one check's end-to-end ratio."""
    import os

    case = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    RATIOS.append((case, ratio, n_over))
    line = f"{case}\t{ratio:.4f}\t{n_over}\t{note}"
    print(f"parity ratio: {line}")
    path = os.environ.get("PARITY_RATIO_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def check_block(inp, g, tokens=None) -> float:
    """Everything, step by step, on all tokens or on ``tokens`` only; returns
    max |d out| / (2e-2 RMS(out)), records it, and requires it <= 1 (the
    plain bound max |d out| <= 2e-2 RMS(out) at every element)."""
    cfg = inp["cfg"]
    lo = check_logits(inp, g)
    check_topk(inp, g, lo)
    bk = check_bucket(inp, g)
    S = cfg.S
    tokens = list(range(S)) if tokens is None else list(tokens)
    R = cfg.S * min(cfg.topk, cfg.n_local)
    # expert FFN of the picks of the chosen tokens, step by step
    sel = sorted({int(p) for t in tokens for p in bk["pick_pos"][t] if p >= 0})
    yo = check_ffn_rows(inp, g, bk, sel)
    ys = check_shared_rows(inp, g, tokens) if cfg.shared_I else {}
    # combine alone: oracle on the GPU's y and weights
    out_c = oracle.combine(cfg, g["y"], g["w"], g["pick_pos"], inp.get("gamma"))
    for t in tokens:
        rms = np.sqrt(np.mean(out_c[t].astype(np.float64) ** 2))
        err = np.abs(g["out"][t] - out_c[t]).max()
        assert err <= 1e-5 * rms + 1e-30, f"combine token {t}: {err:.3g} vs rms {rms:.3g}"
    # end to end on the chosen tokens: the oracle's own chain (y from its own
    # SwiGLU rows, weights from its own logits) on the GPU's routing choice
    y_o = np.zeros_like(g["y"])
    for r, y in yo.items():
        y_o[r] = y
    for t, y in ys.items():
        y_o[R + t] = y
    w_o = oracle.route_weights(lo, g["ids"], cfg.renorm)
    out_o = oracle.combine(cfg, y_o, w_o, g["pick_pos"], inp.get("gamma"))
    ref = out_o[tokens].astype(np.float64)
    got = g["out"][tokens].astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    err = np.abs(got - ref)
    plain = 2e-2 * rms + 1e-30
    ratio = float(err.max() / plain) if err.size else 0.0
    over = err > plain
    _record_ratio(ratio, int(over.sum()))
    if over.any():
        worst = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(
            f"end to end: |d out| {err[worst]:.3g} > 2e-2 RMS = {plain:.3g} "
            f"(token {tokens[worst[0]]}, column {worst[1]}; {int(over.sum())} elements over)"
        )
    zero = np.all(ref == 0, axis=1)
    assert np.all(got[zero] == 0), "tokens without a local pick must be exactly zero"
    return ratio

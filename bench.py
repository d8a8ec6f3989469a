#!/usr/bin/env python3
"""Benchmark of the local-expert MoE block on one MI355X.

A step is one pass of the whole block -- route, bucket, expert FFN, combine --
over one batch of S token rows, all inputs resident in HBM. It is timed as the
library's one-call entry point moe_forward (the headline `value`) and, for
comparison, as the four calls moe_route -> moe_bucket -> moe_expert_ffn ->
moe_combine. The headline workload is the largest of the row counts the
metric spans: S = 128, d = 7168, 256 experts (32 local), I = 2048, top-8
uniform routing, plus the always-on dense bf16 shared expert
("s128_shared"). The S = 8, 16 and 64 workloads ride along under
``workloads`` (same protocol, fewer steps); at S = 8 and 16 they also time
the block as one launch (moe_forward_one_launch, same outputs).

Last-level-cache control: MI355X's 256 MB Infinity Cache would hold one
step's active weights (about 94 MB here), so the benchmark keeps R copies of
every weight set with R x (active bytes) >= 512 MiB and rotates through them
step by step; every step then streams its weights from HBM, as a decode step
does between the other layers' weights.

Output: one JSON line (see the fields below). ``roofline`` covers the dominant
work, the expert FFN (one moe_expert_ffn call, about 95% of a step's bytes: one
kernel without a shared expert, else a gate_up + SwiGLU kernel and a down
kernel), timed with HIP events around each call on the stream its
kernels run on, in a separate timed pass; its
``traffic`` comes from the committed rocprofv3 counter summary when that
summary was taken on the current kernel sources, else null.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload (its first k token rows), with all of the host's OpenMP threads and
with one thread (``single_thread``).
``around_block`` times the steps next to the block (moe_pre_expert,
moe_latent_norm, moe_post_expert) at one GPU's share of their shapes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
LLC_BYTES = 256 * 2**20  # MI355X Infinity Cache
KERNEL_SOURCES = [
    "moe_decode_layer_router_amd/csrc/" + f for f in ("ffn.hip", "ffn_dev.h", "ffn_launch.h", "common.h")
]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes one moe_expert_ffn call moves (both kernels), from profiles/,
    if taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", f"expert_ffn_{workload}_traffic.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


def expert_bytes(cfg) -> int:
    """MXFP4 bytes of one expert: gate_up + down, values + e8m0 scales."""
    return 3 * cfg.I * cfg.d * 17 // 32


def _oracle_tokens(inp, k: int) -> dict:
    """The workload's inputs cut to its first k token rows: same weights,
    router and routing structure, fewer rows."""
    cfg = inp["cfg"]
    sub = dict(inp)
    sub["cfg"] = cfg.with_(S=k)
    sub["x"] = inp["x"][:k]
    return sub


def _time_oracle(inp, k: int, budget_s: float):
    """Whole oracle steps (route, bucket, expert FFN, combine) over the first
    k tokens, repeated until about budget_s seconds: (tokens/s, steps, s)."""
    import oracle

    sub = _oracle_tokens(inp, k)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(sub)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / n * (n + 1) > 2.5 * budget_s:
            break
    return k * n / el, n, el


def cpu_baseline(inp, budget_s: float) -> dict:
    """The CPU oracle as it stands, on this host's cores: all the threads
    OpenMP gives it (the headline) and one thread. A bounded sample: whole
    oracle steps over the workload's first k token rows, k doubled from 1
    until one step takes a quarter of budget_s (or k = S), then steps of k rows
    repeated for about budget_s seconds; tokens/s = k x steps / time."""
    import oracle

    cfg = inp["cfg"]
    res = {}
    n_thr = oracle.max_threads()
    for mode, threads in (("all", n_thr), ("single", 1)):
        oracle.set_threads(threads)
        k = 1
        while k < cfg.S:
            _, _, el1 = _time_oracle(inp, k, 0.0)  # one step
            if el1 >= budget_s / 4:
                break
            k = min(cfg.S, 2 * k)
        rate, n, el = _time_oracle(inp, k, budget_s)
        res[mode] = {
            "value": round(rate, 3),
            "unit": "tokens/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{n} oracle steps over the first {k} of {cfg.S} token rows of {cfg.name} "
            f"(same weights and routing), {threads} thread{'s' if threads > 1 else ''}, {el:.1f} s",
        }
    oracle.set_threads(n_thr)
    out = dict(res["all"])
    out["host_cpu_count"] = os.cpu_count()
    out["single_thread"] = res["single"]
    return out


def around_block(S: int, warmup: int, K: int) -> dict:
    """The steps next to the block at one rank's share of the K5 page's shapes
    (d_model 8192, latent 4096): pre (32 router rows + 512 pre_expert_proj
    rows on ffn_in), the latent norm on a gathered [S, 4096] projection, post
    (1024 post_expert_proj rows). Weight copies rotate as for the block."""
    import torch

    from moe_decode_layer_router_amd.block import ProjSteps
    from synth import PROJ_CONFIGS, make_proj_inputs

    pc = PROJ_CONFIGS["latent_s8"].with_(S=S)
    st = ProjSteps(make_proj_inputs(pc, 0), device="cuda:0")
    b_w = pc.n_pre * pc.D * 2 + pc.e_router * pc.D * 4 + pc.n_post * pc.L * 2
    n = max(1, math.ceil(2 * LLC_BYTES / b_w))
    st.add_weight_copies(n - 1)
    torch.cuda.synchronize()
    res = {"workload": f"latent_s{S}: S={S}, {pc.desc.split(', ', 1)[1]}", "weight_copies_rotated": n}
    steps = {
        "pre": (st.pre, pc.n_pre * pc.D * 2 + pc.e_router * pc.D * 4 + S * pc.D * 2 + S * pc.n_pre * 2
                + S * pc.e_router * 4),
        "norm": (st.norm, 2 * S * pc.L * 2 + pc.L * 2),
        "post": (st.post, pc.n_post * pc.L * 2 + S * pc.L * 4 + S * pc.n_post * 2),
    }
    # These calls are a few microseconds of GPU work, less than the host needs
    # to issue one, so they are timed as HIP graph replays: one graph holds
    # one call per weight copy, replayed back to back between two events.
    stream = torch.cuda.Stream()
    for name, (fn, nbytes) in steps.items():
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        reps = max(1, K // n)
        for _ in range(max(1, warmup // n)):
            g.replay()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        med = t0.elapsed_time(t1) / (reps * n)
        del g
        gbps = nbytes / (med * 1e-3) / 1e9
        res[name] = {"ms_per_call": round(med, 5), "algorithmic_bytes": nbytes, "gbps": round(gbps, 1),
                     "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    del st
    torch.cuda.empty_cache()
    return res


def measure(cfg, K: int, warmup: int, copies_arg: int = 0, calib_copy_mib: int = 0) -> dict:
    """Time one workload: moe_forward steps (the headline), the four calls,
    per-step spread, the warm-cache pass and each expert-FFN call."""
    import torch

    from moe_decode_layer_router_amd.block import MoeBlock
    from synth import make_inputs

    inp = make_inputs(cfg, 0)
    blk = MoeBlock(inp, device="cuda:0")
    blk.forward(0)
    torch.cuda.synchronize()
    counts = blk.counts.cpu().numpy()
    n_active = int((counts > 0).sum())
    picks = int(counts.sum())
    b_mx = n_active * expert_bytes(cfg)
    b_router = cfg.E * cfg.d * 4
    b_shared = 3 * cfg.shared_I * cfg.d * 2
    b_step_w = b_mx + b_router + b_shared
    copies = copies_arg or max(1, math.ceil(2 * LLC_BYTES / max(b_mx + b_shared, 1)))
    blk.add_weight_copies(copies - 1)
    torch.cuda.synchronize()

    if calib_copy_mib:
        n = calib_copy_mib * 2**20 // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    def timed(fn) -> float:
        for i in range(warmup):
            fn(i % copies)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(K):
            fn(i % copies)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / K

    def per_call(fn, n):
        """Event pairs around each of n calls on the current stream -> ms each."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(min(warmup, n)):
            fn(i % copies)
        torch.cuda.synchronize()
        for i in range(n):
            evs[i][0].record()
            fn(i % copies)
            evs[i][1].record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)

    # timed pass 1: whole steps through moe_forward (the headline)
    ms = timed(blk.forward)
    # timed pass 2: whole steps as the four calls
    ms4 = timed(blk.step)
    # pass 3: each step bracketed by its own events (median and spread)
    st = per_call(blk.forward, K)
    # pass 4: the same weight copy every step (warm last-level cache, labelled)
    ms_warm = timed(lambda _i: blk.forward(0))
    # pass 4b: the block as one launch, where moe_forward_one_launch takes it
    # (S <= 16, d <= 4096, no shared expert): same outputs, timed beside
    ms_one = None
    if cfg.S <= 16 and cfg.d <= 4096 and not cfg.shared_I:
        ms_one = timed(blk.forward_one_launch)
        torch.cuda.synchronize()
        assert blk.forward_error() == 0, "a wait in the one launch hit its bound"
    # pass 5: each expert-FFN call bracketed by events on its stream; routing
    # and buckets are those of the step (identical for every weight copy)
    blk.forward(0)
    ffn = per_call(blk.expert_ffn, K)
    ffn_ms = sum(ffn) / len(ffn)
    assert blk.forward_error() == 0 and blk.ffn_error() == 0, "a wait in an FFN launch hit its bound"

    # algorithmic bytes of one expert-FFN call: the active experts' MXFP4
    # weights, the shared expert's bf16 weights, x read, SwiGLU rows written
    # and read, y written
    b_ffn = b_mx + b_shared + cfg.S * cfg.d * 2 + picks * cfg.I * 2 * 2 + picks * cfg.d * 2
    if cfg.shared_I:
        b_ffn += cfg.S * cfg.shared_I * 2 * 2 + cfg.S * cfg.d * 2
    achieved = b_ffn / (ffn_ms * 1e-3) / 1e9
    # without a shared expert: one launch; else gate_up, then down
    single = not cfg.shared_I
    ffn_kernels = "moe_expert_ffn: " + ("ffn_single_kernel" if single else "gate_up_kernel + down_kernel")
    del blk
    torch.cuda.empty_cache()
    return dict(
        inp=inp, ms=ms, ms4=ms4, ms_one=ms_one, st=st, ms_warm=ms_warm, ffn_ms=ffn_ms, b_ffn=b_ffn, b_mx=b_mx,
        b_step_w=b_step_w, achieved=achieved, ffn_kernels=ffn_kernels, n_active=n_active,
        picks=picks, copies=copies,
    )


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # a shorter warm-up leaves the first timed pass a few percent slow at S = 128
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="s128_shared")
    ap.add_argument("--also", default="s8_uniform,s16_local25,s64_zipf",
                    help="more workloads timed beside the headline (comma list, '' for none)")
    ap.add_argument("--also-steps", type=int, default=100)
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="per oracle mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--no-around", action="store_true", help="skip the steps around the block")
    args = ap.parse_args()

    if args.gpus != 1:
        print(
            f"bench.py: --gpus {args.gpus} is not supported: this build measures one GPU's share of the "
            "expert-parallel block (no collectives); run with --gpus 1",
            file=sys.stderr,
        )
        return 2

    import torch

    from synth import get_config

    torch.cuda.set_device(0)
    cfg = get_config(args.workload)
    r = measure(cfg, args.steps, args.warmup, args.copies, args.calib_copy_mib)
    ms, K = r["ms"], args.steps
    traffic = committed_traffic(cfg.name)

    # read bandwidth of a torch reduction over 1 GiB (context only: not a
    # tuned streaming kernel)
    big = torch.ones(2**28, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in evs:
        a.record()
        big.sum()
        b.record()
    torch.cuda.synchronize()
    rd = sorted(a.elapsed_time(b) for a, b in evs)
    read_gbps = big.numel() * 4 / (rd[len(rd) // 2] * 1e-3) / 1e9
    del big

    around = None if args.no_around else around_block(cfg.S, args.warmup, K)

    def summary(c, m) -> dict:
        return {
            "S": c.S,
            "ms_per_step": round(m["ms"], 5),
            "tokens_per_s": round(c.S / (m["ms"] * 1e-3), 1),
            "all_weight_pct_hbm_peak": round(100 * m["b_step_w"] / (m["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "mxfp4_weight_gbps": round(m["b_mx"] / (m["ms"] * 1e-3) / 1e9, 1),
            "four_call_ms_per_step": round(m["ms4"], 5),
            "one_launch_ms_per_step": None if m["ms_one"] is None else round(m["ms_one"], 5),
            "active_local_experts": m["n_active"],
            "ffn_kernel": m["ffn_kernels"],
            "ffn_avg_ms": round(m["ffn_ms"], 5),
            "ffn_frac_hbm_peak": round(m["achieved"] / HBM_PEAK_GBPS, 4),
            "weight_copies_rotated": m["copies"],
        }

    others = {}
    for name in [w for w in args.also.split(",") if w and w != cfg.name]:
        c = get_config(name)
        m = measure(c, args.also_steps, min(args.warmup, args.also_steps))
        others[name] = summary(c, m)
        del m

    tok_s = cfg.S / (ms * 1e-3)
    line = {
        "metric": "tokens/s and MXFP4 weight HBM GB/s (% of peak), local-expert MoE, S=8..128",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator, seed 0)",
        "config": {
            "workload": cfg.name,
            "S": cfg.S,
            "d": cfg.d,
            "E": cfg.E,
            "n_local": cfg.n_local,
            "I": cfg.I,
            "topk": cfg.topk,
            "shared_I": cfg.shared_I,
            "active_local_experts": r["n_active"],
            "local_picks": r["picks"],
            "weight_copies_rotated": r["copies"],
        },
        "mxfp4_weight_gbps": round(r["b_mx"] / (ms * 1e-3) / 1e9, 1),
        "all_weight_pct_hbm_peak": round(100 * r["b_step_w"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "four_call_ms_per_step": round(r["ms4"], 5),
        "step_ms_median": round(r["st"][len(r["st"]) // 2], 5),
        "step_ms_p10": round(r["st"][len(r["st"]) // 10], 5),
        "step_ms_p90": round(r["st"][(9 * len(r["st"])) // 10], 5),
        "warm_llc_ms_per_step": round(r["ms_warm"], 5),
        "torch_sum_read_gbps": round(read_gbps, 1),
        "roofline": {
            "kernel": r["ffn_kernels"],
            "bound": "hbm",
            "achieved": round(r["achieved"], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(r["achieved"] / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes": r["b_ffn"],
            "avg_ms": round(r["ffn_ms"], 5),
        },
        "cpu_baseline": None,
        "workloads": others,
        "around_block": around,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(r["inp"], args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Device buffers for one MoE block and the four-call step.

``MoeBlock`` owns (through torch) the packed weights, the outputs of every call
and the FFN workspace, and runs route -> bucket -> expert FFN -> combine on the
current stream. It allocates only in its constructor and in
``add_weight_copies``; the four calls allocate nothing.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (
    MOE_W13,
    MOE_W2,
    MoeDims,
    dims_from,
    moe_bucket,
    moe_combine,
    moe_expert_ffn,
    moe_ffn_workspace_bytes,
    moe_forward,
    moe_forward_one_launch,
    moe_forward_workspace_bytes,
    moe_pack_bf16,
    moe_pack_mxfp4,
    moe_packed_bf16_bytes,
    moe_packed_mxfp4_bytes,
    moe_route,
    moe_route_workspace_bytes,
)


def _dev(a: np.ndarray | None, device, dtype=None):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def bf16_tensor(bits: np.ndarray | None, device):
    """uint16 bf16 bit patterns -> a torch.bfloat16 device tensor."""
    if bits is None:
        return None
    return _dev(np.ascontiguousarray(bits).view(np.int16), device, torch.bfloat16)


class MoeBlock:
    """Inputs from ``synth.make_inputs`` (canonical layouts) on ``device``."""

    def __init__(self, inp: dict, device="cuda", weight_copies: int = 1):
        cfg = inp["cfg"]
        self.cfg = cfg
        self.dims: MoeDims = dims_from(cfg)
        dv = torch.device(device)
        self.device = dv
        S, d, E, k, n = cfg.S, cfg.d, cfg.E, cfg.topk, cfg.n_local
        R = self.dims.r_max
        self.x = bf16_tensor(inp["x"], dv)
        self.gamma = bf16_tensor(inp.get("gamma"), dv)
        # weight sets (router + routed experts + shared expert); several copies
        # let a benchmark rotate through more bytes than the last-level cache
        self.sets = []
        w13q = _dev(inp["w13q"], dv)
        w13s = _dev(inp["w13s"], dv)
        w2q = _dev(inp["w2q"], dv)
        w2s = _dev(inp["w2s"], dv)
        ws13 = bf16_tensor(inp.get("ws13"), dv)
        ws2 = bf16_tensor(inp.get("ws2"), dv)
        st = {}
        st["wr"] = _dev(inp["wr"], dv)
        st["bias"] = _dev(inp.get("bias"), dv)
        st["w13"] = torch.empty(moe_packed_mxfp4_bytes(self.dims, MOE_W13), dtype=torch.uint8, device=dv)
        st["w2"] = torch.empty(moe_packed_mxfp4_bytes(self.dims, MOE_W2), dtype=torch.uint8, device=dv)
        moe_pack_mxfp4(self.dims, MOE_W13, w13q, w13s, st["w13"])
        moe_pack_mxfp4(self.dims, MOE_W2, w2q, w2s, st["w2"])
        if cfg.shared_I:
            st["ws13"] = torch.empty(moe_packed_bf16_bytes(self.dims, MOE_W13), dtype=torch.uint8, device=dv)
            st["ws2"] = torch.empty(moe_packed_bf16_bytes(self.dims, MOE_W2), dtype=torch.uint8, device=dv)
            moe_pack_bf16(self.dims, MOE_W13, ws13, st["ws13"])
            moe_pack_bf16(self.dims, MOE_W2, ws2, st["ws2"])
        else:
            st["ws13"] = st["ws2"] = None
        self.sets.append(st)
        del w13q, w13s, w2q, w2s, ws13, ws2
        self.add_weight_copies(weight_copies - 1)
        i32 = dict(dtype=torch.int32, device=dv)
        self.logits = torch.empty((S, E), dtype=torch.float32, device=dv)
        self.ids = torch.empty((S, k), **i32)
        self.w = torch.empty((S, k), dtype=torch.float32, device=dv)
        self.counts = torch.empty(n, **i32)
        self.offsets = torch.empty(n + 1, **i32)
        self.rows = torch.empty(max(R, 1), **i32)
        self.pick_pos = torch.empty((S, k), **i32)
        self.active = torch.empty(n + 1, **i32)
        self.y = torch.zeros((R + (S if cfg.shared_I else 0), d), dtype=torch.bfloat16, device=dv)
        self.out = torch.empty((S, d), dtype=torch.float32, device=dv)
        # workspaces: zero-filled once (the calls keep their counters at zero)
        self.ws = torch.zeros(max(moe_ffn_workspace_bytes(self.dims), 16), dtype=torch.uint8, device=dv)
        rw = moe_route_workspace_bytes(self.dims)
        self.rws = torch.empty(rw, dtype=torch.uint8, device=dv) if rw else None
        self.fws = torch.zeros(max(moe_forward_workspace_bytes(self.dims), 16), dtype=torch.uint8, device=dv)

    def add_weight_copies(self, n: int) -> None:
        """Append n device copies of the first weight set (same bytes)."""
        for _ in range(max(n, 0)):
            self.sets.append({k: (None if v is None else v.clone()) for k, v in self.sets[0].items()})

    # the four calls -----------------------------------------------------
    def route(self, s=0):
        st = self.sets[s]
        moe_route(self.dims, self.x, st["wr"], st["bias"], self.logits, self.ids, self.w, self.rws)

    def bucket(self):
        moe_bucket(self.dims, self.ids, self.counts, self.offsets, self.rows, self.pick_pos, self.active)

    def expert_ffn(self, s=0):
        st = self.sets[s]
        moe_expert_ffn(
            self.dims, self.x, st["w13"], st["w2"], self.counts, self.offsets, self.rows, self.active,
            st["ws13"], st["ws2"], self.y, self.ws,
        )

    def combine(self):
        moe_combine(self.dims, self.y, self.w, self.pick_pos, self.gamma, self.out)

    def step(self, s=0):
        """The block as four calls."""
        self.route(s)
        self.bucket()
        self.expert_ffn(s)
        self.combine()

    def forward(self, s=0):
        """The block through moe_forward (same outputs as step)."""
        st = self.sets[s]
        moe_forward(
            self.dims, self.x, st["wr"], st["bias"], st["w13"], st["w2"], st["ws13"], st["ws2"], self.gamma,
            self.logits, self.ids, self.w, self.counts, self.offsets, self.rows, self.pick_pos, self.active,
            self.y, self.out, self.fws,
        )

    def forward_one_launch(self, s=0):
        """The block through moe_forward_one_launch (S <= 16, d <= 4096, no
        shared expert; same outputs as forward)."""
        st = self.sets[s]
        moe_forward_one_launch(
            self.dims, self.x, st["wr"], st["bias"], st["w13"], st["w2"], self.gamma, self.logits,
            self.ids, self.w, self.counts, self.offsets, self.rows, self.pick_pos, self.active, self.y,
            self.out, self.fws,
        )

    @staticmethod
    def _error_word(ws) -> int:
        n = ws.numel()
        return int(ws[n - 256 : n - 252].view(torch.int32).item())

    def ffn_error(self) -> int:
        """moe_expert_ffn's wait-bound error word (0: no wait hit its bound)."""
        return self._error_word(self.ws)

    def forward_error(self) -> int:
        """moe_forward's wait-bound error word (0: no wait hit its bound)."""
        return self._error_word(self.fws)


class ProjSteps:
    """Device buffers of the steps around the block for inputs from
    ``synth.make_proj_inputs``: the pre-expert step (router + pre projection
    of this GPU's rows), the latent norm (on a gathered [S, L] projection) and
    the post-expert step (this GPU's rows). Allocates only in the constructor
    and in ``add_weight_copies``; ``s`` picks a weight copy."""

    def __init__(self, inp: dict, device="cuda"):
        from . import moe_pack_dense, moe_packed_dense_bytes, moe_proj_workspace_bytes, proj_dims_from

        pc = inp["cfg"]
        self.pc = pc
        dv = torch.device(device)
        S, D, L = pc.S, pc.D, pc.L
        self.pre_dims = proj_dims_from(dict(S=S, K=D, N=pc.n_pre, E=pc.e_router, bias_mode=pc.bias_mode))
        self.norm_dims = proj_dims_from(dict(S=S, K=L, N=L, eps=pc.eps))
        self.post_dims = proj_dims_from(dict(S=S, K=L, N=pc.n_post))
        self.ffn_in = bf16_tensor(inp["ffn_in"], dv)
        self.bias = _dev(inp.get("bias_pre"), dv)
        w_pre = torch.empty(moe_packed_dense_bytes(self.pre_dims), dtype=torch.uint8, device=dv)
        moe_pack_dense(self.pre_dims, bf16_tensor(inp["w_pre"], dv), w_pre)
        w_post = torch.empty(moe_packed_dense_bytes(self.post_dims), dtype=torch.uint8, device=dv)
        moe_pack_dense(self.post_dims, bf16_tensor(inp["w_post"], dv), w_post)
        # weight sets: [0] the originals, then copies (add_weight_copies)
        self.sets = [dict(w_pre=w_pre, wr=_dev(inp["wr_pre"], dv) if pc.e_router else None, w_post=w_post)]
        self.logits = torch.empty((S, max(pc.e_router, 1)), dtype=torch.float32, device=dv)
        self.h_raw = torch.empty((S, pc.n_pre), dtype=torch.bfloat16, device=dv)
        # workspaces start zero-filled (their counters); the calls leave them so
        self.ws_pre = torch.zeros(moe_proj_workspace_bytes(self.pre_dims), dtype=torch.uint8, device=dv)
        self.norm_in = bf16_tensor(inp["h_raw"], dv)
        self.gamma = bf16_tensor(inp.get("gamma_l"), dv)
        self.h = torch.empty((S, L), dtype=torch.bfloat16, device=dv)
        self.partial = _dev(inp["partial"], dv)
        self.out = torch.empty((S, pc.n_post), dtype=torch.bfloat16, device=dv)
        self.ws_post = torch.zeros(moe_proj_workspace_bytes(self.post_dims), dtype=torch.uint8, device=dv)

    def add_weight_copies(self, n: int) -> None:
        """n more copies of the weights, for timing with a cold last-level cache."""
        for _ in range(n):
            self.sets.append({k: (None if v is None else v.clone()) for k, v in self.sets[0].items()})

    def pre(self, s=0):
        from . import moe_pre_expert

        st = self.sets[s]
        moe_pre_expert(self.pre_dims, self.ffn_in, st["w_pre"], st["wr"], self.bias,
                       self.logits if self.pc.e_router else None, self.h_raw, self.ws_pre)

    def norm(self, s=0):
        from . import moe_latent_norm

        moe_latent_norm(self.norm_dims, self.norm_in, self.gamma, self.h)

    def post(self, s=0):
        from . import moe_post_expert

        moe_post_expert(self.post_dims, self.partial, self.sets[s]["w_post"], self.out, self.ws_post)

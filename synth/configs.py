"""The five workloads of the local-expert MoE block.

Shapes follow the Muse Spark K3 page (module docstring: one rank of a TP = EP = 8
group owns experts [32 r, 32 r + 32) of 256, top-8 routing) and the K5 page
(HA routing tail: 32 experts a rank, top-8; row sets S = 32..128). Token rows are
spec-verify rows, all valid.

Routing structure is imposed only through the router bias (``bias_kind``):

* ``none``    -- no bias: every expert equally likely.
* ``local``   -- bias ``beta`` on the local experts [local_base, local_base + n_local)
                 so that about a quarter of all picks land on them.
* ``zipf``    -- expert popularity shaped as Zipf(s) through a bias
                 ``-s * ln(rank_e)``, with the ranks interleaved so that the local
                 experts sample the whole popularity curve (rank 8 j + 3 for local
                 expert j) instead of holding only its head.
"""

from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    S: int  # token rows
    d: int  # hidden size seen by the experts
    E: int  # experts routed over
    topk: int  # picks per token
    n_local: int  # experts held by this GPU
    local_base: int  # first local expert id
    I: int  # expert intermediate size  # noqa: E741
    shared_I: int = 0  # 0: no shared expert
    renorm: int = 1  # routing weights renormalised over the top-k
    eps: float = 1e-6  # post-expert RMSNorm epsilon
    bias_kind: str = "none"
    bias_mode: int = 0  # 0: bias in the logit; 1: the bias steers the selection only
    beta: float = 0.0  # "local" bias value
    zipf_s: float = 0.0  # "zipf" exponent
    x_std: float = 1.0
    wr_std: float = 0.02
    # router weights: "normal" N(0, wr_std); "wide": sign x U[1, 2) x 2^U[-40, 4),
    # with about 5% exact zeros (magnitudes over 44 binades)
    wr_kind: str = "normal"
    ws_std: float = 0.02  # shared-expert weights
    e8m0_lo: int = 119  # e8m0 scale bytes drawn uniformly from [lo, hi]
    e8m0_hi: int = 127
    desc: str = ""

    def dims(self) -> dict:
        return dict(
            S=self.S,
            d=self.d,
            E=self.E,
            topk=self.topk,
            n_local=self.n_local,
            local_base=self.local_base,
            I=self.I,
            renorm=self.renorm,
            eps=self.eps,
            shared_I=self.shared_I,
            bias_mode=self.bias_mode,
        )

    def with_(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)


# "local" bias: beta = 0.50 gives 25.1 % local picks with this generator at
# d = 4096, router std 0.02 (mean over seeds 0..63 of 16 tokens x 8 picks; the
# per-seed spread is +- 3.7 %; 0.48 gives 24.4 %, 0.52 gives 25.9 %).
_BETA_25 = 0.50

CONFIGS = {
    "tiny": MoeConfig(
        name="tiny",
        S=8,
        d=256,
        E=8,
        topk=2,
        n_local=8,
        local_base=0,
        I=128,
        desc="S=8, d=256, 8 experts all local, I=128, top-2",
    ),
    "s8_uniform": MoeConfig(
        name="s8_uniform",
        S=8,
        d=4096,
        E=256,
        topk=8,
        n_local=32,
        local_base=0,
        I=2048,
        desc="S=8, d=4096, 256 experts (32 local), I=2048, top-8, uniform routing",
    ),
    "s16_local25": MoeConfig(
        name="s16_local25",
        S=16,
        d=4096,
        E=256,
        topk=8,
        n_local=32,
        local_base=0,
        I=2048,
        bias_kind="local",
        beta=_BETA_25,
        desc="S=16, as s8_uniform, router bias so ~25% of picks are local",
    ),
    "s64_zipf": MoeConfig(
        name="s64_zipf",
        S=64,
        d=4096,
        E=256,
        topk=8,
        n_local=32,
        local_base=0,
        I=2048,
        bias_kind="zipf",
        zipf_s=1.1,
        desc="S=64, as s8_uniform, Zipf(1.1) expert popularity via router bias",
    ),
    "s128_shared": MoeConfig(
        name="s128_shared",
        S=128,
        d=7168,
        E=256,
        topk=8,
        n_local=32,
        local_base=0,
        I=2048,
        shared_I=2048,
        desc="S=128, d=7168, 256 experts (32 local), I=2048, top-8, uniform, "
        "+ dense bf16 shared expert (I_s=2048)",
    ),
}

# the K5 page's other row counts on the S = 8 workload's shapes and routing
for _S in (32, 96):
    CONFIGS[f"s{_S}_uniform"] = CONFIGS["s8_uniform"].with_(
        name=f"s{_S}_uniform", S=_S, desc=f"S={_S}, as s8_uniform (uniform routing)"
    )

# the order the workloads are listed in: tiny first, then S = 8, 16, 64, 128
CONFIG_ORDER = ["tiny", "s8_uniform", "s16_local25", "s64_zipf", "s128_shared"]


def get_config(name: str) -> MoeConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {CONFIG_ORDER}") from None


@dataclasses.dataclass(frozen=True)
class ProjConfig:
    """The steps around the block (Muse Spark K5 page: HA's router and
    pre_expert_proj on ffn_in, pre_expert_norm; HB's post_expert_proj).
    A GPU holds n_pre rows of the pre projection, e_router router rows and
    n_post rows of the post projection; the norm runs on the whole latent."""

    name: str
    S: int  # token rows
    D: int  # model width (ffn_in, post output)
    L: int  # latent width (the experts' d)
    n_pre: int  # pre_expert_proj rows held by this GPU
    e_router: int  # router rows held by this GPU
    n_post: int  # post_expert_proj rows held by this GPU
    eps: float = 1e-6  # pre_expert_norm epsilon
    bias_mode: int = 0
    x_std: float = 1.0  # ffn_in
    w_std: float = 0.02  # dense projection weights
    wr_std: float = 0.02  # router weights
    partial_std: float = 1.0  # the summed expert partial (fp32)
    desc: str = ""

    def with_(self, **kw) -> "ProjConfig":
        return dataclasses.replace(self, **kw)


# K5 page, HA / HB: d_model 8192, latent 4096, 8 ranks: 512 pre rows, 32
# router rows and 1024 post rows a rank
PROJ_CONFIGS = {
    "latent_s8": ProjConfig(
        name="latent_s8", S=8, D=8192, L=4096, n_pre=512, e_router=32, n_post=1024,
        desc="S=8, d_model 8192 -> latent 4096: a rank's 512 pre rows + 32 router rows, norm over 4096, "
        "1024 post rows",
    ),
    "latent_s128": ProjConfig(
        name="latent_s128", S=128, D=8192, L=4096, n_pre=512, e_router=32, n_post=1024,
        desc="as latent_s8 at S=128",
    ),
    "latent_s8_whole": ProjConfig(
        name="latent_s8_whole", S=8, D=8192, L=4096, n_pre=4096, e_router=256, n_post=8192,
        desc="S=8, all 8 ranks' rows on one GPU: 4096 pre rows, 256 router rows, 8192 post rows",
    ),
}

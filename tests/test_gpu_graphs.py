"""HIP graph capture of the library's calls.

moe_forward, moe_forward_one_launch and the steps around the block make no
memset or allocation and leave their counters and flags at zero by the end
of every call (with kernel stores), so they can be captured. Each test captures the calls once, replays the graph several times
with eager calls of the same entry points between the replays, poisons the
outputs before every replay, and checks every replay against the eager
result bit for bit."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from synth import PROJ_CONFIGS, get_config, make_inputs, make_proj_inputs  # noqa: E402
from tests.gpu_util import to_np  # noqa: E402

KEYS = ("logits", "ids", "w", "counts", "offsets", "rows", "pick_pos", "active", "out")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _snapshot(obj, keys):
    return {k: to_np(getattr(obj, k)).copy() for k in keys}


def _poison(obj, keys):
    for k in keys:
        t = getattr(obj, k)
        t.fill_(float("nan") if t.is_floating_point() else -7)


@pytest.mark.parametrize("name", ["tiny", "s8_uniform", "s64_zipf", "s128_shared"])
def test_forward_graph_replays_match_eager(name):
    from moe_decode_layer_router_amd.block import MoeBlock

    inp = make_inputs(get_config(name), 0, gamma="random")
    blk = MoeBlock(inp)
    blk.forward()
    torch.cuda.synchronize()
    ref = _snapshot(blk, KEYS)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        blk.forward()
    for i in range(3):
        _poison(blk, KEYS)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(blk, KEYS)
        for k in KEYS:
            assert np.array_equal(got[k], ref[k]), (name, i, k)
        blk.forward() if i % 2 else blk.step()  # eager work between the replays
        torch.cuda.synchronize()
        assert np.array_equal(to_np(blk.out), ref["out"]), (name, i, "eager")
    assert blk.forward_error() == 0 and blk.ffn_error() == 0


@pytest.mark.parametrize("name", ["tiny", "s8_uniform"])
def test_one_launch_graph_replays_match_eager(name):
    """The block as one launch: its last combine workgroup clears the control
    words for the next call, also between graph replays; moe_forward runs
    eagerly on the same workspace in between."""
    from moe_decode_layer_router_amd.block import MoeBlock

    inp = make_inputs(get_config(name), 0, gamma="random")
    blk = MoeBlock(inp)
    blk.forward_one_launch()
    torch.cuda.synchronize()
    ref = _snapshot(blk, KEYS)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        blk.forward_one_launch()
    for i in range(3):
        _poison(blk, KEYS)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(blk, KEYS)
        for k in KEYS:
            assert np.array_equal(got[k], ref[k]), (name, i, k)
        blk.forward() if i % 2 else blk.forward_one_launch()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(blk.out), ref["out"]), (name, i, "eager")
    assert blk.forward_error() == 0


def test_steps_around_block_graph_replays_match_eager():
    from moe_decode_layer_router_amd.block import ProjSteps

    st = ProjSteps(make_proj_inputs(PROJ_CONFIGS["latent_s8"], 0))
    keys = ("logits", "h_raw", "h", "out")

    def run():
        st.pre()
        st.norm()
        st.post()

    run()
    torch.cuda.synchronize()
    ref = _snapshot(st, keys)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        run()
    for i in range(3):
        _poison(st, keys)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(st, keys)
        for k in keys:
            assert np.array_equal(got[k], ref[k]), (i, k)
        run()
        torch.cuda.synchronize()

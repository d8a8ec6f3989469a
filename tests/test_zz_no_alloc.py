"""moe_forward_static (no workspace, the library's static per-GPU scratch)
against moe_forward on the same inputs, through the C ABI: every output bit
for bit, on two calls in a row, the second with a smaller input (the array
keeps the first call's contents). Also: sizes beyond the static array are
rejected on the host."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import moe_decode_layer_router_amd as mb  # noqa: E402
from moe_decode_layer_router_amd.block import MoeBlock  # noqa: E402
from synth import get_config, make_inputs  # noqa: E402
from tests.gpu_util import to_np  # noqa: E402

KEYS = ("logits", "ids", "w", "counts", "offsets", "rows", "pick_pos", "active", "y", "out")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_both(cfg, seed):
    inp = make_inputs(cfg, seed, gamma="random")
    blk = MoeBlock(inp)
    blk.forward()
    torch.cuda.synchronize()
    assert blk.forward_error() == 0
    ref = {k: to_np(getattr(blk, k)).copy() for k in KEYS}
    for k in KEYS:  # poison every output
        t = getattr(blk, k)
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)
    err = torch.full((4,), 5, dtype=torch.int32, device=blk.x.device)
    st = blk.sets[0]
    mb.moe_forward_static(
        blk.dims, blk.x, st["wr"], st["bias"], st["w13"], st["w2"], st["ws13"], st["ws2"], blk.gamma,
        blk.logits, blk.ids, blk.w, blk.counts, blk.offsets, blk.rows, blk.pick_pos, blk.active, blk.y,
        blk.out, err,
    )
    torch.cuda.synchronize()
    assert int(err[0].item()) == 0, "the call clears the wait-error word and no wait hit its bound"
    assert int(err[1].item()) == 5, "only one word is written"
    got = {k: to_np(getattr(blk, k)) for k in KEYS}
    n = int(ref["offsets"][-1])
    R = blk.dims.r_max
    for k in KEYS:
        if k == "y":
            assert np.array_equal(got["y"][:n], ref["y"][:n]), k
            if cfg.shared_I:
                assert np.array_equal(got["y"][R:], ref["y"][R:]), k
        elif k == "rows":
            assert np.array_equal(got[k][:R], ref[k][:R]), k
        else:
            assert np.array_equal(got[k], ref[k]), k


def test_static_scratch_two_calls_second_smaller():
    """A larger call (S = 128 with the shared expert, split router, 32-row
    items), then a smaller one (S = 16, single-launch FFN) on the same array."""
    big = get_config("tiny").with_(S=128, d=1024, E=64, n_local=16, topk=4, I=256, shared_I=256)
    small = get_config("tiny").with_(S=16, d=512, E=32, n_local=8, topk=4, I=256)
    _run_both(big, 31)
    _run_both(small, 32)


def test_static_scratch_full_workload_then_smaller():
    _run_both(get_config("s128_shared"), 0)
    _run_both(get_config("s8_uniform"), 0)


def test_static_scratch_rejects_sizes_beyond_the_array():
    cfg = get_config("tiny").with_(S=128, d=16384, E=256, n_local=32, topk=8, I=8192, shared_I=8192)
    dims = mb.dims_from(cfg)
    assert mb.moe_forward_workspace_bytes(dims) > mb.MOE_STATIC_SCRATCH_BYTES
    dev = torch.device("cuda")
    z = torch.zeros(16, dtype=torch.uint8, device=dev)
    with pytest.raises(mb.MoeError) as e:
        mb.moe_forward_static(dims, z, z, None, z, z, z, z, None, z, z, z, z, z, z, z, z, z, z)
    assert e.value.code == mb.MOE_ERR_WORKSPACE

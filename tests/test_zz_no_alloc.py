"""dit_block_forward_noalloc (the workspace in the library's own device
array) against dit_block_forward (a caller workspace): the same kernels, so
the outputs agree bit for bit; two calls in a row, the second on a smaller
block, so the second runs on scratch that still holds the first call's data."""
import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R

from gpu_helpers import SMALL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def _both(cfg):
    import torch
    w = I.block_weights(cfg, 0, affine_random=True)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    blk = R.DeviceBlock(w)
    xd = R.to_dev_f32(x) if cfg.x_dtype == "f32" else R.to_dev_bf16(x)
    cd = R.to_dev_f32(c)
    cos, sin = R.rope_tables(cfg, pos)
    desc = R.desc_of(cfg)
    assert N.dit_block_workspace_size(desc) <= N.dit_block_forward_noalloc_max_bytes()
    ref = torch.empty_like(xd)
    ws = R.alloc_ws(N.dit_block_workspace_size(desc))
    N.dit_block_forward(desc, blk.c, xd, cd, cos, sin, ref, ws)
    got = torch.full_like(xd, float("nan"))
    N.dit_block_forward_noalloc(desc, blk.c, xd, cd, cos, sin, got)
    torch.cuda.synchronize()
    return R.to_host_f32(got), R.to_host_f32(ref)


def test_noalloc_matches_workspace_entry_point_twice():
    big, small = SMALL["gqa3_b2_ragged300"], SMALL["c1_ragged200"]
    for cfg in (big, small):
        say(f"noalloc block {cfg.name}: N={cfg.tokens} D={cfg.hidden}, "
            f"workspace {N.dit_block_workspace_size(R.desc_of(cfg))} bytes")
        got, ref = _both(cfg)
        assert np.isfinite(got).all()
        np.testing.assert_array_equal(got, ref)


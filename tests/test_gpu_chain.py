"""dit_block_chain_forward: a chain of blocks in place, with the next block's
AdaLN modulation GEMV on a side stream while the current block runs (layer
pipelining).  Bitwise equal to the same blocks run one dit_block_forward
call after another (same kernels, same order of arithmetic), and against
the float64 oracle block by block."""
import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R
from oracle import dit as O

from gpu_helpers import assert_parity, say

pytestmark = pytest.mark.gpu

CH = I.C1.replace(name="chain_small", cfg_id=28, x_dtype="f32", grid=(1, 12, 23))   # 276 tokens: ragged


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def _run(cfg, ws_np, x0, c, pos, mode):
    """mode: 'seq' (one dit_block_forward per block), 'chain' (no side stream),
    'pipe' (side stream)."""
    import torch
    blocks = [R.DeviceBlock(w) for w in ws_np]
    desc = R.desc_of(cfg)
    x = R.to_dev_f32(x0) if cfg.x_dtype == "f32" else R.to_dev_bf16(x0)
    cd = R.to_dev_f32(c)
    cos, sin = R.rope_tables(cfg, pos)
    if mode == "seq":
        ws = R.alloc_ws(N.dit_block_workspace_size(desc))
        for b in blocks:
            N.dit_block_forward(desc, b.c, x, cd, cos, sin, x, ws)
    else:
        ws = R.alloc_ws(N.dit_block_chain_workspace_size(desc))
        side = torch.cuda.Stream() if mode == "pipe" else None
        N.dit_block_chain_forward(desc, [b.c for b in blocks], x, cd, cos, sin, ws, side_stream=side)
    torch.cuda.synchronize()
    return R.to_host_f32(x)


@pytest.mark.parametrize("shared", [False, True], ids=["per_block_adaln", "shared_adaln"])
def test_chain_pipelined_equals_sequential_and_oracle(shared):
    cfg = CH
    n = 4
    ws_np = [I.block_weights(cfg, l, affine_random=True) for l in range(n)]
    if shared:
        for w in ws_np[1:]:
            w["w_ada"], w["b_ada"] = ws_np[0]["w_ada"], ws_np[0]["b_ada"]
    x0, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    seq = _run(cfg, ws_np, x0, c, pos, "seq")
    for mode in ("chain", "pipe", "pipe"):
        got = _run(cfg, ws_np, x0, c, pos, mode)
        say(f"  {mode}: max |chain - sequential| = {np.abs(got - seq).max():.3e}")
        np.testing.assert_array_equal(got, seq)
    ref = np.asarray(x0, np.float64)
    for w in ws_np:
        ref = O.block_forward(ref, c, w, cfg, pos)
    assert_parity(seq, ref, what=f"{n}-block chain out")
    assert_parity(seq - x0, ref - x0, what=f"{n}-block chain delta")


def test_chain_bf16_x_in_place():
    """bf16 x/out (the single-block workload's dtype) through a 3-block chain."""
    cfg = I.C1.replace(name="chain_bf16", cfg_id=29)
    ws_np = [I.block_weights(cfg, l) for l in range(3)]
    x0, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    np.testing.assert_array_equal(_run(cfg, ws_np, x0, c, pos, "pipe"), _run(cfg, ws_np, x0, c, pos, "seq"))

"""Parity at the widths of the headline workload, through the C ABI.

* The stack step at the 8B stack's shapes (hidden 4096, 32 x 128 heads,
  SwiGLU 12288, 4096 tokens, 128 latent channels, one shared AdaLN linear)
  with two layers: every velocity element against the fp32 oracle.  This
  covers the full-size patch embedding (4096 x 4096, K = 128), the output
  projection (4096 x 128, K = 4096) and the fp32 residual chain across
  blocks at hidden 4096.
* The pre-norm ViT backbone (batch 4 x 1024 tokens, hidden 1024, no AdaLN)
  as a 3-block chain updated in place: every output element against the
  float64 oracle run block after block.
"""
import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R
from oracle import dit as O

from gpu_helpers import assert_parity, metrics, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def _sync():
    import torch
    torch.cuda.synchronize()


def _device_stack(cfg, blocks, shared, edges):
    dev_shared = {"w_ada": R.to_dev_bf16(shared["w_ada"]), "b_ada": R.to_dev_f32(shared["b_ada"])}
    dblocks = []
    for w in blocks:
        t = {k: (None if v is None else (R.to_dev_bf16(v) if k in R._BF16_KEYS else R.to_dev_f32(v)))
             for k, v in w.items() if k not in ("w_ada", "b_ada")}
        t.update(dev_shared)
        dblocks.append(R.DeviceBlock(None, tensors=t))
    return R.DeviceStack(cfg, dblocks, R.upload_edges(edges))


@pytest.mark.slow
def test_stack_step_8b_width_two_layers_vs_oracle():
    import torch
    cfg = I.C4.replace(name="stack_8b_two_layers", layers=2)
    say(f"stack step at hidden {cfg.hidden}, {cfg.tokens} tokens, {cfg.layers} layers: drawing weights")
    shared = I.shared_ada(cfg)
    blocks = [I.stack_block_weights(cfg, l, shared) for l in range(cfg.layers)]
    edges = I.stack_edges(cfg)
    stack = _device_stack(cfg, blocks, shared, edges)
    pos = I.positions(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    lat = I.latent(cfg)
    sig = np.float32(N.dit_flowmatch_sigmas(I.STACK_STEPS, I.STACK_SHIFT)[3])
    cond = torch.empty(cfg.cond_dim, dtype=torch.float32, device="cuda")
    N.dit_sigma_embedding(float(sig), cfg.cond_dim, cond)
    vel = torch.empty((cfg.tokens, cfg.latent_dim), dtype=torch.float32, device="cuda")
    stack.step(R.to_dev_f32(lat), cond, cos, sin, vel)
    _sync()
    got = R.to_host_f32(vel)
    say("  fp32 oracle")
    ref = O.stack_step(lat, float(sig), blocks, edges, cfg, pos, dtype=np.float32)
    assert_parity(got, ref, what="velocity, every element (2 layers x 4096 wide, 4096 tokens)")
    # the patch embedding and the final layer alone are not what the blocks add:
    # the velocity of the stack differs from that of zero blocks
    ref0 = O.stack_step(lat, float(sig), blocks, edges, cfg, pos, dtype=np.float32, layers=0)
    say(f"  blocks' share of the velocity: {metrics(ref, ref0)}")
    assert metrics(ref, ref0)["rel_rms"] > 1e-2


@pytest.mark.slow
def test_vit_backbone_three_block_chain_in_place_vs_oracle():
    cfg = I.C2
    say(f"ViT chain: batch {cfg.batch} x {cfg.seq} tokens, hidden {cfg.hidden}, 3 blocks in place")
    ws = [I.block_weights(cfg, l, affine_random=True) for l in range(3)]
    x0, pos = I.block_x(cfg), I.positions(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    desc = R.desc_of(cfg)
    xd = R.to_dev_f32(x0)
    ptr = xd.data_ptr()
    wsd = R.alloc_ws(N.dit_block_workspace_size(desc))
    dblocks = [R.DeviceBlock(w) for w in ws]
    for b in dblocks:
        N.dit_block_forward(desc, b.c, xd, None, cos, sin, xd, wsd)
    _sync()
    assert xd.data_ptr() == ptr
    got = R.to_host_f32(xd)
    ref = np.asarray(x0, np.float64)
    for w in ws:
        ref = O.block_forward(ref, None, w, cfg, pos)
    assert_parity(got, ref, what="ViT 3-block chain out")
    assert_parity(got - x0, ref - x0, what="ViT 3-block chain delta")

"""dit_stack_step and the flow-match Euler loop against the oracle.

A 3-layer stack of small blocks runs whole denoising loops against the
float64 oracle, eagerly and as the library's recorded HIP graphs; two layers
at the full width replay the recorded loop (bf16 and W8A8) bitwise equal to
the eager one; the full 36 x 4096 stack at 4096 tokens is checked by the
properties that hold at any size (finite, bitwise deterministic).  Two layers at the full width are
compared with the oracle element by element in test_gpu_full_width.py."""
import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R
from oracle import dit as O

from gpu_helpers import assert_parity, metrics, say

pytestmark = pytest.mark.gpu

STK = I.C1.replace(name="stack_small", cfg_id=20, x_dtype="f32", layers=3, latent_dim=128, grid=(1, 16, 20))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def _sync():
    import torch
    torch.cuda.synchronize()


def _small_stack(cfg=STK):
    shared = I.shared_ada(cfg)
    blocks = [I.stack_block_weights(cfg, l, shared) for l in range(cfg.layers)]
    edges = I.stack_edges(cfg)
    dev_shared = {"w_ada": R.to_dev_bf16(shared["w_ada"]), "b_ada": R.to_dev_f32(shared["b_ada"])}
    dblocks = []
    for w in blocks:
        t = {k: (None if v is None else (R.to_dev_bf16(v) if k in R._BF16_KEYS else R.to_dev_f32(v)))
             for k, v in w.items() if k not in ("w_ada", "b_ada")}
        t.update(dev_shared)           # one AdaLN linear shared by every block
        dblocks.append(R.DeviceBlock(None, tensors=t))
    stack = R.DeviceStack(cfg, dblocks, R.upload_edges(edges))
    return blocks, edges, stack


def test_stack_step_vs_oracle():
    import torch
    cfg = STK
    blocks, edges, stack = _small_stack()
    pos = I.positions(cfg)
    lat = I.latent(cfg)
    sig = O.flowmatch_sigmas(8, 4.0)
    cos, sin = R.rope_tables(cfg, pos)
    for i in (0, 5):
        cond = torch.empty(cfg.cond_dim, dtype=torch.float32, device="cuda")
        N.dit_sigma_embedding(float(np.float32(sig[i])), cfg.cond_dim, cond)
        vel = torch.empty((cfg.tokens, cfg.latent_dim), dtype=torch.float32, device="cuda")
        stack.step(R.to_dev_f32(lat), cond, cos, sin, vel)
        _sync()
        ref = O.stack_step(lat, float(np.float32(sig[i])), blocks, edges, cfg, pos)
        assert_parity(R.to_host_f32(vel), ref, max_rel=2e-2, min_cos=0.9995, what=f"velocity step {i}")


def test_denoise_loop_vs_oracle_and_resume():
    cfg = STK
    blocks, edges, stack = _small_stack()
    pos = I.positions(cfg)
    lat0 = I.latent(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    steps = 4
    full = R.denoise(stack, R.to_dev_f32(lat0), cos, sin, steps, 4.0)
    _sync()
    got = R.to_host_f32(full)
    ref = O.denoise(lat0, blocks, edges, cfg, pos, steps, 4.0)
    assert_parity(got, ref, max_rel=2e-2, min_cos=0.9995, what="latent after 4 steps")
    dm = metrics(got - lat0, ref - lat0)
    say(f"  latent change: {dm}")
    assert dm["cos"] >= 0.999
    # resume from step 2 equals the uninterrupted loop, bit for bit
    lat = R.to_dev_f32(lat0)
    import torch
    sig = N.dit_flowmatch_sigmas(steps, 4.0)
    cond = torch.empty(cfg.cond_dim, dtype=torch.float32, device="cuda")
    vel = torch.empty_like(lat)
    for i in range(2):
        N.dit_sigma_embedding(float(sig[i]), cfg.cond_dim, cond)
        stack.step(lat, cond, cos, sin, vel)
        N.euler_flowmatch_update(lat, vel, lat.numel(), float(sig[i]), float(sig[i + 1]))
    saved = R.to_host_f32(lat)
    resumed = R.denoise(stack, R.to_dev_f32(saved), cos, sin, steps, 4.0, start=2)
    _sync()
    np.testing.assert_array_equal(R.to_host_f32(resumed), got)


def test_loop_graph_replays_match_eager_loop():
    """dit_loop_*: the whole loop recorded as HIP graphs reproduces the eager
    loop bit for bit, on every replay, with eager work and synchronisations
    between the replays; single-step replays resume like the eager loop."""
    import torch
    cfg = STK
    blocks, edges, stack = _small_stack()
    pos = I.positions(cfg)
    lat0 = I.latent(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    steps = 4
    eager = R.to_host_f32(R.denoise(stack, R.to_dev_f32(lat0), cos, sin, steps, 4.0))
    lat = R.to_dev_f32(lat0)
    loop = R.DeviceLoop(stack, lat, cos, sin, steps, 4.0)
    try:
        other = R.to_dev_f32(lat0)
        for rep in range(3):
            lat.copy_(R.to_dev_f32(lat0))
            loop.run()
            _sync()
            got = R.to_host_f32(lat)
            say(f"  replay {rep}: max |graph - eager| = {np.abs(got - eager).max():.3e}")
            np.testing.assert_array_equal(got, eager)
            R.denoise(stack, other, cos, sin, 1, 4.0)         # eager work between replays
            _sync()
        # steps 0-1 by graph, 2-3 eagerly: same as the uninterrupted loop
        lat.copy_(R.to_dev_f32(lat0))
        loop.step(0)
        loop.step(1)
        _sync()
        resumed = R.denoise(stack, R.to_dev_f32(R.to_host_f32(lat)), cos, sin, steps, 4.0, start=2)
        _sync()
        np.testing.assert_array_equal(R.to_host_f32(resumed), eager)
        with pytest.raises(N.DitError) as err:
            loop.step(steps)
        assert err.value.status == N.DIT_ERR_INVALID_ARG
    finally:
        loop.close()


@pytest.mark.parametrize("fmt", ["bf16", "w8a8_h256"])
def test_loop_graph_replays_match_eager_full_width(fmt):
    """The recorded loop at the 8B stack's widths (hidden 4096, 32 x 128 heads,
    SwiGLU 12288, 4096 tokens; 2 layers, 2 steps), where the projections run on
    the persistent 4-wave GEMM (bf16 or int8 operands) and the QKV projection
    in its split form with the separate qk-norm + RoPE pass: every replay
    bitwise equal to the eager loop, with eager work between the replays."""
    import bench
    cfg = I.C4.replace(name="stack_8b_graph", layers=2)
    say(f"loop graph at hidden {cfg.hidden}, {cfg.tokens} tokens, {cfg.layers} layers, {fmt}")
    stack, cos, sin = bench.build_full_stack(cfg)
    if fmt == "w8a8_h256":
        cfg = cfg.replace(fmt=fmt)
        stack = R.DeviceStack(cfg, [R.quantize_block(b) for b in stack.blocks], stack.edges)
    lat0 = I.latent(cfg)
    steps = 2
    eager = R.to_host_f32(R.denoise(stack, R.to_dev_f32(lat0), cos, sin, steps, I.STACK_SHIFT))
    assert np.isfinite(eager).all()
    lat = R.to_dev_f32(lat0)
    loop = R.DeviceLoop(stack, lat, cos, sin, steps, I.STACK_SHIFT)
    try:
        other = R.to_dev_f32(lat0)
        for rep in range(3):
            lat.copy_(R.to_dev_f32(lat0))
            loop.run()
            _sync()
            got = R.to_host_f32(lat)
            say(f"  replay {rep}: max |graph - eager| = {np.abs(got - eager).max():.3e}")
            np.testing.assert_array_equal(got, eager)
            R.denoise(stack, other, cos, sin, 1, I.STACK_SHIFT)     # eager work between replays
            _sync()
    finally:
        loop.close()


def test_loop_graph_vs_oracle():
    """dit_loop_*: the whole 8-step loop replayed from its HIP graphs against
    the float64 oracle's loop directly (not only against the eager HIP loop)."""
    cfg = STK
    blocks, edges, stack = _small_stack()
    pos = I.positions(cfg)
    lat0 = I.latent(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    steps = I.STACK_STEPS
    lat = R.to_dev_f32(lat0)
    loop = R.DeviceLoop(stack, lat, cos, sin, steps, I.STACK_SHIFT)
    try:
        loop.run()
        _sync()
        got = R.to_host_f32(lat)
    finally:
        loop.close()
    ref = O.denoise(lat0, blocks, edges, cfg, pos, steps, I.STACK_SHIFT)
    assert_parity(got, ref, max_rel=2e-2, min_cos=0.9995, what=f"graph loop latent after {steps} steps")
    assert_parity(got - lat0, ref - lat0, max_rel=2e-2, min_cos=0.9995, what="graph loop latent change")


def test_full_stack_step_properties():
    """The 36-block, 4096-wide stack at 4096 tokens: one denoising step is
    finite and bitwise reproducible (weights drawn on the device)."""
    import torch
    from bench import build_full_stack
    cfg = I.C4
    say("building the full 36 x 4096 stack on the device")
    stack, cos, sin = build_full_stack(cfg)
    lat = R.to_dev_f32(I.latent(cfg))
    cond = torch.empty(cfg.cond_dim, dtype=torch.float32, device="cuda")
    N.dit_sigma_embedding(1.0, cfg.cond_dim, cond)
    v1 = torch.empty_like(lat)
    v2 = torch.empty_like(lat)
    stack.step(lat, cond, cos, sin, v1)
    stack.step(lat, cond, cos, sin, v2)
    _sync()
    a, b = R.to_host_f32(v1), R.to_host_f32(v2)
    assert np.isfinite(a).all()
    np.testing.assert_array_equal(a, b)
    say(f"  velocity std {a.std():.4f}, mean {a.mean():.4f}")
    assert 0.01 < a.std() < 100.0

"""The fp32 run through the C ABI against the float64 oracle.

Weights are drawn from the same seeded streams as the bf16 runs but kept in
fp32 (not rounded to bf16), x is fp32, and every intermediate of the path is
fp32: fp32 MFMA GEMMs with the same fused epilogues, an fp32 LayerNorm /
modulation, an fp32 attention.  With no bf16 rounding anywhere the only error
left is fp32 arithmetic (about 1e-6 relative after a few thousand-term dot
products), so the gate is much tighter than the bf16 path's: max-rel <= 1e-4
and cosine >= 0.999999, on out and on the branch delta out - x."""
import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R
from oracle import dit as O

from gpu_helpers import SMALL, assert_parity, say

pytestmark = pytest.mark.gpu

MAX_REL_F32 = 1e-4
MIN_COS_F32 = 0.999999


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def _sync():
    import torch
    torch.cuda.synchronize()


def _f32(cfg):
    return cfg.replace(fmt="f32", x_dtype="f32")


def _run_block(cfg, w, x, c, pos):
    blk = R.DeviceBlock(w, f32=True)
    cos, sin = R.rope_tables(cfg, pos)
    o = R.block_forward(cfg, blk, R.to_dev_f32(x), R.to_dev_f32(c), cos, sin)
    _sync()
    return R.to_host_f32(o)


def _check(what, got, ref, x):
    assert_parity(got, ref, MAX_REL_F32, MIN_COS_F32, what=f"{what} out")
    x = np.asarray(x, np.float64)
    assert_parity(got - x, ref - x, MAX_REL_F32, MIN_COS_F32, what=f"{what} delta")


@pytest.mark.parametrize("name", ["c1_tiny", "c1_ragged200", "hd128_ragged400", "gqa3_b2_ragged300", "vit_b2_f32",
                                  "tiny_joint", "c1_rms", "c1_gelu", "c1_gate_tanh", "c1_scale_gate",
                                  "c1_rope_first", "half_hd128_rope_first", "hd128_ernie_diagram"])
def test_block_f32_vs_oracle(name):
    cfg = _f32(SMALL[name])
    say(f"f32 block {name}: N={cfg.tokens} D={cfg.hidden} H={cfg.heads}/{cfg.kv_heads}x{cfg.head_dim} F={cfg.ffn}")
    w = I.block_weights(cfg, 0, affine_random=True)
    assert w["w_qkv"].dtype == np.float32 and not np.array_equal(w["w_qkv"], I.bf16_round(w["w_qkv"]))
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    got = _run_block(cfg, w, x, c, pos)
    ref = O.block_forward(x, c, w, cfg, pos)
    _check(name, got, ref, x)


def test_block_f32_config_tiny():
    """The tiny block of the workload list in its fp32 run."""
    cfg = I.C1_F32
    say(f"f32 block {cfg.name}")
    w = I.block_weights(cfg, 0)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    got = _run_block(cfg, w, x, c, pos)
    ref = O.block_forward(x, c, w, cfg, pos)
    _check(cfg.name, got, ref, x)


@pytest.mark.parametrize("seq,batch", [(1, 1), (2, 3), (65, 1)])
def test_block_f32_degenerate_sequences(seq, batch):
    cfg = _f32(I.C1.replace(name=f"c1_f32_seq{seq}_b{batch}", seq_override=seq, batch=batch))
    say(f"f32 block seq={seq} batch={batch}")
    w = I.block_weights(cfg, 0, affine_random=True)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    got = _run_block(cfg, w, x, c, pos)
    ref = O.block_forward(x, c, w, cfg, pos)
    _check(cfg.name, got, ref, x)


def test_block_f32_full_size_sampled():
    """The 8B-class block at 4096 tokens in fp32, on sampled token rows (the
    oracle projects every key, then runs attention and the FFN for the sampled
    rows only, in fp32 for time)."""
    cfg = _f32(I.C3)
    say(f"f32 full-size block {cfg.name}: N={cfg.tokens} D={cfg.hidden}")
    w = I.block_weights(cfg, 0)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    got = _run_block(cfg, w, x, c, pos)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(0)
    rows = np.unique(np.r_[0, 1, 255, 256, 2047, 4095, rng.choice(cfg.tokens, 16, replace=False)])
    ref = O.block_forward(x, c, w, cfg, pos, dtype=np.float32, rows=rows)
    _check(cfg.name, got[rows], ref, x[rows])


# ---------------------------------------------------------------------------
# stages
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c1_tiny", "hd128_ragged400", "gqa3_b2_ragged300", "vit_b2_f32", "c1_rope_first",
                                  "half_hd128_rope_first", "c1_rms"])
def test_qkv_rope_f32(name):
    import torch
    cfg = _f32(SMALL[name])
    say(f"f32 qkv_rope {name}")
    h = np.random.default_rng(3).standard_normal((cfg.tokens, cfg.hidden), dtype=np.float32)
    w = I.block_weights(cfg, 0, affine_random=True)
    pos = I.positions(cfg)
    B, S, H, Hk, hd = cfg.batch, cfg.seq, cfg.heads, cfg.kv_heads, cfg.head_dim
    spad = N.dit_seq_pad(S)
    q = torch.empty((B, H, S, hd), dtype=torch.float32, device="cuda")
    k = torch.empty((B, Hk, S, hd), dtype=torch.float32, device="cuda")
    vt = torch.full((B, Hk, hd, spad), float("nan"), dtype=torch.float32, device="cuda")
    cos, sin = R.rope_tables(cfg, pos)
    dw = R.DeviceBlock(w, f32=True)
    N.dit_qkv_rope(R.desc_of(cfg), R.to_dev_f32(h), dw.t["w_qkv"], dw.t["q_g"], dw.t["q_b"], dw.t["k_g"], dw.t["k_b"],
                   cos, sin, q, k, vt)
    _sync()
    qo, ko, vo = O.block_qkv(h.astype(np.float64), w, cfg, pos)
    qg = R.to_host_f32(q).transpose(0, 2, 1, 3).reshape(B * S, H, hd)
    kg = R.to_host_f32(k).transpose(0, 2, 1, 3).reshape(B * S, Hk, hd)
    vtg = R.to_host_f32(vt)
    vg = vtg[..., :S].transpose(0, 3, 1, 2).reshape(B * S, Hk, hd)
    assert (vtg[..., S:] == 0).all(), "padded key positions of v^T must be zero"
    for nm, g, o in (("q", qg, qo), ("k", kg, ko), ("v", vg, vo)):
        assert_parity(g, o, MAX_REL_F32, MIN_COS_F32, what=f"{name}:{nm}")


@pytest.mark.parametrize("B,S,H,Hk,hd,amp", [(1, 256, 4, 4, 64, 1.0), (2, 300, 4, 2, 128, 2.0), (1, 1000, 4, 2, 64, 3.0),
                                              (3, 64, 6, 6, 128, 1.0), (1, 1, 2, 2, 128, 1.0), (2, 2, 4, 2, 64, 1.0),
                                              (1, 65, 2, 1, 128, 2.0)])
def test_flash_attention_f32(B, S, H, Hk, hd, amp):
    import torch
    say(f"f32 attention B={B} S={S} H={H} Hkv={Hk} hd={hd} amp={amp}")
    r = np.random.default_rng(4)
    q = r.standard_normal((B, H, S, hd), dtype=np.float32) * np.float32(amp)
    k = r.standard_normal((B, Hk, S, hd), dtype=np.float32) * np.float32(amp)
    v = r.standard_normal((B, Hk, S, hd), dtype=np.float32)
    spad = N.dit_seq_pad(S)
    vt = np.zeros((B, Hk, hd, spad), np.float32)
    vt[..., :S] = v.transpose(0, 1, 3, 2)
    cfg = I.DiTConfig("att", 0, B, (1, 1, S), H * hd, H, Hk, hd, 128, 0, False, "half2d", (hd // 2, hd // 2), 100.0,
                      x_dtype="f32", fmt="f32")
    out = torch.empty((B * S, H * hd), dtype=torch.float32, device="cuda")
    N.dit_flash_attention(R.desc_of(cfg), R.to_dev_f32(q), R.to_dev_f32(k), R.to_dev_f32(vt), out)
    _sync()
    ref = np.concatenate([O.attention(q[b].transpose(1, 0, 2).astype(np.float64), k[b].transpose(1, 0, 2),
                                      v[b].transpose(1, 0, 2), H, Hk) for b in range(B)])
    assert_parity(R.to_host_f32(out), ref, MAX_REL_F32, MIN_COS_F32, what="f32 attention")


# ---------------------------------------------------------------------------
# stack and loop
# ---------------------------------------------------------------------------
STK_F32 = I.C1.replace(name="stack_small_f32", cfg_id=20, x_dtype="f32", layers=3, latent_dim=128, grid=(1, 16, 20),
                       fmt="f32")


def _stack_f32(cfg=STK_F32):
    shared = I.shared_ada(cfg)
    blocks = [I.stack_block_weights(cfg, l, shared) for l in range(cfg.layers)]
    edges = I.stack_edges(cfg)
    dev_shared = {"w_ada": R.to_dev_f32(shared["w_ada"]), "b_ada": R.to_dev_f32(shared["b_ada"])}
    dblocks = []
    for w in blocks:
        t = {k: (None if v is None else R.to_dev_f32(v)) for k, v in w.items() if k not in ("w_ada", "b_ada")}
        t.update(dev_shared)
        dblocks.append(R.DeviceBlock(None, tensors=t))
    return blocks, edges, R.DeviceStack(cfg, dblocks, R.upload_edges(edges, f32=True))


def test_stack_f32_step_and_loop():
    import torch
    cfg = STK_F32
    blocks, edges, stack = _stack_f32()
    pos = I.positions(cfg)
    lat = I.latent(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    sig = O.flowmatch_sigmas(8, 4.0)
    for i in (0, 5):
        say(f"f32 stack step {i}")
        t = float(np.float32(1000.0 * sig[i]))     # the fp32 timestep the device embeds
        cond = torch.empty(cfg.cond_dim, dtype=torch.float32, device="cuda")
        N.dit_timestep_embedding(t, cfg.cond_dim, cond)
        vel = torch.empty((cfg.tokens, cfg.latent_dim), dtype=torch.float32, device="cuda")
        stack.step(R.to_dev_f32(lat), cond, cos, sin, vel)
        _sync()
        ref = O.stack_step(lat, t / 1000.0, blocks, edges, cfg, pos)
        assert_parity(R.to_host_f32(vel), ref, MAX_REL_F32, MIN_COS_F32, what=f"f32 velocity step {i}")
    say("f32 denoise loop, 4 steps")
    got = R.to_host_f32(R.denoise(stack, R.to_dev_f32(lat), cos, sin, 4, 4.0))
    ref = O.denoise(lat, blocks, edges, cfg, pos, 4, 4.0)
    assert_parity(got, ref, MAX_REL_F32, MIN_COS_F32, what="f32 latent after 4 steps")
    assert_parity(got - lat, ref - lat, MAX_REL_F32, MIN_COS_F32, what="f32 latent change")

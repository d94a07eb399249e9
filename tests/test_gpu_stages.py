"""Per-stage parity of the HIP kernels (through the C ABI) against the oracle,
on seeded inputs that span several tiles and ragged tails."""
import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R
from oracle import dit as O

from gpu_helpers import QKV_SPLIT, QKV_TAIL, SMALL, assert_parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def _rng(seed):
    return np.random.default_rng(seed)


def _sync():
    import torch
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("out_dim,in_dim,silu", [(1536, 256, 1), (24576, 4096, 1), (8192, 4096, 0), (36, 264, 1)])
def test_adaln_gemv(out_dim, in_dim, silu):
    import torch
    say(f"adaln_gemv out={out_dim} in={in_dim} silu={silu}")
    r = _rng(1)
    w = I.bf16_round(r.standard_normal((out_dim, in_dim), dtype=np.float32) * 0.02)
    b = I.bf16_round(r.standard_normal(out_dim, dtype=np.float32) * 0.02)
    c = r.standard_normal(in_dim, dtype=np.float32)
    m = torch.empty(out_dim, dtype=torch.float32, device="cuda")
    N.dit_adaln_modulation(R.to_dev_bf16(w), R.to_dev_f32(b), R.to_dev_f32(c), out_dim, in_dim, silu, m)
    _sync()
    ref = O.linear(O.silu(c.astype(np.float64)) if silu else c, w, b)
    assert_parity(R.to_host_f32(m), ref, max_rel=1e-5, min_cos=0.9999999, what="adaln_gemv")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows,dim,xdt,mode", [(300, 256, "f32", 0), (257, 4096, "bf16", 0), (64, 6144, "f32", 1),
                                               (5, 1024, "bf16", 1), (1, 4096, "f32", 0)])
def test_ln_modulate(rows, dim, xdt, mode):
    import torch
    say(f"ln_modulate rows={rows} dim={dim} x={xdt} mode={mode}")
    r = _rng(2)
    x = (r.standard_normal((rows, dim), dtype=np.float32) * 3 + 0.5).astype(np.float32)
    if xdt == "bf16":
        x = I.bf16_round(x)
    shift = (r.standard_normal(dim) * 0.5).astype(np.float32)
    scale = (r.standard_normal(dim) * 0.5).astype(np.float32)
    xd = R.to_dev_f32(x) if xdt == "f32" else R.to_dev_bf16(x)
    h = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    N.dit_ln_modulate(xd, N.DIT_F32 if xdt == "f32" else N.DIT_BF16, rows, dim, R.to_dev_f32(shift),
                      R.to_dev_f32(scale), mode, 1e-6, h)
    _sync()
    n = O.layer_norm(x.astype(np.float64), 1e-6)
    ref = O.modulate(n, shift, scale) if mode == 0 else n * scale + shift
    got = R.to_host_f32(h)
    # one bf16 rounding of the output: |err| <= 2^-8 |ref| (+ fp32 noise)
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5).all()
    assert_parity(got, ref, max_rel=4e-3, min_cos=0.99999, what="ln_modulate")


@pytest.mark.parametrize("rows,dim,xdt,mode,shift", [(300, 256, "f32", 0, True), (257, 4096, "bf16", 0, False),
                                                     (64, 1024, "f32", 1, True)])
def test_ln_modulate_rmsnorm(rows, dim, xdt, mode, shift):
    """RMSNorm rows (no centring) and the no-shift modulation (shift NULL)."""
    import torch
    say(f"ln_modulate RMSNorm rows={rows} dim={dim} x={xdt} mode={mode} shift={shift}")
    r = _rng(12)
    x = (r.standard_normal((rows, dim), dtype=np.float32) * 3 + 0.5).astype(np.float32)
    if xdt == "bf16":
        x = I.bf16_round(x)
    sh = (r.standard_normal(dim) * 0.5).astype(np.float32) if shift else None
    sc = (r.standard_normal(dim) * 0.5).astype(np.float32)
    xd = R.to_dev_f32(x) if xdt == "f32" else R.to_dev_bf16(x)
    h = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    N.dit_ln_modulate(xd, N.DIT_F32 if xdt == "f32" else N.DIT_BF16, rows, dim, R.to_dev_f32(sh), R.to_dev_f32(sc),
                      mode, 1e-6, h, norm=N.DIT_RMSNORM)
    _sync()
    n = O.rms_norm(x.astype(np.float64), 1e-6)
    add = 0.0 if sh is None else sh
    ref = O.modulate(n, add, sc) if mode == 0 else n * sc + add
    got = R.to_host_f32(h)
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5).all()
    assert_parity(got, ref, max_rel=4e-3, min_cos=0.99999, what="ln_modulate rms")


# ---------------------------------------------------------------------------
def _qkv_case(cfg, seed=3):
    """Random bf16 h and block weights with a non-trivial qk-norm affine."""
    r = _rng(seed)
    h = I.bf16_round(r.standard_normal((cfg.tokens, cfg.hidden), dtype=np.float32))
    w = I.block_weights(cfg, 0, affine_random=True)
    return h, w


@pytest.mark.parametrize("name", ["c1_rms", "c1_rope_first", "hd128_ernie_diagram", "half_hd128_rope_first",
                                  "c1_tiny", "c1_ragged200", "hd128_ragged400", "gqa3_b2_ragged300", "vit_b2_f32",
                                  "c1_f32x_t3", "qkv_tail_4170", "qkv_split_b2_1008", "qkv_split_half_1904",
                                  "qkv_split_joint_4170", "qkv_split_mixed_group_3072", "qkv_split_no_qknorm_b2_1008",
                                  "qkv_fused_hd64_1899"])
def test_qkv_rope(name):
    import torch
    cfg = QKV_TAIL if name == "qkv_tail_4170" else QKV_SPLIT.get(name) or SMALL[name]
    say(f"qkv_rope {name}")
    h, w = _qkv_case(cfg)
    pos = I.positions(cfg)
    desc = R.desc_of(cfg)
    B, S, H, Hk, hd = cfg.batch, cfg.seq, cfg.heads, cfg.kv_heads, cfg.head_dim
    spad = N.dit_seq_pad(S)
    q = torch.empty((B, H, S, hd), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((B, Hk, S, hd), dtype=torch.bfloat16, device="cuda")
    vt = torch.full((B, Hk, hd, spad), float("nan"), dtype=torch.bfloat16, device="cuda")
    cos, sin = R.rope_tables(cfg, pos)
    dw = R.DeviceBlock(w)
    N.dit_qkv_rope(desc, R.to_dev_bf16(h), dw.t["w_qkv"], dw.t["q_g"], dw.t["q_b"], dw.t["k_g"], dw.t["k_b"], cos, sin,
                   q, k, vt)
    _sync()
    qo, ko, vo = O.block_qkv(h.astype(np.float64), w, cfg, pos)
    qg = R.to_host_f32(q).transpose(0, 2, 1, 3).reshape(B * S, H, hd)
    kg = R.to_host_f32(k).transpose(0, 2, 1, 3).reshape(B * S, Hk, hd)
    vtg = R.to_host_f32(vt)
    vg = vtg[..., :S].transpose(0, 3, 1, 2).reshape(B * S, Hk, hd)
    assert (vtg[..., S:] == 0).all(), "padded key positions of v^T must be zero"
    for nm, g, o in (("q", qg, qo), ("k", kg, ko), ("v", vg, vo)):
        assert_parity(g, o, max_rel=1e-2, min_cos=0.99999, what=f"{name}:{nm}")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,S,H,Hk,hd,amp", [(1, 256, 4, 4, 64, 1.0), (2, 300, 4, 2, 128, 2.0), (1, 100, 2, 2, 128, 3.0),
                                              (1, 1000, 4, 2, 64, 1.5), (3, 64, 6, 6, 128, 1.0),
                                              (1, 1, 2, 2, 128, 1.0), (2, 2, 4, 2, 64, 1.0),   # one / two tokens
                                              (1, 65, 2, 1, 128, 2.0)])                       # one key past a tile
def test_flash_attention(B, S, H, Hk, hd, amp):
    import torch
    say(f"flash_attention B={B} S={S} H={H} Hkv={Hk} hd={hd} amp={amp}")
    r = _rng(4)
    q = I.bf16_round(r.standard_normal((B, H, S, hd), dtype=np.float32) * amp)
    k = I.bf16_round(r.standard_normal((B, Hk, S, hd), dtype=np.float32) * amp)
    v = I.bf16_round(r.standard_normal((B, Hk, S, hd), dtype=np.float32))
    spad = N.dit_seq_pad(S)
    vt = np.zeros((B, Hk, hd, spad), np.float32)
    vt[..., :S] = v.transpose(0, 1, 3, 2)
    cfg = I.DiTConfig("att", 0, B, (1, 1, S), H * hd, H, Hk, hd, 128, 0, False, "half2d", (hd // 2, hd // 2), 100.0)
    out = torch.empty((B * S, H * hd), dtype=torch.bfloat16, device="cuda")
    N.dit_flash_attention(R.desc_of(cfg), R.to_dev_bf16(q), R.to_dev_bf16(k), R.to_dev_bf16(vt), out)
    _sync()
    ref = np.concatenate([O.attention(q[b].transpose(1, 0, 2).astype(np.float64), k[b].transpose(1, 0, 2),
                                      v[b].transpose(1, 0, 2), H, Hk) for b in range(B)])
    assert_parity(R.to_host_f32(out), ref, max_rel=2e-2, min_cos=0.9999, what="attention")


@pytest.mark.parametrize("B,S,H,Hk,hd,nsplit", [
    (1, 300, 4, 2, 128, 2), (2, 1000, 4, 4, 64, 3), (1, 4170, 2, 2, 128, 8),   # joint 4096 + 74 text rows
    (1, 100, 2, 2, 128, 2),                                                     # one partial q tile only
    (1, 263, 4, 4, 64, 64),                                                     # more chunks than key tiles
    (3, 130, 6, 3, 128, 16),                                                    # batch 3, GQA, 3 key tiles
    (1, 512, 2, 2, 128, 4),                                                     # no tail: plain kernel
    (1, 65, 2, 2, 128, 2), (1, 1, 4, 4, 64, 4),                                 # a 1-key chunk; a 1-token sequence
])
def test_flash_attention_split_tail(B, S, H, Hk, hd, nsplit):
    """The partial last q tile split over key chunks and merged (split-KV)
    against the explicit softmax; the full q tiles run unsplit in the same
    launch."""
    import torch
    say(f"flash_attention_split B={B} S={S} H={H} Hkv={Hk} hd={hd} nsplit={nsplit}")
    r = _rng(8)
    q = I.bf16_round(r.standard_normal((B, H, S, hd), dtype=np.float32) * 1.5)
    k = I.bf16_round(r.standard_normal((B, Hk, S, hd), dtype=np.float32) * 1.5)
    v = I.bf16_round(r.standard_normal((B, Hk, S, hd), dtype=np.float32))
    spad = N.dit_seq_pad(S)
    vt = np.zeros((B, Hk, hd, spad), np.float32)
    vt[..., :S] = v.transpose(0, 1, 3, 2)
    cfg = I.DiTConfig("att", 0, B, (1, 1, S), H * hd, H, Hk, hd, 128, 0, False, "half2d", (hd // 2, hd // 2), 100.0)
    desc = R.desc_of(cfg)
    ws = R.alloc_ws(N.dit_attention_workspace_size(desc, nsplit))
    out = torch.empty((B * S, H * hd), dtype=torch.bfloat16, device="cuda")
    qd, kd, vd = R.to_dev_bf16(q), R.to_dev_bf16(k), R.to_dev_bf16(vt)
    N.dit_flash_attention_split(desc, qd, kd, vd, out, nsplit, ws)
    _sync()
    rows = np.arange(B * S)
    if S > 1024:                      # the oracle on the tail rows and a sample of the others
        tail = np.arange(S // 256 * 256, S)
        rows = np.unique(np.r_[tail, 0, 1, 255, 256, 2047, np.random.default_rng(2).choice(S, 24, replace=False)])
    ref = np.concatenate([O.attention(q[b].transpose(1, 0, 2).astype(np.float64), k[b].transpose(1, 0, 2),
                                      v[b].transpose(1, 0, 2), H, Hk, rows) for b in range(B)]) if B == 1 else \
        np.concatenate([O.attention(q[b].transpose(1, 0, 2).astype(np.float64), k[b].transpose(1, 0, 2),
                                    v[b].transpose(1, 0, 2), H, Hk) for b in range(B)])
    got = R.to_host_f32(out)
    got = got[rows] if B == 1 else got
    assert_parity(got, ref, max_rel=2e-2, min_cos=0.9999, what=f"attention split {nsplit}")
    # the same launch without the split gives the same values up to the merge's rounding
    plain = torch.empty_like(out)
    N.dit_flash_attention(desc, qd, kd, vd, plain)
    _sync()
    pm = R.to_host_f32(plain)
    pm = pm[rows] if B == 1 else pm
    assert_parity(got, pm, max_rel=1e-2, min_cos=0.99999, what="split vs unsplit")


@pytest.mark.parametrize("kind,S,hd,nsplit", [("ramp", 1000, 128, 1), ("ramp", 1000, 64, 1), ("ramp", 700, 128, 4),
                                               ("late_spike", 900, 128, 1), ("late_spike", 333, 64, 3)])
def test_flash_attention_reference_moves(kind, S, hd, nsplit):
    """Scores that keep growing along the keys move the softmax reference many
    times (ramp: key norms grow 4x from the first key to the last); one late
    key whose score tops every earlier one by far more than the exponent range
    (late_spike: every query leans on one direction u, that key is 40 u) must
    be caught before its probability overflows.  Both against the explicit
    softmax."""
    import torch
    say(f"flash_attention reference moves kind={kind} S={S} hd={hd} nsplit={nsplit}")
    B, H, Hk = 1, 4, 2
    r = _rng(12)
    if kind == "ramp":
        q = r.standard_normal((B, H, S, hd), dtype=np.float32)
        k = r.standard_normal((B, Hk, S, hd), dtype=np.float32) * np.linspace(0.5, 2.0, S, dtype=np.float32)[:, None]
    else:
        u = r.standard_normal(hd, dtype=np.float32)
        q = u + 0.5 * r.standard_normal((B, H, S, hd), dtype=np.float32)
        k = r.standard_normal((B, Hk, S, hd), dtype=np.float32)
        k[:, :, S - 10] = 40.0 * u
    q, k = I.bf16_round(q), I.bf16_round(k)
    v = I.bf16_round(r.standard_normal((B, Hk, S, hd), dtype=np.float32))
    spad = N.dit_seq_pad(S)
    vt = np.zeros((B, Hk, hd, spad), np.float32)
    vt[..., :S] = v.transpose(0, 1, 3, 2)
    cfg = I.DiTConfig("att", 0, B, (1, 1, S), H * hd, H, Hk, hd, 128, 0, False, "half2d", (hd // 2, hd // 2), 100.0)
    desc = R.desc_of(cfg)
    out = torch.empty((B * S, H * hd), dtype=torch.bfloat16, device="cuda")
    if nsplit > 1:
        ws = R.alloc_ws(N.dit_attention_workspace_size(desc, nsplit))
        N.dit_flash_attention_split(desc, R.to_dev_bf16(q), R.to_dev_bf16(k), R.to_dev_bf16(vt), out, nsplit, ws)
    else:
        N.dit_flash_attention(desc, R.to_dev_bf16(q), R.to_dev_bf16(k), R.to_dev_bf16(vt), out)
    _sync()
    ref = O.attention(q[0].transpose(1, 0, 2).astype(np.float64), k[0].transpose(1, 0, 2), v[0].transpose(1, 0, 2),
                      H, Hk)
    got = R.to_host_f32(out)
    assert np.isfinite(got).all()
    assert_parity(got, ref, max_rel=2e-2, min_cos=0.9999, what=f"attention {kind}")


def test_flash_attention_closed_forms():
    """V == 1 gives O == 1; Q == 0 gives the mean of V over the keys."""
    import torch
    B, S, H, hd = 1, 200, 2, 128
    r = _rng(5)
    k = I.bf16_round(r.standard_normal((B, H, S, hd), dtype=np.float32))
    cfg = I.DiTConfig("att", 0, B, (1, 1, S), H * hd, H, H, hd, 128, 0, False, "half2d", (64, 64), 100.0)
    spad = N.dit_seq_pad(S)
    vt1 = np.zeros((B, H, hd, spad), np.float32)
    vt1[..., :S] = 1.0
    out = torch.empty((S, H * hd), dtype=torch.bfloat16, device="cuda")
    q = I.bf16_round(r.standard_normal((B, H, S, hd), dtype=np.float32) * 2)
    N.dit_flash_attention(R.desc_of(cfg), R.to_dev_bf16(q), R.to_dev_bf16(k), R.to_dev_bf16(vt1), out)
    _sync()
    np.testing.assert_allclose(R.to_host_f32(out), 1.0, rtol=0, atol=2 ** -7)
    v = I.bf16_round(r.standard_normal((B, H, S, hd), dtype=np.float32))
    vt = np.zeros((B, H, hd, spad), np.float32)
    vt[..., :S] = v.transpose(0, 1, 3, 2)
    N.dit_flash_attention(R.desc_of(cfg), R.to_dev_bf16(np.zeros_like(q)), R.to_dev_bf16(k), R.to_dev_bf16(vt), out)
    _sync()
    mean = v[0].mean(axis=1)       # [H, hd]
    got = R.to_host_f32(out).reshape(S, H, hd)
    np.testing.assert_allclose(got, np.broadcast_to(mean, (S, H, hd)), atol=2e-3)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,Nn,K,rdt,odt,gate,bias", [
    (1, 256, 64, "f32", "f32", True, True),           # a single row
    (300, 512, 320, "f32", "f32", True, False),
    (300, 512, 320, "bf16", "f32", True, True),
    (513, 256, 768, "f32", "bf16", False, False),
    (100, 128, 256, None, "f32", False, True),        # narrow N tile, no residual
    (4096, 384, 128, None, "f32", False, True),       # patch-embed-like K = 128
    (4170, 4096, 256, "f32", "f32", True, True),      # ragged rows: the 320-row tile (one round of tiles)
    (2200, 2048, 256, "f32", "f32", True, True),      # ragged rows: the 8-wave 3-stage 256 x 128 tile (144 tiles)
    (2200, 4096, 128, "bf16", "bf16", True, False),   # ragged rows: the 8-wave 2-stage 128 x 128 tile (576 tiles)
    (4096, 6144, 128, "f32", "f32", True, True),      # column split: 4096 columns of 256 x 256, 2048 of 128 x 256
    (4096, 5120, 128, "bf16", "bf16", True, True),    # column split: 4096 columns of 256 x 256, 1024 of 128 x 128
    (4096, 8192, 128, "f32", "f32", True, True),      # 512 tiles of 256 x 256: two per persistent workgroup
])
def test_gemm_gated_residual(M, Nn, K, rdt, odt, gate, bias):
    import torch
    say(f"gemm_residual M={M} N={Nn} K={K} resid={rdt} out={odt} gate={gate} bias={bias}")
    r = _rng(6)
    a = I.bf16_round(r.standard_normal((M, K), dtype=np.float32))
    w = I.bf16_round(r.standard_normal((Nn, K), dtype=np.float32) * 0.05)
    res = None if rdt is None else r.standard_normal((M, Nn), dtype=np.float32)
    if rdt == "bf16":
        res = I.bf16_round(res)
    g = r.standard_normal(Nn, dtype=np.float32) if gate else None
    bb = r.standard_normal(Nn, dtype=np.float32) if bias else None
    resd = None if res is None else (R.to_dev_f32(res) if rdt == "f32" else R.to_dev_bf16(res))
    out = torch.empty((M, Nn), dtype=torch.float32 if odt == "f32" else torch.bfloat16, device="cuda")
    N.dit_gemm_gated_residual(R.to_dev_bf16(a), R.to_dev_bf16(w), M, Nn, K, resd,
                              N.DIT_F32 if rdt != "bf16" else N.DIT_BF16, R.to_dev_f32(g), R.to_dev_f32(bb), out,
                              N.DIT_F32 if odt == "f32" else N.DIT_BF16)
    _sync()
    ref = O.gated_residual(0.0 if res is None else res, 1.0 if g is None else g, O.linear(a, w))
    if bb is not None:
        ref = ref + bb
    tol = 1e-5 if odt == "f32" else 8e-3
    assert_parity(R.to_host_f32(out), ref, max_rel=tol, min_cos=0.99999, what="gemm_residual")


@pytest.mark.parametrize("gate_fn,kind", [(N.DIT_GATE_TANH, "tanh"), (N.DIT_GATE_SIGMOID, "sigmoid")])
def test_gemm_gated_residual_gate_functions(gate_fn, kind):
    import torch
    M, Nn, K = 300, 512, 320
    r = _rng(13)
    a = I.bf16_round(r.standard_normal((M, K), dtype=np.float32))
    w = I.bf16_round(r.standard_normal((Nn, K), dtype=np.float32) * 0.05)
    res = r.standard_normal((M, Nn), dtype=np.float32)
    g = (r.standard_normal(Nn, dtype=np.float32) * 3).astype(np.float32)
    out = torch.empty((M, Nn), dtype=torch.float32, device="cuda")
    N.dit_gemm_gated_residual(R.to_dev_bf16(a), R.to_dev_bf16(w), M, Nn, K, R.to_dev_f32(res), N.DIT_F32,
                              R.to_dev_f32(g), None, out, N.DIT_F32, gate_fn=gate_fn)
    _sync()
    ref = O.gated_residual(res, O.gate_fn(g.astype(np.float64), kind), O.linear(a, w))
    assert_parity(R.to_host_f32(out), ref, max_rel=1e-5, min_cos=0.99999, what=f"gated residual {kind}")


def test_gemm_residual_in_place_and_identity():
    """W = I gives y = a exactly; resid == out (in place) is legal."""
    import torch
    M, D = 300, 256
    r = _rng(7)
    a = I.bf16_round(r.standard_normal((M, D), dtype=np.float32))
    x = r.standard_normal((M, D), dtype=np.float32)
    xd = R.to_dev_f32(x)
    N.dit_gemm_gated_residual(R.to_dev_bf16(a), R.to_dev_bf16(np.eye(D, dtype=np.float32)), M, D, D, xd, N.DIT_F32,
                              None, None, xd, N.DIT_F32)
    _sync()
    np.testing.assert_array_equal(R.to_host_f32(xd), x + a)


@pytest.mark.parametrize("M,F,K", [(300, 384, 256), (256, 768, 256), (4097, 256, 512), (1, 128, 64),
                                   (4170, 2048, 256),    # ragged rows over one full round of tiles
                                   (2200, 1024, 256),    # the 256 x 128 tile
                                   (3000, 1536, 128),    # the 2-stage 128 x 128 tile (576 tiles)
                                   (4096, 4096, 128),    # 512 tiles of 256 x 256: two per persistent workgroup
                                   (3840, 3456, 64)])    # 405 tiles (not a multiple of 8), a single K tile
def test_gemm_swiglu(M, F, K):
    import torch
    say(f"gemm_swiglu M={M} F={F} K={K}")
    r = _rng(8)
    a = I.bf16_round(r.standard_normal((M, K), dtype=np.float32))
    w = I.bf16_round(r.standard_normal((2 * F, K), dtype=np.float32) * 0.08)
    u = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    N.dit_gemm_swiglu(R.to_dev_bf16(a), R.to_dev_bf16(w), M, F, K, u)
    _sync()
    assert_parity(R.to_host_f32(u), O.swiglu(a, w), max_rel=8e-3, min_cos=0.99999, what="swiglu")


def test_gemm_glu_gelu_tanh_with_clamps():
    """The clamped GELU-tanh GLU; one block of rows is scaled so that gate
    projections reach the tanh-argument clamp and the +-65504 output clamp."""
    import torch
    M, F, K = 300, 384, 256
    r = _rng(14)
    a = r.standard_normal((M, K), dtype=np.float32)
    a[:32] *= 3e3                     # |gate| ~ 1e5 on these rows: both clamps engage
    a[32:64] *= 8.0                   # |gate| ~ 20: the tanh argument clamp
    a = I.bf16_round(a)
    w = I.bf16_round(r.standard_normal((2 * F, K), dtype=np.float32) * 0.08)
    u = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    N.dit_gemm_swiglu(R.to_dev_bf16(a), R.to_dev_bf16(w), M, F, K, u, act=N.DIT_ACT_GELU_TANH)
    _sync()
    got = R.to_host_f32(u)
    ref = O.swiglu(a, w, act="gelu_tanh")
    assert np.isfinite(got).all()
    for sl, what in ((slice(0, 32), "clamped rows"), (slice(32, 64), "large rows"), (slice(64, M), "normal rows")):
        assert_parity(got[sl], ref[sl], max_rel=8e-3, min_cos=0.99999, what=f"gelu glu {what}")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [4096 * 128, 1003, 3])
def test_euler(n):
    r = _rng(9)
    lat = r.standard_normal(n, dtype=np.float32)
    v = r.standard_normal(n, dtype=np.float32)
    sig = O.flowmatch_sigmas(8, 4.0)
    ld = R.to_dev_f32(lat)
    N.euler_flowmatch_update(ld, R.to_dev_f32(v), n, float(sig[2]), float(sig[3]))
    _sync()
    ref = O.euler_update(lat.astype(np.float64), v, np.float32(sig[2]), np.float32(sig[3]))
    np.testing.assert_allclose(R.to_host_f32(ld), ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("dim", [256, 4096, 6144])
def test_timestep_embedding(dim):
    import torch
    out = torch.empty(dim, dtype=torch.float32, device="cuda")
    for s in O.flowmatch_sigmas(8, 4.0):
        t = float(np.float32(1000.0 * s))
        N.dit_timestep_embedding(t, dim, out)
        _sync()
        np.testing.assert_allclose(R.to_host_f32(out), O.timestep_embedding(t, dim), atol=2e-4)

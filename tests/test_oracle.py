"""Pins for the CPU oracle: closed forms, invariants, special cases and
brute-force scalar loops, chosen so that a dropped term, a wrong sign or index
or a transposed operand anywhere in oracle/dit.py fails at least one test."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from oracle import dit as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# tiny shapes for brute force: 2 sequences of a 1x2x3 grid, GQA 2 -> 1
T0 = I.DiTConfig("t0", 9, 2, (1, 2, 3), 16, 2, 1, 8, 24, 12, True,
                 "interleaved3d", (2, 2, 4), 256.0, x_dtype="f32")
T0_HALF = T0.replace(name="t0h", cfg_id=10, cond_dim=0, qk_norm=False, rope="half2d",
                     rope_axes=(4, 4), rope_theta=100.0)


def _rand_weights(cfg, seed=0, affine=True):
    """Weights at a scale that makes every term of the block matter."""
    w = I.block_weights(cfg, 0, affine_random=affine)
    r = np.random.default_rng(seed)
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "w_ada", "b_ada"):
        if w.get(k) is not None:
            w[k] = (w[k] * 10.0).astype(np.float32)   # std 0.2: O(1) branch contributions
    if cfg.qk_norm:
        for k in ("q_g", "k_g"):
            w[k] = (1 + 0.3 * r.standard_normal(cfg.head_dim)).astype(np.float32)
        for k in ("q_b", "k_b"):
            w[k] = (0.3 * r.standard_normal(cfg.head_dim)).astype(np.float32)
    return w


# ---------------------------------------------------------------------------
# brute force: the block as scalar float64 loops, written independently of the
# vectorised oracle (no numpy broadcasting, no reshapes)
# ---------------------------------------------------------------------------
def _bf_silu(z):
    return z / (1.0 + math.exp(-z)) if z > -700 else 0.0


def _bf_ln(row, eps, g=None, b=None):
    n = len(row)
    mu = sum(row) / n
    var = sum((v - mu) ** 2 for v in row) / n
    r = 1.0 / math.sqrt(var + eps)
    out = [(v - mu) * r for v in row]
    if g is not None:
        out = [out[i] * float(g[i]) + float(b[i]) for i in range(n)]
    return out


def _bf_angle(cfg, p, m):
    """Angle of pair slot m for integer position p=(t,h,w)."""
    cols = [0, 1, 2] if cfg.rope == "interleaved3d" else [1, 2]
    start = 0
    for col, da in zip(cols, cfg.rope_axes):
        if m < start + da // 2:
            j = m - start
            return float(p[col]) * cfg.rope_theta ** (-2.0 * j / da)
        start += da // 2
    raise AssertionError


def _bf_rope(vec, cfg, p):
    hd = len(vec)
    out = list(vec)
    for m in range(hd // 2):
        a_i, b_i = (2 * m, 2 * m + 1) if cfg.rope == "interleaved3d" else (m, m + hd // 2)
        th = _bf_angle(cfg, p, m)
        a, b = vec[a_i], vec[b_i]
        out[a_i] = a * math.cos(th) - b * math.sin(th)
        out[b_i] = a * math.sin(th) + b * math.cos(th)
    return out


def _bf_matvec(W, v):
    return [sum(float(W[o][i]) * v[i] for i in range(len(v))) for o in range(len(W))]


def bf_block(x, c, w, cfg, pos):
    N, D = x.shape
    H, Hk, hd, S, eps = cfg.heads, cfg.kv_heads, cfg.head_dim, cfg.seq, cfg.eps
    if cfg.cond_dim:
        sc = [_bf_silu(float(v)) for v in c]
        m = [a + float(b) for a, b in zip(_bf_matvec(w["w_ada"], sc), w["b_ada"])]
        sh1, s1, g1, sh2, s2, g2 = (m[i * D:(i + 1) * D] for i in range(6))
    else:
        sh1 = s1 = sh2 = s2 = [0.0] * D
        g1 = g2 = [1.0] * D

    def pre(row, sh, s, which):
        if cfg.cond_dim:
            n = _bf_ln(row, eps)
            return [n[i] * (1.0 + s[i]) + sh[i] for i in range(D)]
        return _bf_ln(row, eps, w[which + "_g"], w[which + "_b"])

    Q, K, V = [], [], []
    for t in range(N):
        h = pre([float(v) for v in x[t]], sh1, s1, "ln1")
        qkv = _bf_matvec(w["w_qkv"], h)
        qs, ks, vs = [], [], []
        for hh in range(H + 2 * Hk):
            vec = qkv[hh * hd:(hh + 1) * hd]
            if hh < H + Hk:
                if cfg.qk_norm:
                    g, b = (w["q_g"], w["q_b"]) if hh < H else (w["k_g"], w["k_b"])
                    vec = _bf_ln(vec, eps, g, b)
                vec = _bf_rope(vec, cfg, pos[t % S])
            (qs if hh < H else ks if hh < H + Hk else vs).append(vec)
        Q.append(qs), K.append(ks), V.append(vs)
    out = np.zeros((N, D))
    for t in range(N):
        b0 = (t // S) * S
        att = []
        for hh in range(H):
            g = hh // (H // Hk)
            sc = [sum(Q[t][hh][d] * K[u][g][d] for d in range(hd)) / math.sqrt(hd) for u in range(b0, b0 + S)]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            att += [sum(e[u - b0] / z * V[u][g][d] for u in range(b0, b0 + S)) for d in range(hd)]
        o = _bf_matvec(w["w_o"], att)
        x1 = [float(x[t][i]) + g1[i] * o[i] for i in range(D)]
        h2 = pre(x1, sh2, s2, "ln2")
        gu = _bf_matvec(w["w_gate_up"], h2)
        F = len(gu) // 2
        ff = [_bf_silu(gu[i]) * gu[F + i] for i in range(F)]
        dn = _bf_matvec(w["w_down"], ff)
        out[t] = [x1[i] + g2[i] * dn[i] for i in range(D)]
    return out


@pytest.mark.parametrize("cfg", [T0, T0_HALF], ids=["adaln_gqa_interleaved3d", "vit_half2d"])
def test_block_matches_brute_force(cfg):
    w = _rand_weights(cfg)
    x = np.random.default_rng(1).standard_normal((cfg.tokens, cfg.hidden))
    # off-origin positions so that every rotary axis rotates
    pos = I.positions(cfg) + np.array([3, 1, 2])
    c = np.random.default_rng(2).standard_normal(cfg.cond_dim) if cfg.cond_dim else None
    got = O.block_forward(x, c, w, cfg, pos)
    ref = bf_block(x, c, w, cfg, pos)
    assert np.abs(got - ref).max() < 1e-10 * max(1.0, np.abs(ref).max())
    # the branch contributions are not negligible (the test would be vacuous otherwise)
    assert np.abs(ref - x).max() > 0.1


def test_sampled_rows_equal_full():
    cfg = T0
    w = _rand_weights(cfg)
    x = np.random.default_rng(3).standard_normal((cfg.tokens, cfg.hidden))
    c = np.random.default_rng(4).standard_normal(cfg.cond_dim)
    pos = I.positions(cfg)
    full = O.block_forward(x, c, w, cfg, pos)
    rows = np.array([0, 5, 7, 11])
    part = O.block_forward(x, c, w, cfg, pos, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


# ---------------------------------------------------------------------------
# special cases
# ---------------------------------------------------------------------------
def test_p1_zero_adaln_is_identity_bitwise():
    """AdaLN-Zero: zero modulation weights give shift=scale=gate=0, so out == x."""
    cfg = I.C1
    w = I.block_weights(cfg, 0, zero_ada=True)
    x = I.block_x(cfg)
    out = O.block_forward(x, I.cond(cfg), w, cfg, I.positions(cfg), dtype=np.float32)
    assert np.array_equal(out, x)


def test_p2_zero_shift_scale_gives_plain_layernorm():
    cfg = T0
    w = _rand_weights(cfg)
    D = cfg.hidden
    w["w_ada"] = np.zeros_like(w["w_ada"])
    b = np.zeros(6 * D, np.float32)
    b[2 * D:3 * D] = 1.0        # gate1 = 1
    w["b_ada"] = b
    w["w_o"] = np.zeros_like(w["w_o"])
    x = np.random.default_rng(5).standard_normal((cfg.tokens, D))
    keep = {}
    O.block_forward(x, np.ones(cfg.cond_dim), w, cfg, I.positions(cfg), keep=keep)
    xc = x - x.mean(1, keepdims=True)
    np.testing.assert_allclose(keep["h"], xc / np.sqrt((xc ** 2).mean(1, keepdims=True) + cfg.eps), rtol=1e-12)
    np.testing.assert_array_equal(keep["x1"], x)


def test_p9_zero_gate_weights_kill_ffn():
    cfg = T0
    w = _rand_weights(cfg)
    F = cfg.ffn
    w["w_gate_up"][:F] = 0
    x = np.random.default_rng(6).standard_normal((cfg.tokens, cfg.hidden))
    keep = {}
    out = O.block_forward(x, np.ones(cfg.cond_dim), w, cfg, I.positions(cfg), keep=keep)
    np.testing.assert_array_equal(out, keep["x1"])


def test_silu_closed_form():
    z = np.array([0.0, 1.0, -1.0, 2.0, -30.0, 30.0])
    ref = np.array([0.0, 1 / (1 + math.exp(-1)), -1 / (1 + math.e), 2 / (1 + math.exp(-2)),
                    -30 / (1 + math.exp(30)), 30 / (1 + math.exp(-30))])
    np.testing.assert_allclose(O.silu(z), ref, rtol=1e-15, atol=1e-300)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout,axes", [("interleaved3d", (32, 48, 48)), ("half2d", (32, 32))])
def test_p3_rope_position_zero_identity_and_norm(layout, axes):
    hd = sum(axes)
    spec = T0.replace(rope=layout, rope_axes=axes, head_dim=hd)
    x = np.random.default_rng(7).standard_normal((5, 3, hd))
    pos0 = np.zeros((5, 3), np.int64)
    assert np.array_equal(O.apply_rope(x, O.rope_angles(pos0, spec), layout), x)
    pos = np.random.default_rng(8).integers(0, 64, (5, 3))
    y = O.apply_rope(x, O.rope_angles(pos, spec), layout)
    # every rotated pair keeps its length
    if layout == "interleaved3d":
        na, nb = x[..., 0::2] ** 2 + x[..., 1::2] ** 2, y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    else:
        na = x[..., :hd // 2] ** 2 + x[..., hd // 2:] ** 2
        nb = y[..., :hd // 2] ** 2 + y[..., hd // 2:] ** 2
    np.testing.assert_allclose(na, nb, rtol=1e-12)


def test_rope_angles_closed_form():
    """theta^(-2j/d) per axis chunk, at the ERNIE axes [32,48,48], theta 256."""
    spec = I.C3
    pos = np.array([[1, 2, 3]])
    a = O.rope_angles(pos, spec)[0]
    assert a.shape == (64,)
    assert a[0] == 1.0 and a[16] == 2.0 and a[40] == 3.0           # j = 0 of each axis
    assert math.isclose(a[1], 256 ** (-2 / 32), rel_tol=1e-15)
    assert math.isclose(a[17], 2 * 256 ** (-2 / 48), rel_tol=1e-15)
    assert math.isclose(a[63], 3 * 256 ** (-46 / 48), rel_tol=1e-15)


@pytest.mark.parametrize("cfg", [T0, T0_HALF])
def test_p4_relative_position_invariance(cfg):
    """RoPE scores depend only on position differences: shifting every token
    along each axis leaves the block output unchanged (t axis included)."""
    w = _rand_weights(cfg)
    x = np.random.default_rng(9).standard_normal((cfg.tokens, cfg.hidden))
    c = np.random.default_rng(10).standard_normal(cfg.cond_dim) if cfg.cond_dim else None
    pos = I.positions(cfg)
    a = O.block_forward(x, c, w, cfg, pos)
    b = O.block_forward(x, c, w, cfg, pos + np.array([7, 3, 5]))
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)
    # and a non-uniform change of positions does change it (the rotation is live)
    pos2 = pos.copy()
    pos2[0] += np.array([1, 1, 1])
    assert np.abs(O.block_forward(x, c, w, cfg, pos2) - a).max() > 1e-4


def test_p7_rms_norm_commutes_with_rope():
    spec = T0
    x = np.random.default_rng(11).standard_normal((6, 2, 8))
    ang = O.rope_angles(np.random.default_rng(12).integers(0, 9, (6, 3)), spec)
    a = O.rms_norm(O.apply_rope(x, ang, spec.rope), 1e-6)
    b = O.apply_rope(O.rms_norm(x, 1e-6), ang, spec.rope)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_p7_layernorm_moments():
    x = np.random.default_rng(13).standard_normal((7, 33)) * 5 + 3
    y = O.layer_norm(x, 0.0)
    np.testing.assert_allclose(y.mean(1), 0, atol=1e-13)
    np.testing.assert_allclose((y ** 2).mean(1), 1, rtol=1e-12)
    y = O.rms_norm(x, 0.0)
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(1)), 1, rtol=1e-12)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def test_p5_softmax_rows_sum_to_one():
    s = np.random.default_rng(14).standard_normal((9, 40)) * 30
    np.testing.assert_allclose(O.softmax_rows(s).sum(1), 1, rtol=1e-14)


def test_p5_attention_closed_forms():
    r = np.random.default_rng(15)
    q, k = r.standard_normal((10, 4, 8)), r.standard_normal((10, 2, 8))
    v1 = np.ones((10, 2, 8))
    np.testing.assert_allclose(O.attention(q, k, v1, 4, 2), 1, rtol=1e-14)
    v = r.standard_normal((10, 2, 8))
    o = O.attention(np.zeros_like(q), k, v, 4, 2).reshape(10, 4, 8)
    for h in range(4):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(v[:, h // 2].mean(0), (10, 8)), rtol=1e-12)


def test_p6_attention_brute_force_and_gqa():
    r = np.random.default_rng(16)
    S, H, Hk, hd = 7, 6, 2, 4
    q, k, v = r.standard_normal((S, H, hd)), r.standard_normal((S, Hk, hd)), r.standard_normal((S, Hk, hd))
    got = O.attention(q, k, v, H, Hk).reshape(S, H, hd)
    for i in range(S):
        for h in range(H):
            g = h // 3
            sc = [sum(q[i, h, d] * k[j, g, d] for d in range(hd)) / 2.0 for j in range(S)]
            e = [math.exp(s - max(sc)) for s in sc]
            for d in range(hd):
                ref = sum(e[j] * v[j, g, d] for j in range(S)) / sum(e)
                assert abs(got[i, h, d] - ref) < 1e-12
    # GQA equals MHA with the KV heads replicated per group
    mha = O.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), H, H)
    np.testing.assert_allclose(mha.reshape(S, H, hd), got, rtol=1e-13)


# ---------------------------------------------------------------------------
# equivariance / batching
# ---------------------------------------------------------------------------
def test_p10_token_permutation_equivariance():
    cfg = T0.replace(batch=1, grid=(2, 2, 3))
    w = _rand_weights(cfg)
    x = np.random.default_rng(17).standard_normal((cfg.tokens, cfg.hidden))
    c = np.random.default_rng(18).standard_normal(cfg.cond_dim)
    pos = I.positions(cfg)
    perm = np.random.default_rng(19).permutation(cfg.tokens)
    a = O.block_forward(x, c, w, cfg, pos)
    b = O.block_forward(x[perm], c, w, cfg, pos[perm])
    np.testing.assert_allclose(b, a[perm], rtol=1e-10, atol=1e-12)


def test_p11_batch_element_alone_equals_in_batch():
    cfg = T0_HALF.replace(batch=3)
    w = _rand_weights(cfg)
    x = np.random.default_rng(20).standard_normal((cfg.tokens, cfg.hidden))
    pos = I.positions(cfg)
    full = O.block_forward(x, None, w, cfg, pos)
    S = cfg.seq
    one = O.block_forward(x[S:2 * S], None, w, cfg.replace(batch=1), pos)
    np.testing.assert_allclose(one, full[S:2 * S], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# loop pieces
# ---------------------------------------------------------------------------
def test_p12_sigmas_golden_and_constant_velocity():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "sigmas_8steps_shift4.txt")) if l[0] != "#"]
    exact = [Fraction(int(n), int(d)) for _, n, d in rows]
    sig = O.flowmatch_sigmas(8, 4.0)
    assert len(sig) == 9
    for s, e in zip(sig, exact):
        assert abs(s - float(e)) < 1e-15
    lat0 = np.random.default_rng(21).standard_normal((4, 3))
    v = np.random.default_rng(22).standard_normal((4, 3))
    lat = lat0
    for i in range(8):
        lat = O.euler_update(lat, v, sig[i], sig[i + 1])
    np.testing.assert_allclose(lat, lat0 - v, rtol=1e-13, atol=1e-14)


def test_p13_timestep_embedding_closed_form():
    e0 = O.timestep_embedding(0.0, 16)
    np.testing.assert_array_equal(e0, np.r_[np.ones(8), np.zeros(8)])
    e = O.timestep_embedding(500.0, 8)
    w = [1.0, 10000 ** -0.25, 10000 ** -0.5, 10000 ** -0.75]
    np.testing.assert_allclose(e, [math.cos(500 * x) for x in w] + [math.sin(500 * x) for x in w], rtol=1e-12)


def test_final_layer_chunk_order_scale_then_shift():
    """Final norm chunks are (scale, shift), the reverse of the per-layer order."""
    spec = T0
    D, C = spec.hidden, 3
    x = np.random.default_rng(23).standard_normal((5, D))
    edges = {"w_fmod": np.zeros((2 * D, spec.cond_dim)), "b_fmod": np.r_[np.full(D, 2.0), np.full(D, 0.5)],
             "w_out": np.eye(C, D), "b_out": np.zeros(C)}
    v = O.final_layer(x, np.zeros(spec.cond_dim), edges, spec)
    n = O.layer_norm(x, spec.eps)
    np.testing.assert_allclose(v, (n * 3.0 + 0.5)[:, :C], rtol=1e-12)


def test_stack_loop_resume_equals_uninterrupted():
    cfg = T0.replace(batch=1, layers=2, latent_dim=4)
    blocks = [_rand_weights(cfg, seed=l) for l in range(2)]
    edges = {"w_in": np.random.default_rng(24).standard_normal((cfg.hidden, 4)) * 0.3,
             "b_in": np.zeros(cfg.hidden), "w_fmod": np.random.default_rng(25).standard_normal((2 * cfg.hidden, cfg.cond_dim)) * 0.1,
             "b_fmod": np.zeros(2 * cfg.hidden), "w_out": np.random.default_rng(26).standard_normal((4, cfg.hidden)) * 0.3,
             "b_out": np.zeros(4)}
    pos = I.positions(cfg)
    lat0 = np.random.default_rng(27).standard_normal((cfg.tokens, 4))
    full = O.denoise(lat0, blocks, edges, cfg, pos, 4, 4.0)
    sig = O.flowmatch_sigmas(4, 4.0)
    lat = lat0
    for i in range(2):
        lat = O.euler_update(lat, O.stack_step(lat, sig[i], blocks, edges, cfg, pos), sig[i], sig[i + 1])
    resumed = O.denoise(lat, blocks, edges, cfg, pos, 4, 4.0, start=2)
    np.testing.assert_array_equal(resumed, full)


# ---------------------------------------------------------------------------
# the stack step's edges, from scalar loops: timestep features, patch
# embedding with its bias, the blocks, the final (scale, shift) linear of the
# raw conditioning (no SiLU) and the output projection with its bias
# ---------------------------------------------------------------------------
def _bf_temb(t, dim):
    half = dim // 2
    w = [10000.0 ** (-j / half) for j in range(half)]
    return [math.cos(t * x) for x in w] + [math.sin(t * x) for x in w]


def bf_stack_step(lat, sigma, blocks, edges, cfg, pos):
    """ERNIE page §IV (36 layers per step) and §V Bug 4 (the final layer's
    linear of the conditioning), zml-flow-rs page §IV (flip_sin_to_cos
    timestep sinusoid at t = 1000 sigma), as scalar float64 loops."""
    c = _bf_temb(1000.0 * sigma, cfg.cond_dim)
    D, C = cfg.hidden, cfg.latent_dim
    x = np.array([[sum(float(edges["w_in"][o][i]) * float(row[i]) for i in range(C)) + float(edges["b_in"][o])
                   for o in range(D)] for row in lat])
    for w in blocks:
        x = bf_block(x, np.array(c), w, cfg, pos)
    m = [a + float(b) for a, b in zip(_bf_matvec(edges["w_fmod"], c), edges["b_fmod"])]
    scale, shift = m[:D], m[D:]
    v = []
    for row in x:
        n = _bf_ln([float(e) for e in row], cfg.eps)
        h = [n[i] * (1.0 + scale[i]) + shift[i] for i in range(D)]
        v.append([a + float(b) for a, b in zip(_bf_matvec(edges["w_out"], h), edges["b_out"])])
    return np.array(v)


def _stack_case():
    cfg = T0.replace(batch=1, layers=2, latent_dim=4)
    D, Dc, C = cfg.hidden, cfg.cond_dim, cfg.latent_dim
    r = np.random.default_rng(28)
    blocks = [_rand_weights(cfg, seed=l) for l in range(cfg.layers)]
    # every edge tensor nonzero and at a scale where it moves the velocity
    edges = {"w_in": r.standard_normal((D, C)) * 0.5, "b_in": r.standard_normal(D) * 0.5,
             "w_fmod": r.standard_normal((2 * D, Dc)) * 0.3, "b_fmod": r.standard_normal(2 * D) * 0.3,
             "w_out": r.standard_normal((C, D)) * 0.3, "b_out": r.standard_normal(C) * 0.3}
    lat = r.standard_normal((cfg.tokens, C))
    return cfg, blocks, edges, lat, I.positions(cfg) + np.array([1, 2, 0])


def test_stack_step_matches_brute_force():
    cfg, blocks, edges, lat, pos = _stack_case()
    sigma = 0.8
    ref = bf_stack_step(lat, sigma, blocks, edges, cfg, pos)
    got = O.stack_step(lat, sigma, blocks, edges, cfg, pos)
    assert np.abs(got - ref).max() < 1e-10 * max(1.0, np.abs(ref).max())
    assert np.abs(ref).max() > 0.5


def test_stack_step_pin_catches_planted_edge_mistakes(monkeypatch):
    """Three plausible misreadings of the edges, each planted in the oracle
    (on the CPU), move the velocity far beyond the pin's tolerance: the
    timestep fed as sigma instead of 1000 sigma, the patch-embedding bias
    dropped, SiLU applied to the conditioning before the final linear."""
    cfg, blocks, edges, lat, pos = _stack_case()
    sigma = 0.8
    ref = bf_stack_step(lat, sigma, blocks, edges, cfg, pos)
    tol = 1e-10 * max(1.0, np.abs(ref).max())

    def worst(fn):
        return np.abs(fn() - ref).max()

    temb = O.timestep_embedding
    with monkeypatch.context() as m:
        m.setattr(O, "timestep_embedding", lambda t, dim, dtype=O.F64: temb(t / 1000.0, dim, dtype))
        assert worst(lambda: O.stack_step(lat, sigma, blocks, edges, cfg, pos)) > 1e3 * tol
    no_bias = dict(edges, b_in=np.zeros_like(edges["b_in"]))     # an oracle that ignores b_in
    assert worst(lambda: O.stack_step(lat, sigma, blocks, no_bias, cfg, pos)) > 1e3 * tol
    final = O.final_layer
    with monkeypatch.context() as m:
        m.setattr(O, "final_layer", lambda x, c, e, s, dtype=O.F64: final(x, O.silu(c), e, s, dtype))
        assert worst(lambda: O.stack_step(lat, sigma, blocks, edges, cfg, pos)) > 1e3 * tol
    # and unplanted, the same comparison holds
    assert worst(lambda: O.stack_step(lat, sigma, blocks, edges, cfg, pos)) < tol


# ---------------------------------------------------------------------------
# the oracle's own rounding floor (fp32 vs fp64) and the workload dims
# ---------------------------------------------------------------------------
def test_p14_fp32_vs_fp64_floor_c1():
    cfg = I.C1
    w, x, c, pos = I.block_weights(cfg), I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    a = O.block_forward(x, c, w, cfg, pos, dtype=np.float64)
    b = O.block_forward(x, c, w, cfg, pos, dtype=np.float32)
    d, dd = b - a, a - x
    assert np.abs(d).max() / np.abs(a).max() < 1e-5
    assert np.abs(d).max() / np.abs(dd).max() < 1e-4


def test_workload_dims_match_ernie_page():
    g = json.load(open(os.path.join(GOLDEN, "ernie_dims.json")))
    for c in (I.C3, I.C4):
        assert c.hidden == g["hidden"] and c.ffn == g["ffn"] and c.heads == g["heads"]
        assert c.head_dim == g["head_dim"] and list(c.rope_axes) == g["rope_axes"]
        assert c.rope_theta == g["rope_theta"] and c.qk_norm == g["qk_norm"]
        assert c.seq == g["latent_tokens"] and list(c.grid[1:]) == g["latent_grid"]
    assert I.C4.layers == g["layers"] and I.C4.latent_dim == g["latent_channels"]
    assert I.STACK_STEPS == g["euler_steps"] and I.STACK_SHIFT == g["scheduler_shift"]


# ---------------------------------------------------------------------------
# joint text + image sequence (ERNIE page, "Token Layout" and §VII Decision 3)
# ---------------------------------------------------------------------------
def test_joint_positions_follow_the_token_layout():
    g = json.load(open(os.path.join(GOLDEN, "ernie_dims.json")))
    cfg = I.C3_JOINT
    assert cfg.text_len == g["joint_text_tokens"] and cfg.seq == g["joint_tokens"]
    assert g["joint_order"] == "spatial_first" and not cfg.text_first
    pos = I.positions(cfg)
    n_sp = g["latent_tokens"]
    assert pos.shape == (g["joint_tokens"], 3)
    sp, tx = pos[:n_sp], pos[n_sp:]
    assert (sp[:, 0] == g["joint_text_tokens"]).all()                   # spatial t = text_len
    hh, ww = g["latent_grid"]
    np.testing.assert_array_equal(sp[:, 1], np.arange(n_sp) // ww)     # row-major h, w
    np.testing.assert_array_equal(sp[:, 2], np.arange(n_sp) % ww)
    np.testing.assert_array_equal(tx[:, 0], np.arange(g["joint_text_tokens"]))   # text (j, 0, 0)
    assert (tx[:, 1:] == 0).all()
    # text-first order: the same ids, text rows moved to the front
    tf = I.positions(cfg.replace(text_first=True))
    np.testing.assert_array_equal(tf, np.concatenate([tx, sp]))


def test_joint_text_tokens_rotate_only_along_t():
    """Text tokens sit at h = w = 0: their rotation on the h and w chunks of
    the head dim is the identity, and on the t chunk it is position j."""
    cfg = I.C1_JOINT
    pos = I.positions(cfg)
    ang = O.rope_angles(pos, cfg)
    t_pairs = cfg.rope_axes[0] // 2
    text = ang[cfg.spatial:]
    assert np.all(text[:, t_pairs:] == 0.0)
    j = np.arange(cfg.text_len, dtype=np.float64)
    np.testing.assert_allclose(text[:, 0], j)                             # pair 0 of t: angle = position
    assert np.all(ang[: cfg.spatial, 0] == cfg.text_len)                  # spatial t offset by text_len


def test_joint_text_first_is_a_row_permutation():
    """Moving the text rows to the front (with their positions) permutes the
    block's output rows and changes nothing else."""
    cfg = I.C1_JOINT
    cft = I.C1_JOINT_TF
    w, c = I.block_weights(cfg), I.cond(cfg)
    x = I.block_x(cfg)
    n = cfg.spatial
    perm = np.r_[np.arange(n, cfg.seq), np.arange(n)]      # text-first row order
    a = O.block_forward(x, c, w, cfg, I.positions(cfg))
    b = O.block_forward(x[perm], c, w, cft, I.positions(cft))
    np.testing.assert_allclose(b, a[perm], rtol=1e-10, atol=1e-12)



# ---------------------------------------------------------------------------
# semantics switches: norm kind, GLU activation, gate function, modulation
# chunks, qk-norm / RoPE order
# ---------------------------------------------------------------------------
def test_gelu_tanh_against_erf_gelu_and_its_clamps():
    """ERNIE page §V Bug 1: GELU in its tanh approximation with the argument
    clamped to +-20 and the result to +-65504."""
    import scipy.special as sp
    x = np.linspace(-10.0, 10.0, 20001)
    exact = 0.5 * x * (1.0 + sp.erf(x / np.sqrt(2.0)))      # GELU's definition, x Phi(x)
    assert np.abs(O.gelu_tanh(x) - exact).max() < 5e-4         # the tanh approximation's deviation
    # odd part: f(x) - f(-x) = x, since tanh is odd (holds through the argument clamp)
    x = np.linspace(-50.0, 50.0, 10001)
    np.testing.assert_allclose(O.gelu_tanh(x) - O.gelu_tanh(-x), x, rtol=0, atol=1e-12)
    # the clamps: large gate projections stay finite and saturate
    g = O.gelu_tanh(np.array([30.0, -30.0, 1e6, -1e6]))
    assert g[0] == 30.0 and abs(g[1]) < 1e-12 and g[2] == 65504.0 and abs(g[3]) < 1e-6
    g32 = O.gelu_tanh(np.array([1e30], np.float32))           # z^3 overflows fp32: still finite
    assert np.isfinite(g32).all() and g32[0] == 65504.0


def _zero_ada_weights(cfg, b_gate=None):
    w = I.block_weights(cfg)
    w["w_ada"] = np.zeros_like(w["w_ada"])
    return w


def test_gate_function_tanh_and_sigmoid():
    """With W_ada = 0 the modulation is b_ada, so a tanh / sigmoid gate equals
    the identity gate with those functions applied to b_ada's gate chunks; a
    zero tanh gate kills both branches."""
    base = I.C1.replace(name="t_gate")
    D = base.hidden
    x, c, pos = I.block_x(base), I.cond(base), I.positions(base)
    w = _zero_ada_weights(base)
    for kind, f in (("tanh", np.tanh), ("sigmoid", lambda g: 1.0 / (1.0 + np.exp(-g)))):
        got = O.block_forward(x, c, w, base.replace(gate=kind), pos)
        w2 = dict(w)
        b = np.array(w["b_ada"], np.float64)
        for chunk in (2, 5):                                    # gate1, gate2
            b[chunk * D:(chunk + 1) * D] = f(b[chunk * D:(chunk + 1) * D])
        w2["b_ada"] = b
        ref = O.block_forward(x, c, w2, base, pos)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    w0 = dict(w)
    w0["b_ada"] = np.zeros_like(w["b_ada"])
    np.testing.assert_array_equal(O.block_forward(x, c, w0, base.replace(gate="tanh"), pos), x)


def test_scale_gate_modulation_is_the_six_way_one_with_zero_shift():
    """mod = "scale_gate" (chunks scale1, gate1, scale2, gate2; no shift) equals
    the six-way modulation whose shift rows are zero."""
    cfg = I.C1.replace(name="t_sg", mod="scale_gate")
    D = cfg.hidden
    w4 = I.block_weights(cfg)
    assert w4["w_ada"].shape[0] == 4 * D
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    got = O.block_forward(x, c, w4, cfg, pos)
    w6 = dict(w4)
    wz, bz = np.zeros((D, cfg.cond_dim)), np.zeros(D)
    W, B = w4["w_ada"], w4["b_ada"]
    w6["w_ada"] = np.concatenate([wz, W[:D], W[D:2 * D], wz, W[2 * D:3 * D], W[3 * D:]])
    w6["b_ada"] = np.concatenate([bz, B[:D], B[D:2 * D], bz, B[2 * D:3 * D], B[3 * D:]])
    ref = O.block_forward(x, c, w6, cfg.replace(mod="shift_scale_gate"), pos)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_rmsnorm_of_centred_rows_is_layernorm():
    x = np.random.default_rng(31).standard_normal((7, 96))
    xc = x - x.mean(axis=-1, keepdims=True)
    np.testing.assert_allclose(O.rms_norm(xc, 1e-6), O.layer_norm(x, 1e-6), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.rms_norm(5.0 * xc, 0.0), O.rms_norm(xc, 0.0), rtol=1e-12)
    spec = I.C1.replace(norm="rmsnorm")
    g, b = np.full(96, 2.0), np.full(96, 0.5)
    np.testing.assert_allclose(O.norm(x, spec, g, b), O.rms_norm(x, spec.eps) * 2.0 + 0.5, rtol=1e-12)


def test_qk_order_rope_then_norm():
    """RoPE is a rotation of pairs: it preserves the RMS, so with RMSNorm
    (gamma 1, beta 0) both orders agree; at position 0 (identity rotation) they
    agree for LayerNorm too; in general LayerNorm does not commute with RoPE."""
    cfg = I.C1.replace(name="t_order")
    w = I.block_weights(cfg)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    w1 = dict(w, q_g=np.ones(cfg.head_dim), k_g=np.ones(cfg.head_dim),
              q_b=np.zeros(cfg.head_dim), k_b=np.zeros(cfg.head_dim))
    rms = cfg.replace(norm="rmsnorm")
    np.testing.assert_allclose(O.block_forward(x, c, w1, rms.replace(qk_order="rope_norm"), pos),
                               O.block_forward(x, c, w1, rms, pos), rtol=1e-9, atol=1e-10)
    z = np.zeros_like(pos)
    np.testing.assert_allclose(O.block_forward(x, c, w, cfg.replace(qk_order="rope_norm"), z),
                               O.block_forward(x, c, w, cfg, z), rtol=1e-10, atol=1e-12)
    a = O.block_forward(x, c, w, cfg.replace(qk_order="rope_norm"), pos)
    b = O.block_forward(x, c, w, cfg, pos)
    assert np.abs((a - x) - (b - x)).max() > 1e-3 * np.abs(b - x).max()


# ---------------------------------------------------------------------------
# W8A8 with the 256-point Hadamard rotation (zml-flow-rs page §VII)
# ---------------------------------------------------------------------------
def test_hadamard_is_the_library_sylvester_matrix():
    from scipy.linalg import hadamard as sylvester
    H = O.hadamard(256)
    np.testing.assert_array_equal(H * 16.0, sylvester(256).astype(np.float64))
    np.testing.assert_array_equal(H, H.T)
    np.testing.assert_array_equal(H @ H.T, np.eye(256))   # entries +-1/16: every product and sum is exact


def test_rotation_is_blockwise_and_orthogonal():
    r = np.random.default_rng(41)
    x, w = r.standard_normal((5, 768)), r.standard_normal((7, 768))
    # rotation invariance (x H)(W H)^T = x W^T, the identity the format rests on
    np.testing.assert_allclose(O.rotate_h256(x) @ O.rotate_h256(w).T, x @ w.T, rtol=1e-12, atol=1e-11)
    # each run of 256 inputs is rotated on its own: a unit input at offset 5 of
    # the second run becomes row 5 of H256 in that run only, by the sign formula
    e = np.zeros(768)
    e[256 + 5] = 1.0
    got = O.rotate_h256(e)
    assert not got[:256].any() and not got[512:].any()
    expect = np.array([(-1.0) ** bin(5 & j).count("1") / 16.0 for j in range(256)])
    np.testing.assert_array_equal(got[256:512], expect)
    # a constant run maps to (16 c, 0, ..., 0)
    c = np.full(256, 0.75)
    np.testing.assert_array_equal(O.rotate_h256(c), np.r_[16 * 0.75, np.zeros(255)])


def test_quantize_rows_closed_form():
    v = np.zeros((3, 8), np.float32)
    v[0, :4] = [1.0, -0.5, 0.25, 0.125]   # amax 1: 127, -63.5 -> -64 (half to even), 31.75 -> 32, 15.875 -> 16
    v[1, :3] = [-2.0, 1.0, 0.0]           # amax 2 at a negative value: -127, 63.5 -> 64 (half to even), 0
    q, s = O.quantize_rows(v)
    assert q.dtype == np.int8 and s.dtype == np.float32
    np.testing.assert_array_equal(q[0, :4], [127, -64, 32, 16])
    np.testing.assert_array_equal(q[1, :3], [-127, 64, 0])
    assert not q[2].any() and s[2] == 0.0                      # a zero row
    assert s[0] == np.float32(1.0) / np.float32(127.0) and s[1] == np.float32(2.0) / np.float32(127.0)


def test_quantize_rows_range_and_half_step_error():
    r = np.random.default_rng(43)
    v = r.standard_normal((64, 512)) * np.exp(2.0 * r.standard_normal((64, 1)))
    q, s = O.quantize_rows(v)
    assert np.abs(q.astype(int)).max() == 127
    i = np.abs(v.astype(np.float32)).argmax(axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(64), i].astype(int)), 127)   # the row max maps to +-127
    assert (np.sign(q) * np.sign(v) >= 0).all()                                    # no sign flips
    err = np.abs(q * s[:, None].astype(np.float64) - v)
    assert (err <= s[:, None] * (0.5 + 1e-4)).all()                                 # within half a step


def _bf_rot(row):
    out = []
    for b0 in range(0, len(row), 256):
        for j in range(256):
            acc = 0.0
            for a in range(256):
                acc += row[b0 + a] if bin(a & j).count("1") % 2 == 0 else -row[b0 + a]
            out.append(acc / 16.0)
    return out


def _bf_quant(row):
    v = [np.float32(t) for t in row]
    amax = max(abs(t) for t in v)
    inv = np.float32(127.0) / amax
    codes = [max(-127, min(127, round(float(np.float32(t * inv))))) for t in v]   # round(): half to even
    return codes, float(amax / np.float32(127.0))


def test_w8a8_linear_brute_force():
    """The W8A8 H256 product from scalar loops: rotation from the sign formula,
    codes from per-element float32 steps, integer dot products in Python ints."""
    r = np.random.default_rng(47)
    x = r.standard_normal((3, 512))
    w = r.standard_normal((2, 512)) * 0.02
    qx = [_bf_quant(_bf_rot(list(row))) for row in x]
    qw = [_bf_quant(_bf_rot(list(row))) for row in w]
    ref = np.array([[sx * sw * sum(a * b for a, b in zip(cx, cw)) for (cw, sw) in qw] for (cx, sx) in qx])
    np.testing.assert_allclose(O.w8a8_linear(x, w), ref, rtol=1e-12, atol=0)
    # the prepared-weight form is the same product
    np.testing.assert_array_equal(O.w8a8_linear(x, O.quantize_h256(w)), O.w8a8_linear(x, w))


def test_w8a8_error_within_the_quantisation_bound():
    """With xr = x H = sx (qx + dx), wr = W H = sw (qw + dw), |d| <= 1/2:
    |x W^T - y8| <= sum_k |xr_k| sw / 2 + |wr_k| sx / 2 + sx sw / 4."""
    r = np.random.default_rng(53)
    K = 1024
    x = r.standard_normal((16, K))
    w = r.standard_normal((24, K)) * 0.02
    y = O.w8a8_linear(x, w)
    exact = x @ w.T
    xr, wr = O.rotate_h256(x), O.rotate_h256(w)
    _, sx = O.quantize_rows(xr)
    _, sw = O.quantize_rows(wr)
    sx, sw = sx.astype(np.float64)[:, None], sw.astype(np.float64)[None, :]
    half = 0.5 + 1e-4
    bound = (np.abs(xr).sum(1)[:, None] * sw * half + np.abs(wr).sum(1)[None, :] * sx * half + K * sx * sw * half ** 2)
    err = np.abs(y - exact)
    assert (err <= bound).all()
    assert err.max() > 0 and err.max() < 0.05 * np.abs(exact).max()


def test_w8a8_block_zero_adaln_is_identity_and_close_to_fp64():
    """In the W8A8 format too, zero AdaLN weights give zero gates and out == x
    exactly; with the drawn weights the block stays near the float64 block
    (a synthetic numerics gate: the pages gate on image quality from trained
    weights, which random weights cannot give)."""
    cfg = I.C1_W8A8
    w = I.block_weights(cfg)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    wz = dict(w, w_ada=np.zeros_like(w["w_ada"]), b_ada=np.zeros_like(w["b_ada"]))
    np.testing.assert_array_equal(O.block_forward(x, c, wz, cfg, pos), np.asarray(x, np.float64))
    q8 = O.block_forward(x, c, w, cfg, pos) - x
    ref = O.block_forward(x, c, w, I.C1, pos) - x
    rel_rms = np.sqrt(((q8 - ref) ** 2).mean() / (ref ** 2).mean())
    assert 1e-4 < rel_rms < 3e-2, rel_rms
    # prepared weights (codes and scales made once) give the same block
    wp = dict(w, **{k + "_q8": O.quantize_h256(w[k]) for k in ("w_qkv", "w_o", "w_gate_up", "w_down")})
    np.testing.assert_array_equal(O.block_forward(x, c, wp, cfg, pos) - x, q8)

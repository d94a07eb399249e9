"""CPU oracle for one pre-norm AdaLN DiT block and the flow-match Euler loop.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
routes through it.  It imports nothing from the HIP package and shares no
code with it: every step below is the plain definition, written with NumPy,
computed in float64 by default (``dtype=np.float32`` gives the fp32 variant),
with the full attention matrix materialised and no blocking or fusion.

Sources (the three pages the method comes from):
  [ERNIE]   "Porting ERNIE-Image-Turbo to Zig and Metal: An 8B Diffusion
            Transformer From Scratch on Apple Silicon" (engineering.oakoliver.com)
  [ZML]     "From Python + CUDA to Pure Rust + Metal 4: How zml-flow-rs Stops
            Us Writing a Kernel Per Model" (engineering.oakoliver.com)
  [MAKEPAD] makepad commit log, libs/ai/metal/shaders/ggml (gitdab.com)

Readings taken where the pages are silent or disagree (each also pinned by a
test): LayerNorm (no affine in AdaLN mode) for the pre-modulation norm;
qk-LayerNorm over head_dim applied before RoPE; eps = 1e-6; modulation input
is SiLU(c) with a bias; identity gate; SwiGLU feed-forward with the gate rows
first; 3D RoPE with contiguous per-axis chunks and interleaved pairs,
rotate-half pairs for the ViT; timestep embedding [cos | sin] with
omega_j = exp(-ln(1e4) j / (dim/2)); sigma grid s_i = 1 - i/n shifted by
shift*s/(1+(shift-1)s); final layer chunks (scale, shift) with no SiLU.

`spec` arguments are any object with the attributes: batch, seq, heads,
kv_heads, head_dim, cond_dim, qk_norm, rope ("interleaved3d" | "half2d"),
rope_axes, rope_theta, eps, and optionally the semantics switches the pages
disagree on (defaults in brackets): norm ["layernorm"] | "rmsnorm"; act
["silu"] | "gelu_tanh"; gate ["identity"] | "tanh" | "sigmoid"; mod
["shift_scale_gate"] | "scale_gate"; qk_order ["norm_rope"] | "rope_norm";
fmt ["bf16"] | "f32" | "w8a8_h256" (the four block projections in int8 with a
256-point Hadamard rotation on both operands, per-row scales; "bf16" and
"f32" differ only in the weight values the caller passes, the arithmetic here
is the same float64 x W^T).

Parity status: every function here is pinned by a closed form, an invariant,
a special case or a brute-force loop in tests/test_oracle.py, except the
semantic choices listed above against the real trained model, which no file
available here can decide ("parity unpinned" for that question only).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------
def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).

    [ERNIE] §IV: the modulation input is the SiLU-modulated time embedding;
    the SwiGLU gate of the feed-forward uses the same function."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def layer_norm(x, eps, gamma=None, beta=None):
    """LayerNorm over the last axis: (x - mean) / sqrt(biased var + eps), then
    the optional affine gamma/beta ([MAKEPAD] pre-norm ViT block uses it)."""
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    y = xc / np.sqrt(var + eps)
    if gamma is not None:
        y = y * gamma
    if beta is not None:
        y = y + beta
    return y


def rms_norm(x, eps, gamma=None):
    """RMSNorm: x / sqrt(mean(x^2) + eps) ([ERNIE] §IV names this norm kind)."""
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * gamma


def gelu_tanh(z):
    """GELU in its tanh approximation, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))),
    with the tanh argument clamped to [-20, 20] and the result to the fp16
    range +-65504 ([ERNIE] §V Bug 1: the FFN activation, and the clamps that
    keep a large gate projection from producing inf - inf)."""
    with np.errstate(over="ignore", invalid="ignore"):      # z^3 may overflow; the clamp absorbs it
        a = np.sqrt(2.0 / np.pi) * (z + 0.044715 * z * z * z)
        return np.clip(0.5 * z * (1.0 + np.tanh(np.clip(a, -20.0, 20.0))), -65504.0, 65504.0)


def gate_fn(g, kind="identity"):
    """The function applied to a modulation gate before the gated residual:
    identity ([ERNIE] §VII Decision 1 prints r + g y), tanh or sigmoid (the
    alternatives [ZML] §IV's semantics search chooses between)."""
    if kind == "identity":
        return g
    if kind == "tanh":
        return np.tanh(g)
    if kind == "sigmoid":
        return 1.0 / (1.0 + np.exp(-g))
    raise ValueError(kind)


def norm(x, spec, gamma=None, beta=None):
    """The block's norm kind: LayerNorm, or RMSNorm ([ERNIE] §IV draws RMSNorm
    for the AdaLN norm and the qk-norm), then the optional affine."""
    if getattr(spec, "norm", "layernorm") == "rmsnorm":
        y = rms_norm(x, spec.eps)
        if gamma is not None:
            y = y * gamma
        return y if beta is None else y + beta
    return layer_norm(x, spec.eps, gamma, beta)


def modulate(n, shift, scale):
    """AdaLN modulation n * (1 + scale) + shift ([ERNIE] §V Bug 4 prints the
    form; [ZML] §IV calls the `1 + scale` variant plus_one)."""
    return n * (1.0 + scale) + shift


def linear(x, w, b=None, dtype=F64):
    """y = x W^T (+ b) for W stored [out, in]."""
    y = np.asarray(x, dtype) @ np.asarray(w, dtype).T
    return y if b is None else y + np.asarray(b, dtype)


def gated_residual(r, gate, y):
    """r + gate * y, with the residual kept in full precision ([ERNIE] §VII
    Decision 1 prints this gated residual)."""
    return r + gate * y


def swiglu(h, w_gate_up, dtype=F64, act="silu"):
    """act(h Wg^T) * (h Wu^T) with W = [Wg; Wu] stacked gate rows first
    ([ZML] §VI: Glu step with gate_first; SwiGLU names the SiLU gate; [ERNIE]
    §IV / §V Bug 1: GELU(gate) x up with the clamped tanh GELU)."""
    w = np.asarray(w_gate_up, dtype)
    F = w.shape[0] // 2
    f = silu if act == "silu" else gelu_tanh
    return f(linear(h, w[:F], dtype=dtype)) * linear(h, w[F:], dtype=dtype)


# ---------------------------------------------------------------------------
# W8A8 with a 256-point Hadamard rotation on both operands ([ZML] §VII
# "Precision Formats Derived, Not Picked": the I8 per-row format with H256 on
# both sides, legal by rotation invariance (x H)(W H)^T = x W^T for orthogonal H)
# ---------------------------------------------------------------------------
ROT_BLOCK = 256
QMAX = 127


def hadamard(n):
    """Normalised Sylvester-Hadamard matrix of order n (a power of two), built
    by doubling [[H, H], [H, -H]]; entry (a, b) is (-1)^popcount(a & b) / sqrt(n).
    Orthogonal and symmetric."""
    h = np.ones((1, 1), F64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def rotate_h256(x):
    """x [..., K] times blockdiag(H256, ..., H256) along the last axis (K a
    multiple of 256): every consecutive run of 256 inputs is rotated on its own
    (a reading: the page names H256 but not its placement along K)."""
    x = np.asarray(x, F64)
    K = x.shape[-1]
    assert K % ROT_BLOCK == 0, "reduction length must be a multiple of 256"
    blocks = x.reshape(x.shape[:-1] + (K // ROT_BLOCK, ROT_BLOCK))
    return (blocks @ hadamard(ROT_BLOCK)).reshape(x.shape)


def quantize_rows(v):
    """Symmetric per-row int8 codes ("I8 per-row"): amax = max |v| over the
    row, scale = amax / 127, code = v * (127 / amax) rounded half to even and
    clamped to [-127, 127]; a zero row has codes 0 and scale 0.

    The code is an integer decided by floating point, so it is decided in
    float32, the precision the device kernels use: v is rounded to float32,
    and 127 / amax, the product and amax / 127 are each rounded to float32.
    Returns (codes int8 [..., K], scale float32 [...])."""
    v32 = np.asarray(v, np.float32)
    amax = np.abs(v32).max(axis=-1, keepdims=True)
    safe = np.where(amax > 0, amax, np.float32(1))
    inv = np.where(amax > 0, np.float32(QMAX) / safe, np.float32(0)).astype(np.float32)
    q = np.clip(np.rint((v32 * inv).astype(np.float32)), -QMAX, QMAX).astype(np.int8)
    scale = (amax[..., 0] / np.float32(QMAX)).astype(np.float32)
    return q, scale


def quantize_h256(x):
    """Rotate then quantize per row: the form both the weights [out, in] (one
    scale per output channel, prepared once) and the activations [tokens, in]
    (one scale per token) take."""
    return quantize_rows(rotate_h256(x))


def w8a8_matmul(qx, sx, qw, sw):
    """y[m, n] = sx[m] sw[n] sum_k qx[m, k] qw[n, k]: the integer dot products
    are exact (a float64 matmul of the codes: every partial sum is an integer
    of magnitude <= K 127^2 < 2^53), then scaled in float64."""
    K = np.shape(qx)[-1]
    assert K * QMAX * QMAX < 2 ** 53
    acc = np.asarray(qx, F64) @ np.asarray(qw, F64).T
    return acc * np.asarray(sx, F64)[:, None] * np.asarray(sw, F64)[None, :]


def w8a8_linear(x, w):
    """y ~ x W^T in the W8A8 H256 format: both x [M, K] and W [N, K] rotated
    and quantized per row.  `w` is the weight matrix or its prepared
    (codes, scales) pair."""
    qw, sw = w if isinstance(w, tuple) else quantize_h256(w)
    qx, sx = quantize_h256(x)
    return w8a8_matmul(qx, sx, qw, sw)


def block_linear(x, w, name, spec, dtype=F64):
    """One of the block's four projections (w_qkv, w_o, w_gate_up, w_down) in
    the block's format: spec.fmt "bf16" (default; plain x W^T) or "w8a8_h256".
    In the W8A8 format `w` may hold the prepared pair under name + "_q8"."""
    if getattr(spec, "fmt", "bf16") == "w8a8_h256":
        return np.asarray(w8a8_linear(x, w.get(name + "_q8") or w[name]), dtype)
    return linear(x, w[name], dtype=dtype)


def glu(gu, act="silu"):
    """act(gate) * up for gu = [gate | up] along the last axis (gate first)."""
    F = gu.shape[-1] // 2
    f = silu if act == "silu" else gelu_tanh
    return f(gu[..., :F]) * gu[..., F:]


# ---------------------------------------------------------------------------
# conditioning
# ---------------------------------------------------------------------------
def adaln_modulation(w_ada, b_ada, c, dtype=F64, mod="shift_scale_gate"):
    """AdaLN modulation m = W_ada . SiLU(c) + b_ada, returned as (shift1,
    scale1, gate1, shift2, scale2, gate2): six [D] chunks in that order
    ([ERNIE] §IV, last paragraph of the per-layer graph), or for mod =
    "scale_gate" four chunks (scale1, gate1, scale2, gate2) with no shift
    ([ZML] §IV table: modulation "[scale, gate], 1 + scale, no shift"; the
    order of the four chunks is a reading: [scale, gate] per branch)."""
    w = np.asarray(w_ada, dtype)
    m = w @ silu(np.asarray(c, dtype)) + np.asarray(b_ada, dtype)
    if mod == "scale_gate":
        scale1, gate1, scale2, gate2 = np.split(m, 4)
        z = np.zeros_like(scale1)
        return z, scale1, gate1, z, scale2, gate2
    return tuple(np.split(m, 6))


def timestep_embedding(t, dim, dtype=F64):
    """Sinusoidal timestep features with flip_sin_to_cos: [cos(t w) | sin(t w)],
    w_j = exp(-ln(10000) j / (dim/2)), j < dim/2 ([ZML] §IV table row
    "timestep sinusoid: flip_sin_to_cos")."""
    half = dim // 2
    j = np.arange(half, dtype=dtype)
    w = np.exp(-np.log(dtype(10000.0)) * j / dtype(half))
    a = dtype(t) * w
    return np.concatenate([np.cos(a), np.sin(a)]).astype(dtype)


# ---------------------------------------------------------------------------
# rotary position embedding
# ---------------------------------------------------------------------------
def rope_angles(pos, spec, dtype=F64):
    """Rotation angle of every (token, pair) slot, [S, head_dim/2].

    The head dim is cut into contiguous per-axis chunks of widths rope_axes
    ([ERNIE] §I: axes [32,48,48], theta=256).  Within the chunk of axis a (width
    d_a) pair j rotates by p_a * theta^(-2j/d_a).  interleaved3d uses the three
    (t, h, w) coordinates; half2d (the ViT, [MAKEPAD]) uses (h, w)."""
    pos = np.asarray(pos)
    cols = [0, 1, 2] if spec.rope == "interleaved3d" else [1, 2]
    assert len(cols) == len(spec.rope_axes) and sum(spec.rope_axes) == spec.head_dim
    out = []
    for col, da in zip(cols, spec.rope_axes):
        j = np.arange(da // 2, dtype=dtype)
        w = dtype(spec.rope_theta) ** (-2.0 * j / dtype(da))
        out.append(pos[:, col].astype(dtype)[:, None] * w[None, :])
    return np.concatenate(out, axis=1)


def apply_rope(x, ang, layout):
    """Rotate pairs (a, b) -> (a cos - b sin, a sin + b cos).

    x: [S, heads, hd]; ang: [S, hd/2].  "interleaved3d" pairs (2m, 2m+1)
    (interleaved layout, [ZML] §IV table); "half2d" pairs (m, m + hd/2)
    (rotate-half from tables, [MAKEPAD])."""
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    y = np.empty_like(x)
    if layout == "interleaved3d":
        a, b = x[..., 0::2], x[..., 1::2]
        y[..., 0::2] = a * c - b * s
        y[..., 1::2] = a * s + b * c
    else:
        h = x.shape[-1] // 2
        a, b = x[..., :h], x[..., h:]
        y[..., :h] = a * c - b * s
        y[..., h:] = a * s + b * c
    return y


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def softmax_rows(s):
    """Row softmax with the row maximum subtracted first."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(q, k, v, heads, kv_heads, q_rows=None):
    """Mask-free scaled dot-product attention of one sequence ([ERNIE] §VII
    Decision 2: text truncated so attention needs no mask).

    q: [S, H, hd], k/v: [S, Hkv, hd].  Query head h reads KV head
    h // (H / Hkv) (grouped heads, [ZML] §VI attention(heads, kv_heads, ...)).
    Scores are q k^T / sqrt(hd); the full [S, S] matrix is materialised.
    q_rows restricts the queries (sampled outputs); returns [len(q_rows), H*hd]."""
    S, H, hd = q.shape
    group = heads // kv_heads
    if q_rows is None:
        q_rows = np.arange(S)
    out = np.empty((len(q_rows), H, hd), dtype=q.dtype)
    inv = 1.0 / np.sqrt(q.dtype.type(hd))
    for h in range(H):
        g = h // group
        s = (q[q_rows, h, :] @ k[:, g, :].T) * inv
        out[:, h, :] = softmax_rows(s) @ v[:, g, :]
    return out.reshape(len(q_rows), H * hd)


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------
def _mods(w, c, spec, dtype):
    """(shift1, scale1, gate1, shift2, scale2, gate2); the gates already
    passed through the gate function."""
    D = w["w_qkv"].shape[1]
    if spec.cond_dim > 0:
        sh1, sc1, g1, sh2, sc2, g2 = adaln_modulation(w["w_ada"], w["b_ada"], c, dtype,
                                                      getattr(spec, "mod", "shift_scale_gate"))
        kind = getattr(spec, "gate", "identity")
        return sh1, sc1, gate_fn(g1, kind), sh2, sc2, gate_fn(g2, kind)
    z, one = np.zeros(D, dtype), np.ones(D, dtype)
    return z, z, one, z, z, one


def _prenorm(x, w, which, shift, scale, spec, dtype):
    if spec.cond_dim > 0:
        return modulate(norm(x, spec), shift, scale)
    g, b = w[which + "_g"], w[which + "_b"]
    return norm(x, spec, None if g is None else np.asarray(g, dtype), None if b is None else np.asarray(b, dtype))


def block_qkv(h, w, spec, pos, dtype=F64):
    """QKV projection, per-head qk-norm and RoPE on q and k.

    [ZML] §I/§VI fuse "QKV + norm + RoPE" with the norm first (the default,
    qk_order "norm_rope"); [ERNIE] §IV's per-layer graph draws 3D RoPE before
    qk_layernorm (qk_order "rope_norm").  Returns q [N,H,hd], k/v [N,Hkv,hd]."""
    H, Hk, hd = spec.heads, spec.kv_heads, spec.head_dim
    N = h.shape[0]
    qkv = block_linear(h, w, "w_qkv", spec, dtype)
    q = qkv[:, : H * hd].reshape(N, H, hd)
    k = qkv[:, H * hd: (H + Hk) * hd].reshape(N, Hk, hd)
    v = qkv[:, (H + Hk) * hd:].reshape(N, Hk, hd)
    ang = rope_angles(pos, spec, dtype)                       # [S, hd/2]
    ang = np.tile(ang, (spec.batch, 1))                       # every sequence uses the same positions

    def qknorm(q, k):
        if not spec.qk_norm:
            return q, k
        return (norm(q, spec, np.asarray(w["q_g"], dtype), np.asarray(w["q_b"], dtype)),
                norm(k, spec, np.asarray(w["k_g"], dtype), np.asarray(w["k_b"], dtype)))

    if getattr(spec, "qk_order", "norm_rope") == "rope_norm":
        q, k = qknorm(apply_rope(q, ang, spec.rope), apply_rope(k, ang, spec.rope))
    else:
        q, k = qknorm(q, k)
        q, k = apply_rope(q, ang, spec.rope), apply_rope(k, ang, spec.rope)
    return q, k, v


def block_forward(x, c, w, spec, pos, dtype=F64, rows=None, keep=None):
    """out = block(x, c) for x [B*S, D] ([ERNIE] §IV per-layer graph, with the
    SwiGLU feed-forward the workload names):

      m = W_ada SiLU(c) + b_ada  -> shift1, scale1, gate1, shift2, scale2, gate2
      h   = LN(x)(1 + scale1) + shift1
      q,k,v = qk-LN + RoPE of h W_qkv^T
      x1  = x + gate1 * (Attn(q,k,v) W_o^T)          (gated residual, [ERNIE] §VII Decision 1)
      h2  = LN(x1)(1 + scale2) + shift2
      out = x1 + gate2 * ((SiLU(h2 Wg^T) * (h2 Wu^T)) W_down^T)

    Without AdaLN (cond_dim 0, the ViT) LN is affine and the gates are 1.
    `rows` computes only those output rows (all keys are still projected).
    `keep` (a dict) receives the intermediates when given."""
    x = np.asarray(x, dtype)
    shift1, scale1, gate1, shift2, scale2, gate2 = _mods(w, c, spec, dtype)
    N, D = x.shape
    B, S = spec.batch, spec.seq
    h = _prenorm(x, w, "ln1", shift1, scale1, spec, dtype)
    q, k, v = block_qkv(h, w, spec, pos, dtype)
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    att = np.empty((len(rows), spec.heads * spec.head_dim), dtype)
    for b in range(B):
        sel = np.nonzero(rows // S == b)[0]
        if len(sel) == 0:
            continue
        sl = slice(b * S, (b + 1) * S)
        att[sel] = attention(q[sl], k[sl], v[sl], spec.heads, spec.kv_heads, rows[sel] - b * S)
    x1 = gated_residual(x[rows], gate1, block_linear(att, w, "w_o", spec, dtype))
    h2 = _prenorm(x1, w, "ln2", shift2, scale2, spec, dtype)
    ff = glu(block_linear(h2, w, "w_gate_up", spec, dtype), getattr(spec, "act", "silu"))
    out = gated_residual(x1, gate2, block_linear(ff, w, "w_down", spec, dtype))
    if keep is not None:
        keep.update(dict(mods=(shift1, scale1, gate1, shift2, scale2, gate2), h=h, q=q, k=k, v=v,
                         att=att, x1=x1, h2=h2, ff=ff, out=out))
    return out


# ---------------------------------------------------------------------------
# the denoising loop
# ---------------------------------------------------------------------------
def flowmatch_sigmas(steps, shift, dtype=F64):
    """Sigma grid of the flow-match Euler scheduler: s_i = 1 - i/steps for
    i = 0..steps (the last one 0), then shift*s / (1 + (shift-1) s)
    ([ERNIE] §I: FlowMatchEulerDiscreteScheduler, shift 4.0, 8 steps; an
    exponential time shift with mu = ln(shift) and exponent 1 is the same map)."""
    s = 1.0 - np.arange(steps + 1, dtype=dtype) / dtype(steps)
    return shift * s / (1.0 + (shift - 1.0) * s)


def euler_update(latent, v, sigma, sigma_next):
    """One Euler step of the flow ODE: latent + (sigma_next - sigma) v
    ([ZML] §IV table "Euler sign +1"; §V "euler = primitive")."""
    return latent + (sigma_next - sigma) * v


def final_layer(x, c, edges, spec, dtype=F64):
    """Final AdaLN-continuous norm and projection to the latent channels:
    [scale | shift] = W_f c + b_f (scale first, [ERNIE] §V Bug 4),
    v = (LN(x)(1 + scale) + shift) W_out^T + b_out."""
    m = np.asarray(edges["w_fmod"], dtype) @ np.asarray(c, dtype) + np.asarray(edges["b_fmod"], dtype)
    scale, shift = np.split(m, 2)
    h = modulate(norm(x, spec), shift, scale)
    return h @ np.asarray(edges["w_out"], dtype).T + np.asarray(edges["b_out"], dtype)


def stack_step(latent, sigma, blocks, edges, spec, pos, dtype=F64, layers=None):
    """Velocity v for one denoising step of the block stack.

    c = temb(1000 sigma); x = latent W_in^T + b_in; x = block_l(x, c) for every
    layer ([ERNIE] §IV: 36 layers per step); v = final_layer(x, c).
    `blocks` is a sequence (or a callable l -> weights) of per-block weights."""
    L = spec.layers if layers is None else layers
    c = timestep_embedding(1000.0 * sigma, spec.cond_dim, dtype)
    x = np.asarray(latent, dtype) @ np.asarray(edges["w_in"], dtype).T + np.asarray(edges["b_in"], dtype)
    for l in range(L):
        w = blocks(l) if callable(blocks) else blocks[l]
        x = block_forward(x, c, w, spec, pos, dtype)
    return final_layer(x, c, edges, spec, dtype)


def denoise(latent, blocks, edges, spec, pos, steps, shift, dtype=F64, layers=None, start=0):
    """The flow-match Euler loop from step `start` to the end ([ERNIE] §IV:
    8 Euler steps around the DiT)."""
    sig = flowmatch_sigmas(steps, shift, dtype)
    lat = np.asarray(latent, dtype)
    for i in range(start, steps):
        v = stack_step(lat, sig[i], blocks, edges, spec, pos, dtype, layers)
        lat = euler_update(lat, v, sig[i], sig[i + 1])
    return lat

"""Seeded synthetic inputs for the DiT block / flow-match loop.

This module only draws random numbers and lays out shapes; it holds none of
the method's arithmetic (no norms, rotations, attention, schedules).  Both the
HIP path's tests/bench and the CPU oracle consume what it produces, so neither
side can hide a mistake by generating its own data.

Workload shapes follow the pages' models:
  * ERNIE-Image-Turbo (Zig+Metal port page, §I "What Shipped" and §IV
    "Architecture Overview"): 36 layers, hidden 4096, 32 heads x 128,
    FFN 12288, 3D RoPE axes [32,48,48], theta 256, qk-norm, 64x64 latent
    grid of 4096 tokens with 128 latent channels, 8 Euler steps, shift 4.0.
  * Krea-2-Turbo (zml-flow-rs page, §III): a 6144-wide GQA DiT, SwiGLU 16384.
  * the resident pre-norm ViT backbone (makepad commit log): LayerNorm,
    rotate-half RoPE from precomputed tables, SwiGLU, residuals in place.
Weights and biases are N(0, 0.02) rounded to bf16 (round-to-nearest-even;
kept fp32 in the fp32 format), activations N(0, 1); every tensor has its own PCG64 stream keyed by
(config id, block index, tensor id) under one root seed.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

ROOT_SEED = 20261202

# Stable tensor ids for the spawn keys (never reorder: they fix the data).
TENSOR_IDS = {
    "w_ada": 1, "b_ada": 2, "w_qkv": 3, "w_o": 4, "w_gate_up": 5, "w_down": 6,
    "q_g": 7, "q_b": 8, "k_g": 9, "k_b": 10, "ln1_g": 11, "ln1_b": 12,
    "ln2_g": 13, "ln2_b": 14, "x": 20, "cond": 21, "latent": 22,
    "w_in": 30, "b_in": 31, "w_fmod": 32, "b_fmod": 33, "w_out": 34, "b_out": 35,
}


@dataclasses.dataclass(frozen=True)
class DiTConfig:
    """Shape and semantic switches of one DiT block (and of a stack of them)."""
    name: str
    cfg_id: int
    batch: int
    grid: Tuple[int, int, int]      # (frames, rows, cols) of the latent grid; seq = product
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    ffn: int
    cond_dim: int                    # 0: no AdaLN (affine LayerNorm, gate 1)
    qk_norm: bool
    rope: str                        # "interleaved3d" or "half2d"
    rope_axes: Tuple[int, ...]       # per-axis rotary widths, sum == head_dim
    rope_theta: float
    eps: float = 1e-6
    x_dtype: str = "bf16"            # dtype of x / out at the block boundary
    layers: int = 1
    latent_dim: int = 0              # stack only: latent channels (patch-embed input)
    seq_override: int = 0            # ragged sequence: use the first `seq` grid positions
    text_len: int = 0                # joint sequence: text tokens packed with the spatial ones
    text_first: bool = False         # joint order: text rows before the spatial rows
    # semantics switches the pages disagree on (defaults = the readings of the main path)
    norm: str = "layernorm"          # "layernorm" | "rmsnorm" (block norms and qk-norm)
    act: str = "silu"                # FFN GLU activation: "silu" | "gelu_tanh" (clamped)
    gate: str = "identity"           # gate function: "identity" | "tanh" | "sigmoid"
    mod: str = "shift_scale_gate"    # AdaLN chunks: "shift_scale_gate" (6D) | "scale_gate" (4D, no shift)
    qk_order: str = "norm_rope"      # "norm_rope" | "rope_norm"
    # format of the four block projections: "bf16", "w8a8_h256" (int8 codes
    # of both operands after a 256-point Hadamard rotation, one scale per row),
    # or "f32" (the fp32 run: every weight fp32, not rounded to bf16, and x fp32)
    fmt: str = "bf16"

    @property
    def spatial(self) -> int:
        if self.seq_override:
            return self.seq_override
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def seq(self) -> int:
        return self.spatial + self.text_len

    @property
    def ada_rows(self) -> int:
        """Rows of the AdaLN linear: 6 or 4 chunks of hidden."""
        return (4 if self.mod == "scale_gate" else 6) * self.hidden

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def qkv_dim(self) -> int:
        return (self.heads + 2 * self.kv_heads) * self.head_dim

    @property
    def bf16_weights(self) -> bool:
        return self.fmt != "f32"

    def replace(self, **kw) -> "DiTConfig":
        return dataclasses.replace(self, **kw)


# configs in the order the workload list gives them
C1 = DiTConfig("tiny_block", 1, 1, (1, 16, 16), 256, 4, 4, 64, 768, 256, True,
               "interleaved3d", (16, 24, 24), 256.0, x_dtype="bf16")
C2 = DiTConfig("vit_backbone", 2, 4, (1, 32, 32), 1024, 16, 16, 64, 4096, 0, False,
               "half2d", (32, 32), 100.0, x_dtype="f32", layers=24)
C3 = DiTConfig("block_8b", 3, 1, (1, 64, 64), 4096, 32, 32, 128, 12288, 4096, True,
               "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16")
C4 = C3.replace(name="stack_8b", cfg_id=4, x_dtype="f32", layers=36, latent_dim=128)
C5_4096 = DiTConfig("gqa_wide_4096", 5, 1, (1, 64, 64), 6144, 48, 8, 128, 16384, 6144, True,
                    "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16", layers=28)
C5_1024 = C5_4096.replace(name="gqa_wide_1024", grid=(1, 32, 32))
# joint text + image sequences (ERNIE page, "Token Layout"): 4096 spatial + 74
# text tokens = 4170, spatial rows first; the text-first order is the variant
# the zml-flow-rs page (§IV semantics table) found for another model
C3_JOINT = C3.replace(name="block_8b_joint", cfg_id=6, text_len=74)
C1_JOINT = C1.replace(name="tiny_joint", cfg_id=7, text_len=7)
C1_JOINT_TF = C1_JOINT.replace(name="tiny_joint_text_first", text_first=True)

# the W8A8 H256 format of the zml-flow-rs page (§VII) on the same shapes (same data)
C1_W8A8 = C1.replace(name="tiny_block_w8a8", fmt="w8a8_h256")
C3_W8A8 = C3.replace(name="block_8b_w8a8", fmt="w8a8_h256")
C4_W8A8 = C4.replace(name="stack_8b_w8a8", fmt="w8a8_h256")
# the fp32 run of the tiny block (same seeds; weights not rounded to bf16)
C1_F32 = C1.replace(name="tiny_block_f32", fmt="f32", x_dtype="f32")

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5_4096, C5_1024, C3_JOINT, C1_JOINT, C1_JOINT_TF,
                               C1_W8A8, C3_W8A8, C4_W8A8, C1_F32)}

STACK_STEPS = 8
STACK_SHIFT = 4.0


def _rng(cfg_id: int, block: int, tensor: str) -> np.random.Generator:
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=(cfg_id, block, TENSOR_IDS[tensor]))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Values of `a` rounded to the nearest bf16, returned as fp32."""
    return bf16_to_f32(bf16_bits(a))


def _normal(cfg_id, block, tensor, shape, std, bf16=True):
    a = _rng(cfg_id, block, tensor).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return bf16_round(a) if bf16 else a


def positions(cfg: DiTConfig) -> np.ndarray:
    """Integer (t, h, w) position of every token of one sequence, [S, 3].

    Spatial token i of a frames x rows x cols grid sits at
    (i // (rows*cols), (i // cols) % rows, i % cols); the latent grid is
    walked row-major (ERNIE page, §VII Decision 3, spatial positions).
    In a joint sequence (text_len > 0) the spatial tokens' t is offset by
    text_len and text token j sits at (j, 0, 0) (ERNIE page, "Token Layout"
    and §VII Decision 3); the spatial rows come first unless text_first.
    """
    f, hh, ww = cfg.grid
    i = np.arange(f * hh * ww, dtype=np.int64)
    pos = np.stack([i // (hh * ww), (i // ww) % hh, i % ww], axis=1)[: cfg.spatial]
    if cfg.text_len == 0:
        return pos.copy()
    pos = pos.copy()
    pos[:, 0] += cfg.text_len
    text = np.zeros((cfg.text_len, 3), np.int64)
    text[:, 0] = np.arange(cfg.text_len)
    return np.concatenate([text, pos] if cfg.text_first else [pos, text], axis=0)


def block_weights(cfg: DiTConfig, block: int = 0, affine_random: bool = False,
                  zero_ada: bool = False, draw_ada: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """One block's parameters as fp32 arrays holding bf16-representable values.

    GEMM weights are [out, in] row-major. w_gate_up stacks the gate rows first,
    then the up rows. Norm gammas/betas are fp32 (1 and 0 unless
    `affine_random`, which draws 1+0.1N and 0.1N to exercise the affine path).
    """
    D, F, Dc = cfg.hidden, cfg.ffn, cfg.cond_dim
    hd, cid = cfg.head_dim, cfg.cfg_id
    w: Dict[str, Optional[np.ndarray]] = {}
    if Dc > 0:
        if draw_ada:
            w["w_ada"] = _normal(cid, block, "w_ada", (cfg.ada_rows, Dc), 0.02, cfg.bf16_weights)
            w["b_ada"] = _normal(cid, block, "b_ada", (cfg.ada_rows,), 0.02, cfg.bf16_weights)
        else:
            w["w_ada"] = w["b_ada"] = None
        if zero_ada and draw_ada:
            w["w_ada"][:] = 0
            w["b_ada"][:] = 0
        w["ln1_g"] = w["ln1_b"] = w["ln2_g"] = w["ln2_b"] = None
    else:
        w["w_ada"] = w["b_ada"] = None
        for n in ("ln1", "ln2"):
            if affine_random:
                w[n + "_g"] = (1 + 0.1 * _rng(cid, block, n + "_g").standard_normal(D)).astype(np.float32)
                w[n + "_b"] = (0.1 * _rng(cid, block, n + "_b").standard_normal(D)).astype(np.float32)
            else:
                w[n + "_g"] = np.ones(D, np.float32)
                w[n + "_b"] = np.zeros(D, np.float32)
    bw = cfg.bf16_weights
    w["w_qkv"] = _normal(cid, block, "w_qkv", (cfg.qkv_dim, D), 0.02, bw)
    w["w_o"] = _normal(cid, block, "w_o", (D, cfg.heads * hd), 0.02, bw)
    w["w_gate_up"] = _normal(cid, block, "w_gate_up", (2 * F, D), 0.02, bw)
    w["w_down"] = _normal(cid, block, "w_down", (D, F), 0.02, bw)
    if cfg.qk_norm:
        if affine_random:
            for n in ("q", "k"):
                w[n + "_g"] = (1 + 0.1 * _rng(cid, block, n + "_g").standard_normal(hd)).astype(np.float32)
                w[n + "_b"] = (0.1 * _rng(cid, block, n + "_b").standard_normal(hd)).astype(np.float32)
        else:
            w["q_g"] = w["k_g"] = np.ones(hd, np.float32)
            w["q_b"] = w["k_b"] = np.zeros(hd, np.float32)
    else:
        w["q_g"] = w["q_b"] = w["k_g"] = w["k_b"] = None
    return w


def block_x(cfg: DiTConfig, block: int = 0) -> np.ndarray:
    """Block input x [B*S, D] ~ N(0,1); bf16-rounded when x is a bf16 tensor."""
    a = _rng(cfg.cfg_id, block, "x").standard_normal(size=(cfg.tokens, cfg.hidden), dtype=np.float32)
    return bf16_round(a) if cfg.x_dtype == "bf16" else a


def cond(cfg: DiTConfig) -> Optional[np.ndarray]:
    """Conditioning vector c [Dc] ~ N(0,1) (fp32), or None without AdaLN."""
    if cfg.cond_dim == 0:
        return None
    return _rng(cfg.cfg_id, 0, "cond").standard_normal(size=(cfg.cond_dim,), dtype=np.float32)


def stack_edges(cfg: DiTConfig) -> Dict[str, np.ndarray]:
    """Patch-embed, final modulation and output projection of the stack."""
    D, C, Dc, cid, bw = cfg.hidden, cfg.latent_dim, cfg.cond_dim, cfg.cfg_id, cfg.bf16_weights
    return {
        "w_in": _normal(cid, 1000, "w_in", (D, C), 0.02, bw),
        "b_in": _normal(cid, 1000, "b_in", (D,), 0.02, bw),
        "w_fmod": _normal(cid, 1000, "w_fmod", (2 * D, Dc), 0.02, bw),   # rows: scale then shift
        "b_fmod": _normal(cid, 1000, "b_fmod", (2 * D,), 0.02, bw),
        "w_out": _normal(cid, 1000, "w_out", (C, D), 0.02, bw),
        "b_out": _normal(cid, 1000, "b_out", (C,), 0.02, bw),
    }


def latent(cfg: DiTConfig) -> np.ndarray:
    """Initial latent noise [B*S, C] ~ N(0,1), fp32."""
    return _rng(cfg.cfg_id, 0, "latent").standard_normal(size=(cfg.tokens, cfg.latent_dim), dtype=np.float32)


def stack_block_weights(cfg: DiTConfig, block: int, shared_ada: Dict[str, np.ndarray]):
    """Block `block` of a stack: its own GEMM weights, the stack's one shared AdaLN linear."""
    w = block_weights(cfg, block, draw_ada=False)
    w["w_ada"], w["b_ada"] = shared_ada["w_ada"], shared_ada["b_ada"]
    return w


def shared_ada(cfg: DiTConfig) -> Dict[str, np.ndarray]:
    D, Dc, cid = cfg.hidden, cfg.cond_dim, cfg.cfg_id
    return {"w_ada": _normal(cid, 999, "w_ada", (cfg.ada_rows, Dc), 0.02, cfg.bf16_weights),
            "b_ada": _normal(cid, 999, "b_ada", (cfg.ada_rows,), 0.02, cfg.bf16_weights)}


# ---------------------------------------------------------------------------
# Device-side generation for the full-size timing workload (16 GB of weights
# would take minutes to draw with NumPy).  Seeded torch generator on the
# device; values are N(0, 0.02) rounded to bf16 like the host generator.
# ---------------------------------------------------------------------------
def torch_normal_bf16(shape, std, seed, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(torch.bfloat16)


def torch_seed(cfg_id: int, block: int, tensor: str) -> int:
    return (ROOT_SEED * 1000003 + cfg_id * 10007 + block * 101 + TENSOR_IDS[tensor]) & 0x7FFFFFFFFFFF

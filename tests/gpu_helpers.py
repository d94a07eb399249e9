"""Shared helpers of the GPU parity tests (metrics, uploads, configs)."""
import sys

import numpy as np

from diffusion_transformer_dit_amd import inputs as I

# The parity bar on block outputs (bf16 path): max relative error
# max|g - o| / max|o| <= 2e-2 and cosine similarity >= 0.9995.
MAX_REL = 2e-2
MIN_COS = 0.9995


def metrics(got, ref):
    g = np.asarray(got, np.float64).ravel()
    o = np.asarray(ref, np.float64).ravel()
    d = g - o
    return {
        "max_rel": float(np.abs(d).max() / max(np.abs(o).max(), 1e-300)),
        "cos": float(g @ o / max(np.linalg.norm(g) * np.linalg.norm(o), 1e-300)),
        "rel_rms": float(np.linalg.norm(d) / max(np.linalg.norm(o), 1e-300)),
    }


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_parity(got, ref, max_rel=MAX_REL, min_cos=MIN_COS, what=""):
    m = metrics(got, ref)
    say(f"  parity {what}: max_rel={m['max_rel']:.3e} cos={m['cos']:.8f} rel_rms={m['rel_rms']:.3e}")
    assert np.isfinite(np.asarray(got)).all(), f"{what}: non-finite output"
    assert m["max_rel"] <= max_rel, (what, m)
    assert m["cos"] >= min_cos, (what, m)
    return m


# small block shapes for GPU parity: several tiles and ragged tails
SMALL = {
    "c1_tiny": I.C1,
    "c1_ragged200": I.C1.replace(name="c1_ragged200", seq_override=200),
    "hd128_ragged400": I.DiTConfig("hd128_ragged400", 11, 1, (1, 20, 20), 512, 4, 4, 128, 1024, 256, True,
                                   "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16"),
    "gqa3_b2_ragged300": I.DiTConfig("gqa3_b2_ragged300", 12, 2, (1, 15, 20), 768, 6, 2, 128, 1536, 512, True,
                                     "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16"),
    "vit_b2_f32": I.DiTConfig("vit_b2_f32", 13, 2, (1, 16, 16), 512, 8, 8, 64, 1024, 0, False,
                              "half2d", (32, 32), 100.0, x_dtype="f32"),
    "c1_f32x_t3": I.C1.replace(name="c1_f32x_t3", cfg_id=14, x_dtype="f32", grid=(3, 8, 12)),
    # joint text + image sequences: 256 spatial + 7 text tokens, both orders
    "tiny_joint": I.C1_JOINT,
    "tiny_joint_text_first": I.C1_JOINT_TF,
    # semantics switches, one at a time and in combination
    "c1_rms": I.C1.replace(name="c1_rms", cfg_id=15, norm="rmsnorm"),
    "c1_gelu": I.C1.replace(name="c1_gelu", cfg_id=16, act="gelu_tanh"),
    "c1_gate_tanh": I.C1.replace(name="c1_gate_tanh", cfg_id=17, gate="tanh"),
    "c1_gate_sigmoid": I.C1.replace(name="c1_gate_sigmoid", cfg_id=18, gate="sigmoid"),
    "c1_scale_gate": I.C1.replace(name="c1_scale_gate", cfg_id=19, mod="scale_gate"),
    "c1_rope_first": I.C1.replace(name="c1_rope_first", cfg_id=21, qk_order="rope_norm"),
    "hd128_ernie_diagram": I.DiTConfig("hd128_ernie_diagram", 22, 1, (1, 20, 20), 512, 4, 4, 128, 1024, 256, True,
                                       "interleaved3d", (32, 48, 48), 256.0, x_dtype="f32", norm="rmsnorm",
                                       act="gelu_tanh", qk_order="rope_norm"),
    "half_hd128_rope_first": I.DiTConfig("half_hd128_rope_first", 23, 2, (1, 12, 16), 512, 4, 2, 128, 1024, 256, True,
                                         "half2d", (64, 64), 100.0, x_dtype="bf16", qk_order="rope_norm"),
    "qwen_like": I.C1.replace(name="qwen_like", cfg_id=24, gate="tanh", mod="scale_gate", x_dtype="f32"),
}


# QKV projection shapes shared by the bf16 and W8A8 stage tests: a 74-row tail
# of 128-row tiles after full 256-row tiles, and the split-form cases.
# 4170 tokens (30 x 139 grid), 16 + 2 x 8 heads of 128: 16 full row tiles x 16 column
# tiles fill one round of 256 CUs, so the 74-row tail runs as a 128-row tile launch
QKV_TAIL = I.DiTConfig("qkv_tail_4170", 25, 1, (1, 30, 139), 2048, 16, 8, 128, 4096, 256, True,
                       "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16")


# bf16 shapes whose 256 x 256 tile count fills a round: with 128-wide heads and a
# sequence length that is a multiple of 16 the projection takes the split form
# (plain-epilogue 4-wave GEMM, then the in-place qk-norm + RoPE pass).  Two
# sequences of 1008 tokens, GQA 32 / 16 heads, a ragged last row tile; 1904
# tokens, GQA 32 / 8, rotate-half RoPE before an RMS qk-norm.  The last keeps
# the fused epilogue (64-wide heads, 1899 tokens) at a similar size.
QKV_SPLIT = {
    "qkv_split_b2_1008": I.DiTConfig("qkv_split_b2_1008", 26, 2, (1, 28, 36), 4096, 32, 16, 128, 256, 256, True,
                                     "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16"),
    "qkv_split_half_1904": I.DiTConfig("qkv_split_half_1904", 41, 1, (1, 28, 68), 4096, 32, 8, 128, 256, 256, True,
                                       "half2d", (64, 64), 100.0, x_dtype="bf16", norm="rmsnorm",
                                       qk_order="rope_norm"),
    # one sequence of 4170 tokens (not a multiple of 16): the 4096 rows of full
    # 256-row tiles split, the 74-row tail in the fused 128-row launch
    "qkv_split_joint_4170": I.DiTConfig("qkv_split_joint_4170", 42, 1, (1, 30, 139), 4096, 32, 32, 128, 256, 256, True,
                                        "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16"),
    # 34 q heads and 2 k heads: the qk-norm pass's last group of 8 heads holds
    # both q and k rows
    "qkv_split_mixed_group_3072": I.DiTConfig("qkv_split_mixed_group_3072", 43, 1, (1, 48, 64), 4352, 34, 2, 128, 256,
                                              256, True, "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16"),
    # no qk-norm: the pass applies RoPE only
    "qkv_split_no_qknorm_b2_1008": I.DiTConfig("qkv_split_no_qknorm_b2_1008", 44, 2, (1, 28, 36), 4096, 32, 16, 128,
                                               256, 256, False, "interleaved3d", (32, 48, 48), 256.0, x_dtype="bf16"),
    "qkv_fused_hd64_1899": I.DiTConfig("qkv_fused_hd64_1899", 27, 1, (1, 9, 211), 4096, 64, 32, 64, 256, 256, True,
                                       "half2d", (32, 32), 100.0, x_dtype="bf16", norm="rmsnorm",
                                       qk_order="rope_norm"),
}

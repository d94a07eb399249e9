"""C-ABI checks that need no GPU: the library loads, exports every function
include/dit.h declares, validates arguments before touching a device, and its
host helpers agree with the oracle."""
import ctypes as C
import os
import re
from fractions import Fraction

import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from oracle import dit as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit.h")

pytestmark = pytest.mark.skipif(not os.path.exists(N.LIB_PATH), reason="libdit.so not built")

FAKE = 1 << 20          # a 16-byte aligned address that is never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 18
    L = N.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(N.EXPORTED)
    assert N.dit_version().startswith("dit-gfx950")


def test_status_strings():
    for st in range(0, -7, -1):
        assert N.dit_status_string(st) != "unknown status"
    assert N.dit_status_string(5) == "unknown status"


def _desc(**kw):
    cfg = I.C1
    d = dict(batch=1, seq=256, hidden=256, heads=4, kv_heads=4, head_dim=64, ffn=768, cond_dim=256)
    d.update(kw)
    return N.make_desc(**d)


def test_desc_accepts_every_semantics_switch():
    for kw in (dict(norm=N.DIT_RMSNORM), dict(act=N.DIT_ACT_GELU_TANH), dict(gate=N.DIT_GATE_TANH),
               dict(gate=N.DIT_GATE_SIGMOID), dict(mod=N.DIT_MOD_SCALE_GATE), dict(qk_order=N.DIT_QK_ROPE_NORM)):
        assert N.dit_block_workspace_size(_desc(**kw)) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=320, heads=5, kv_heads=5), N.DIT_ERR_UNSUPPORTED),   # hidden % 256
    (dict(heads=3), N.DIT_ERR_INVALID_ARG),                   # heads*hd != hidden
    (dict(kv_heads=3), N.DIT_ERR_INVALID_ARG),                # heads % kv_heads
    (dict(head_dim=32, heads=8), N.DIT_ERR_UNSUPPORTED),      # head_dim not built
    (dict(ffn=100), N.DIT_ERR_UNSUPPORTED),
    (dict(seq=0), N.DIT_ERR_INVALID_ARG),
    (dict(cond_dim=12), N.DIT_ERR_UNSUPPORTED),
    (dict(eps=0.0), N.DIT_ERR_INVALID_ARG),
    (dict(norm=2), N.DIT_ERR_INVALID_ARG),
    (dict(act=2), N.DIT_ERR_INVALID_ARG),
    (dict(gate=3), N.DIT_ERR_INVALID_ARG),
    (dict(gate=-1), N.DIT_ERR_INVALID_ARG),
    (dict(mod=2), N.DIT_ERR_INVALID_ARG),
    (dict(qk_order=2), N.DIT_ERR_INVALID_ARG),
    (dict(w_dtype=N.DIT_F32), N.DIT_ERR_UNSUPPORTED),                      # fp32 weights need x fp32
    (dict(w_dtype=N.DIT_F32, x_dtype=N.DIT_F32, fmt=N.DIT_FMT_W8A8_H256), N.DIT_ERR_UNSUPPORTED),
    (dict(w_dtype=2), N.DIT_ERR_INVALID_ARG),
    (dict(fmt=2), N.DIT_ERR_INVALID_ARG),
    (dict(fmt=N.DIT_FMT_W8A8_H256, ffn=640), N.DIT_ERR_UNSUPPORTED),     # W8A8: ffn % 256
    (dict(fmt=N.DIT_FMT_W8A8_H256, ffn=9216), N.DIT_ERR_UNSUPPORTED),    # no rotation kernel for 9 rounds
])
def test_desc_validation(kw, status):
    with pytest.raises(N.DitError) as e:
        N.dit_block_workspace_size(_desc(**kw))
    assert e.value.status == status
    assert N.dit_last_error()


def test_workspace_size_accounts_for_buffers():
    d = _desc()
    n = N.dit_block_workspace_size(d)
    N_, D, F = 256, 256, 768
    # h, q, k, vt, att bf16 + x1 fp32 + u bf16 + modulation
    assert n >= N_ * D * 2 * 5 + N_ * D * 4 + N_ * F * 2 + 6 * D * 4
    assert N.dit_seq_pad(200) == 256 and N.dit_seq_pad(256) == 256 and N.dit_seq_pad(257) == 320


def _weights(**over):
    names = dict(w_ada=FAKE, b_ada=FAKE, w_qkv=FAKE, q_g=FAKE, q_b=FAKE, k_g=FAKE, k_b=FAKE, w_o=FAKE,
                 w_gate_up=FAKE, w_down=FAKE)
    names.update(over)
    return N.make_weights(names)


def test_block_forward_validation_before_device():
    d = _desc()
    ws_need = N.dit_block_workspace_size(d)
    ws = 1 << 40
    good = dict(x=FAKE, cond=FAKE, rope_cos=FAKE, rope_sin=FAKE, out=FAKE, ws=ws)

    def call(w=None, ws_bytes=ws_need, **kw):
        a = dict(good)
        a.update(kw)
        N.dit_block_forward(d, w or _weights(), a["x"], a["cond"], a["rope_cos"], a["rope_sin"], a["out"], a["ws"],
                            stream=0, ws_bytes=ws_bytes)

    cases = [
        (dict(w=_weights(w_qkv=None)), N.DIT_ERR_INVALID_ARG),
        (dict(w=_weights(w_o=FAKE + 8)), N.DIT_ERR_ALIGNMENT),
        (dict(w=_weights(w_ada=None)), N.DIT_ERR_INVALID_ARG),
        (dict(w=_weights(q_g=None)), N.DIT_ERR_INVALID_ARG),
        (dict(w=_weights(ln1_g=FAKE)), N.DIT_ERR_UNSUPPORTED),
        (dict(cond=None), N.DIT_ERR_INVALID_ARG),
        (dict(x=FAKE + 4), N.DIT_ERR_ALIGNMENT),
        (dict(ws_bytes=ws_need - 1), N.DIT_ERR_WORKSPACE),
        (dict(out=FAKE + 256), N.DIT_ERR_INVALID_ARG),       # partial overlap with x
        (dict(ws=FAKE), N.DIT_ERR_INVALID_ARG),              # workspace overlaps x
    ]
    for kw, st in cases:
        with pytest.raises(N.DitError) as e:
            call(**kw)
        assert e.value.status == st, (kw, e.value)


@pytest.mark.skipif(os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK), reason="a GPU may be present")
def test_valid_calls_report_no_device():
    d = _desc()
    ws_need = N.dit_block_workspace_size(d)
    with pytest.raises(N.DitError) as e:
        N.dit_block_forward(d, _weights(), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, stream=0, ws_bytes=ws_need)
    assert e.value.status == N.DIT_ERR_NO_DEVICE
    with pytest.raises(N.DitError) as e:
        N.euler_flowmatch_update(FAKE, FAKE + 4096, 16, 1.0, 0.5, stream=0)
    assert e.value.status == N.DIT_ERR_NO_DEVICE
    with pytest.raises(N.DitError) as e:
        N.dit_timestep_embedding(3.0, 16, FAKE, stream=0)
    assert e.value.status == N.DIT_ERR_NO_DEVICE


def test_stage_entry_validation():
    with pytest.raises(N.DitError) as e:
        N.dit_gemm_gated_residual(FAKE, FAKE, 100, 100, 64, None, 0, None, None, FAKE + (1 << 24), 0, stream=0)
    assert e.value.status == N.DIT_ERR_UNSUPPORTED
    with pytest.raises(N.DitError) as e:
        N.dit_gemm_swiglu(FAKE, FAKE, 100, 128, 60, FAKE, stream=0)
    assert e.value.status == N.DIT_ERR_UNSUPPORTED
    with pytest.raises(N.DitError) as e:
        N.dit_ln_modulate(FAKE, 0, 10, 300, FAKE, FAKE, 0, 1e-6, FAKE + (1 << 24), stream=0)
    assert e.value.status == N.DIT_ERR_UNSUPPORTED
    with pytest.raises(N.DitError) as e:
        N.dit_ln_modulate(FAKE, 0, 10, 256, FAKE, None, 0, 1e-6, FAKE + (1 << 24), stream=0)   # mode 0 needs scale
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.dit_ln_modulate(FAKE, 0, 10, 256, FAKE, FAKE, 0, 1e-6, FAKE + (1 << 24), stream=0, norm=7)
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.dit_gemm_gated_residual(FAKE, FAKE, 256, 256, 64, None, 0, FAKE, None, FAKE + (1 << 24), 0, stream=0,
                                  gate_fn=3)
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.dit_gemm_swiglu(FAKE, FAKE, 256, 128, 64, FAKE + (1 << 24), stream=0, act=2)
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.euler_flowmatch_update(FAKE, FAKE + 8, 64, 1.0, 0.5, stream=0)
    assert e.value.status in (N.DIT_ERR_ALIGNMENT, N.DIT_ERR_INVALID_ARG)


def test_stack_validation():
    d = _desc(x_dtype=N.DIT_BF16)
    e = dict(w_in=FAKE, b_in=FAKE, w_fmod=FAKE, b_fmod=FAKE, w_out=FAKE, b_out=FAKE)
    m = N.make_model(d, [_weights()] * 2, 128, e)
    with pytest.raises(N.DitError) as err:
        N.dit_stack_workspace_size(m)
    assert err.value.status == N.DIT_ERR_UNSUPPORTED           # stack needs an fp32 residual stream
    m = N.make_model(_desc(x_dtype=N.DIT_F32), [_weights()] * 2, 100, e)
    with pytest.raises(N.DitError) as err:
        N.dit_stack_workspace_size(m)
    assert err.value.status == N.DIT_ERR_UNSUPPORTED           # latent_dim % 128
    m = N.make_model(_desc(x_dtype=N.DIT_F32), [_weights()] * 2, 128, e)
    assert N.dit_stack_workspace_size(m) > N.dit_block_workspace_size(_desc(x_dtype=N.DIT_F32))


def test_loop_validation_before_device():
    """dit_loop_*: every argument is checked before any HIP call."""
    e = dict(w_in=FAKE, b_in=FAKE, w_fmod=FAKE, b_fmod=FAKE, w_out=FAKE, b_out=FAKE)
    m = N.make_model(_desc(x_dtype=N.DIT_F32), [_weights()] * 2, 128, e)
    need = N.dit_loop_workspace_size(m)
    assert need > N.dit_stack_workspace_size(m)
    big = 1 << 40
    cases = [
        (dict(steps=0), N.DIT_ERR_INVALID_ARG),
        (dict(steps=1001), N.DIT_ERR_INVALID_ARG),
        (dict(shift=0.0), N.DIT_ERR_INVALID_ARG),
        (dict(shift=float("nan")), N.DIT_ERR_INVALID_ARG),
        (dict(latent=None), N.DIT_ERR_INVALID_ARG),
        (dict(latent=FAKE + 4), N.DIT_ERR_ALIGNMENT),
        (dict(ws_bytes=need - 1), N.DIT_ERR_WORKSPACE),
        (dict(latent=big + 4096), N.DIT_ERR_INVALID_ARG),      # latent inside the workspace
    ]
    for kw, st in cases:
        args = dict(latent=FAKE, steps=8, shift=4.0, ws_bytes=need)
        args.update(kw)
        with pytest.raises(N.DitError) as err:
            N.dit_loop_create(m, args["latent"], FAKE, FAKE, args["steps"], args["shift"], big, ws_bytes=args["ws_bytes"])
        assert err.value.status == st, (kw, err.value)
    with pytest.raises(N.DitError) as err:
        N.dit_loop_launch_step(None, 0, stream=0)
    assert err.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as err:
        N.dit_loop_launch(None, stream=0)
    assert err.value.status == N.DIT_ERR_INVALID_ARG
    N.dit_loop_destroy(None)                                      # NULL is accepted
    if not (os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK)):
        with pytest.raises(N.DitError) as err:
            N.dit_loop_create(m, FAKE, FAKE, FAKE, 8, 4.0, big, ws_bytes=need)
        assert err.value.status == N.DIT_ERR_NO_DEVICE


# ---------------------------------------------------------------------------
# host helpers against the oracle
# ---------------------------------------------------------------------------
def test_sigmas_match_oracle_and_golden():
    got = N.dit_flowmatch_sigmas(8, 4.0)
    ref = O.flowmatch_sigmas(8, 4.0)
    np.testing.assert_allclose(got, ref, rtol=1e-7, atol=1e-8)
    assert got[0] == 1.0 and got[-1] == 0.0


@pytest.mark.parametrize("cfg", [I.C1, I.C2, I.C3], ids=lambda c: c.name)
def test_rope_tables_match_oracle(cfg):
    pos = I.positions(cfg) + np.array([2, 0, 0])    # nonzero t so the t-axis slots rotate
    rope = N.DIT_ROPE_INTERLEAVED if cfg.rope == "interleaved3d" else N.DIT_ROPE_HALF
    cos, sin = N.dit_rope_tables(pos, rope, cfg.rope_axes, cfg.rope_theta, cfg.head_dim)
    ang = O.rope_angles(pos, cfg)
    np.testing.assert_allclose(cos, np.cos(ang), atol=2e-7)
    np.testing.assert_allclose(sin, np.sin(ang), atol=2e-7)
    # position 0 is the identity rotation, exactly
    c0, s0 = N.dit_rope_tables(np.zeros((3, 3), np.int32), rope, cfg.rope_axes, cfg.rope_theta, cfg.head_dim)
    assert (c0 == 1).all() and (s0 == 0).all()


def test_rope_tables_validation():
    with pytest.raises(N.DitError):
        N.dit_rope_tables(np.zeros((4, 3)), N.DIT_ROPE_INTERLEAVED, (16, 24, 20), 256.0, 64)   # widths sum != hd
    with pytest.raises(N.DitError):
        N.dit_rope_tables(np.zeros((4, 3)), N.DIT_ROPE_HALF, (16, 24, 24), 256.0, 64)          # half takes 2 axes


def test_w8a8_workspace_and_weight_scales():
    """The W8A8 format adds int8 copies of the attention and GLU outputs and
    three row-scale vectors to the block workspace, and needs the weights'
    row scales."""
    d8 = _desc(fmt=N.DIT_FMT_W8A8_H256)
    N_, D, F = 256, 256, 768
    assert N.dit_block_workspace_size(d8) >= N.dit_block_workspace_size(_desc()) + N_ * (D + F) + 3 * N_ * 4
    ws_need = N.dit_block_workspace_size(d8)
    scales = dict(s_qkv=FAKE, s_o=FAKE, s_gate_up=FAKE, s_down=FAKE)
    for over, st in ((dict(scales, s_o=None), N.DIT_ERR_INVALID_ARG), (dict(scales, s_down=FAKE + 4), N.DIT_ERR_ALIGNMENT)):
        with pytest.raises(N.DitError) as e:
            N.dit_block_forward(d8, _weights(**over), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, stream=0, ws_bytes=ws_need)
        assert e.value.status == st, (over, e.value)


def test_w8a8_stage_entry_validation():
    big = FAKE + (1 << 24)

    def expect(st, f, *a, **kw):
        with pytest.raises(N.DitError) as e:
            f(*a, stream=0, **kw)
        assert e.value.status == st, (f.__name__, a, e.value)

    expect(N.DIT_ERR_UNSUPPORTED, N.dit_quantize_h256, FAKE, N.DIT_BF16, 10, 300, big, big + (1 << 20))   # cols % 256
    expect(N.DIT_ERR_UNSUPPORTED, N.dit_quantize_h256, FAKE, N.DIT_BF16, 10, 9216, big, big + (1 << 20))
    expect(N.DIT_ERR_INVALID_ARG, N.dit_quantize_h256, FAKE, 7, 10, 4096, big, big + (1 << 20))
    expect(N.DIT_ERR_INVALID_ARG, N.dit_quantize_h256, FAKE, N.DIT_BF16, 10, 4096, FAKE + 1024, big)      # x overlaps q
    expect(N.DIT_ERR_ALIGNMENT, N.dit_quantize_h256, FAKE, N.DIT_BF16, 10, 4096, big + 8, big + (1 << 20))
    expect(N.DIT_ERR_UNSUPPORTED, N.dit_ln_modulate_h256q, FAKE, 0, 10, 8448, FAKE, FAKE, 0, 1e-6, big, big + 4096)
    expect(N.DIT_ERR_INVALID_ARG, N.dit_ln_modulate_h256q, FAKE, 0, 10, 256, FAKE, None, 0, 1e-6, big, big + 4096)
    expect(N.DIT_ERR_UNSUPPORTED, N.dit_gemm_w8a8_gated_residual, FAKE, FAKE, FAKE, FAKE, 256, 256, 192, None, 0,
           None, None, big, 0)                                                                             # K % 128
    expect(N.DIT_ERR_UNSUPPORTED, N.dit_gemm_w8a8_gated_residual, FAKE, FAKE, FAKE, FAKE, 256, 100, 256, None, 0,
           None, None, big, 0)
    expect(N.DIT_ERR_INVALID_ARG, N.dit_gemm_w8a8_gated_residual, FAKE, None, FAKE, FAKE, 256, 256, 256, None, 0,
           None, None, big, 0)                                                                             # a_scale
    expect(N.DIT_ERR_ALIGNMENT, N.dit_gemm_w8a8_swiglu, FAKE, FAKE + 4, FAKE, FAKE, 256, 128, 256, big)
    expect(N.DIT_ERR_INVALID_ARG, N.dit_gemm_w8a8_swiglu, FAKE, FAKE, FAKE, FAKE, 256, 128, 256, big, act=5)
    expect(N.DIT_ERR_INVALID_ARG, N.dit_qkv_rope_w8a8, _desc(fmt=N.DIT_FMT_W8A8_H256), FAKE, None, FAKE, FAKE, FAKE,
           FAKE, FAKE, FAKE, FAKE, FAKE, big, big, big)


@pytest.mark.skipif(os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK), reason="a GPU may be present")
def test_w8a8_valid_calls_report_no_device():
    big = FAKE + (1 << 24)
    for f, a in ((N.dit_quantize_h256, (FAKE, N.DIT_BF16, 10, 4096, big, big + (1 << 20))),
                 (N.dit_quantize_h256, (FAKE, N.DIT_F32, 10, 12288, big, big + (1 << 20))),
                 (N.dit_ln_modulate_h256q, (FAKE, 0, 10, 6144, FAKE, FAKE, 0, 1e-6, big, big + (1 << 20))),
                 (N.dit_gemm_w8a8_swiglu, (FAKE, FAKE, FAKE, FAKE, 256, 128, 256, big))):
        with pytest.raises(N.DitError) as e:
            f(*a, stream=0)
        assert e.value.status == N.DIT_ERR_NO_DEVICE, f.__name__


def test_attention_split_validation():
    d = _desc(seq=300)
    assert N.dit_attention_workspace_size(d, 1) == 0
    n8 = N.dit_attention_workspace_size(d, 8)
    assert n8 == 1 * 4 * 8 * 256 * (64 * 4 + 8)          # partial O fp32 + (max, sum) per chunk slot
    for nsplit, ws, nb, st in ((0, FAKE, n8, N.DIT_ERR_INVALID_ARG), (65, FAKE, n8, N.DIT_ERR_INVALID_ARG),
                               (8, None, 0, N.DIT_ERR_INVALID_ARG), (8, FAKE, n8 - 1, N.DIT_ERR_WORKSPACE),
                               (8, FAKE + 8, n8, N.DIT_ERR_ALIGNMENT)):
        with pytest.raises(N.DitError) as e:
            N.dit_flash_attention_split(d, FAKE, FAKE, FAKE, FAKE + (1 << 24), nsplit, ws, stream=0, ws_bytes=nb)
        assert e.value.status == st, (nsplit, e.value)
    # a ragged sequence grows the block workspace by the partials of up to 16 chunks
    assert N.dit_block_workspace_size(_desc(seq=300)) > N.dit_block_workspace_size(_desc(seq=256))


def test_f32_path_desc_and_workspace():
    """fp32 weights select the fp32 path: fp32 intermediates, no split-KV partials."""
    d16 = _desc(x_dtype=N.DIT_F32)
    d32 = _desc(x_dtype=N.DIT_F32, w_dtype=N.DIT_F32)
    n16, n32 = N.dit_block_workspace_size(d16), N.dit_block_workspace_size(d32)
    N_, D, F = 256, 256, 768
    # h, q, k, vt, att, x1 fp32 + u fp32 + modulation
    assert n32 >= N_ * D * 4 * 6 + N_ * F * 4 + 6 * D * 4
    assert n32 > n16
    # a ragged fp32 sequence needs no split partials
    r32 = N.dit_block_workspace_size(_desc(x_dtype=N.DIT_F32, w_dtype=N.DIT_F32, seq=300))
    assert r32 - n32 < 300 * 4 * (5 * D + F) - 256 * 4 * (5 * D + F) + 64 * D * 4 + 8 * 256
    with pytest.raises(N.DitError) as e:
        N.dit_flash_attention_split(d32, FAKE, FAKE, FAKE, FAKE + (1 << 24), 4, FAKE, stream=0, ws_bytes=1 << 30)
    assert e.value.status == N.DIT_ERR_UNSUPPORTED


def test_f32_operands_bounded_by_bytes():
    """Buffer resources address 32-bit byte counts: fp32 operands are held
    below 2^30 elements (4 GiB), bf16 ones below 2^31."""
    # 65536 tokens x hidden 4096 x ffn 16384: u is 2^30 elements
    big = dict(seq=65536, hidden=4096, heads=32, kv_heads=32, head_dim=128, ffn=16384, cond_dim=256)
    with pytest.raises(N.DitError) as e:
        N.dit_block_workspace_size(_desc(x_dtype=N.DIT_F32, w_dtype=N.DIT_F32, **big))
    assert e.value.status == N.DIT_ERR_UNSUPPORTED
    assert N.dit_block_workspace_size(_desc(**big)) > 0                        # 2^31 bytes of bf16: fine
    # one below the limit is accepted, fp32 too
    ok = dict(big, seq=65535)
    assert N.dit_block_workspace_size(_desc(x_dtype=N.DIT_F32, w_dtype=N.DIT_F32, **ok)) > 0
    with pytest.raises(N.DitError) as e:        # bf16 at 2^31 elements
        N.dit_block_workspace_size(_desc(**dict(big, seq=131072)))
    assert e.value.status == N.DIT_ERR_UNSUPPORTED


def test_sigma_embedding_validation():
    with pytest.raises(N.DitError) as e:
        N.dit_sigma_embedding(float("nan"), 256, FAKE)
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.dit_sigma_embedding(0.5, 255, FAKE)
    assert e.value.status == N.DIT_ERR_INVALID_ARG


def test_noalloc_block_validation_before_device():
    """The allocation-free block entry point validates like dit_block_forward
    and rejects a block whose workspace exceeds its scratch before any device
    work."""
    assert N.dit_block_forward_noalloc_max_bytes() == 128 << 20
    far = FAKE + (1 << 40)
    big = _desc(seq=4096, hidden=4096, heads=32, kv_heads=32, head_dim=128, ffn=12288, cond_dim=4096)
    assert N.dit_block_workspace_size(big) > N.dit_block_forward_noalloc_max_bytes()
    with pytest.raises(N.DitError) as e:
        N.dit_block_forward_noalloc(big, _weights(), FAKE, FAKE, FAKE, FAKE, far)
    assert e.value.status == N.DIT_ERR_WORKSPACE
    d = _desc()
    for kw, st in [(dict(w=_weights(w_qkv=None)), N.DIT_ERR_INVALID_ARG), (dict(x=FAKE + 4), N.DIT_ERR_ALIGNMENT),
                   (dict(cond=None), N.DIT_ERR_INVALID_ARG), (dict(out=FAKE + 256), N.DIT_ERR_INVALID_ARG)]:
        a = dict(w=_weights(), x=FAKE, cond=FAKE, out=far)
        a.update(kw)
        with pytest.raises(N.DitError) as e:
            N.dit_block_forward_noalloc(d, a["w"], a["x"], a["cond"], FAKE, FAKE, a["out"])
        assert e.value.status == st, (kw, e.value)


def test_block_chain_validation_before_device():
    d = _desc()
    need = N.dit_block_chain_workspace_size(d)
    assert need > N.dit_block_workspace_size(d)            # plus a second modulation buffer
    w = [_weights(), _weights(w_ada=FAKE + (1 << 22))]
    far = 1 << 40
    with pytest.raises(N.DitError) as e:
        N.dit_block_chain_forward(d, [], FAKE, FAKE, FAKE, FAKE, far, stream=0, ws_bytes=need)
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.dit_block_chain_forward(d, w, FAKE, FAKE, FAKE, FAKE, far, stream=0, ws_bytes=need - 1)
    assert e.value.status == N.DIT_ERR_WORKSPACE
    with pytest.raises(N.DitError) as e:
        N.dit_block_chain_forward(d, [w[0], _weights(w_o=None)], FAKE, FAKE, FAKE, FAKE, far, stream=0, ws_bytes=need)
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.dit_block_chain_forward(d, w, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0, ws_bytes=need)   # ws overlaps x
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    if not (os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK)):
        with pytest.raises(N.DitError) as e:
            N.dit_block_chain_forward(d, w, FAKE, FAKE, FAKE, FAKE, far, stream=0, side_stream=8, ws_bytes=need)
        assert e.value.status == N.DIT_ERR_NO_DEVICE


def test_trace_validation():
    with pytest.raises(N.DitError) as e:
        N.dit_trace_end("/tmp/never.json")            # not tracing
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    with pytest.raises(N.DitError) as e:
        N.dit_trace_begin(0)
    assert e.value.status == N.DIT_ERR_INVALID_ARG
    if not (os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK)):
        with pytest.raises(N.DitError) as e:
            N.dit_trace_begin(16)
        assert e.value.status == N.DIT_ERR_NO_DEVICE

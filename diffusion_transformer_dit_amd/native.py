"""ctypes binding of libdit.so: the C ABI of include/dit.h with the same names.

Argument marshalling only -- every step of the computation runs in the HIP
kernels of libdit.so.  Device buffers may be passed as torch tensors (their
data_ptr() is used) or as raw integer addresses; `stream` defaults to torch's
current HIP stream.  A missing library raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Any, Dict, Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit.so")

DIT_OK, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED, DIT_ERR_WORKSPACE = 0, -1, -2, -3
DIT_ERR_ALIGNMENT, DIT_ERR_NO_DEVICE, DIT_ERR_HIP = -4, -5, -6
DIT_F32, DIT_BF16 = 0, 1
DIT_LAYERNORM, DIT_RMSNORM = 0, 1
DIT_ROPE_INTERLEAVED, DIT_ROPE_HALF = 0, 1
DIT_ACT_SILU, DIT_ACT_GELU_TANH = 0, 1
DIT_GATE_IDENTITY, DIT_GATE_TANH, DIT_GATE_SIGMOID = 0, 1, 2
DIT_MOD_SHIFT_SCALE_GATE, DIT_MOD_SCALE_GATE = 0, 1
DIT_QK_NORM_ROPE, DIT_QK_ROPE_NORM = 0, 1
DIT_FMT_BF16, DIT_FMT_W8A8_H256 = 0, 1

EXPORTED = (
    "dit_block_workspace_size", "dit_block_forward", "dit_stack_workspace_size", "dit_stack_step",
    "euler_flowmatch_update", "dit_timestep_embedding", "dit_flowmatch_sigmas", "dit_rope_tables",
    "dit_adaln_modulation", "dit_ln_modulate", "dit_qkv_rope", "dit_seq_pad", "dit_flash_attention",
    "dit_gemm_gated_residual", "dit_gemm_swiglu", "dit_status_string", "dit_last_error", "dit_version",
    "dit_loop_workspace_size", "dit_loop_create", "dit_loop_launch_step", "dit_loop_launch", "dit_loop_destroy",
    "dit_quantize_h256", "dit_ln_modulate_h256q", "dit_gemm_w8a8_gated_residual", "dit_gemm_w8a8_swiglu",
    "dit_qkv_rope_w8a8", "dit_attention_workspace_size", "dit_flash_attention_split", "dit_sigma_embedding",
    "dit_block_forward_noalloc", "dit_block_forward_noalloc_max_bytes", "dit_block_chain_workspace_size",
    "dit_block_chain_forward", "dit_trace_begin", "dit_trace_end",
)


class DitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class dit_block_desc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("batch", "seq", "hidden", "heads", "kv_heads", "head_dim", "ffn",
                                         "cond_dim", "qk_norm", "norm", "rope")] + \
               [("eps", C.c_float), ("x_dtype", C.c_int32), ("w_dtype", C.c_int32)] + \
               [(n, C.c_int32) for n in ("act", "gate", "mod", "qk_order", "fmt")]


WEIGHT_FIELDS = ("w_ada", "b_ada", "ln1_g", "ln1_b", "ln2_g", "ln2_b", "w_qkv", "q_g", "q_b", "k_g", "k_b",
                 "w_o", "w_gate_up", "w_down", "s_qkv", "s_o", "s_gate_up", "s_down")


class dit_block_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS]


class dit_model(C.Structure):
    _fields_ = [("blk", dit_block_desc), ("layers", C.c_int32), ("latent_dim", C.c_int32),
                ("blocks", C.POINTER(dit_block_weights)),
                ("w_in", C.c_void_p), ("b_in", C.c_void_p), ("w_fmod", C.c_void_p), ("b_fmod", C.c_void_p),
                ("w_out", C.c_void_p), ("b_out", C.c_void_p)]


_lib = None


def lib():
    """Load libdit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m diffusion_transformer_dit_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
        pd, pw, pm = C.POINTER(dit_block_desc), C.POINTER(dit_block_weights), C.POINTER(dit_model)
        sig = {
            "dit_block_workspace_size": (C.c_int, [pd, C.POINTER(sz)]),
            "dit_block_forward": (C.c_int, [pd, pw, vp, vp, vp, vp, vp, vp, sz, vp]),
            "dit_block_forward_noalloc": (C.c_int, [pd, pw, vp, vp, vp, vp, vp, vp]),
            "dit_block_forward_noalloc_max_bytes": (sz, []),
            "dit_block_chain_workspace_size": (C.c_int, [pd, C.POINTER(sz)]),
            "dit_block_chain_forward": (C.c_int, [pd, pw, i32, vp, vp, vp, vp, vp, sz, vp, vp]),
            "dit_trace_begin": (C.c_int, [i32]),
            "dit_trace_end": (C.c_int, [C.c_char_p]),
            "dit_stack_workspace_size": (C.c_int, [pm, C.POINTER(sz)]),
            "dit_stack_step": (C.c_int, [pm, vp, vp, vp, vp, vp, vp, sz, vp]),
            "euler_flowmatch_update": (C.c_int, [vp, vp, i64, f32, f32, vp]),
            "dit_timestep_embedding": (C.c_int, [f32, i32, vp, vp]),
            "dit_sigma_embedding": (C.c_int, [f32, i32, vp, vp]),
            "dit_flowmatch_sigmas": (C.c_int, [i32, f32, vp]),
            "dit_rope_tables": (C.c_int, [vp, i32, i32, vp, i32, f32, i32, vp, vp]),
            "dit_adaln_modulation": (C.c_int, [vp, vp, vp, i32, i32, i32, vp, vp]),
            "dit_ln_modulate": (C.c_int, [vp, i32, i64, i32, i32, vp, vp, i32, f32, vp, vp]),
            "dit_qkv_rope": (C.c_int, [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "dit_seq_pad": (i32, [i32]),
            "dit_flash_attention": (C.c_int, [pd, vp, vp, vp, vp, vp]),
            "dit_gemm_gated_residual": (C.c_int, [vp, vp, i64, i32, i32, vp, i32, vp, i32, vp, vp, i32, vp]),
            "dit_gemm_swiglu": (C.c_int, [vp, vp, i64, i32, i32, i32, vp, vp]),
            "dit_status_string": (C.c_char_p, [C.c_int]),
            "dit_last_error": (C.c_char_p, []),
            "dit_version": (C.c_char_p, []),
            "dit_loop_workspace_size": (C.c_int, [pm, C.POINTER(sz)]),
            "dit_loop_create": (C.c_int, [pm, vp, vp, vp, i32, f32, vp, sz, C.POINTER(vp)]),
            "dit_loop_launch_step": (C.c_int, [vp, i32, vp]),
            "dit_loop_launch": (C.c_int, [vp, vp]),
            "dit_loop_destroy": (C.c_int, [vp]),
            "dit_quantize_h256": (C.c_int, [vp, i32, i64, i32, vp, vp, vp]),
            "dit_ln_modulate_h256q": (C.c_int, [vp, i32, i64, i32, i32, vp, vp, i32, f32, vp, vp, vp]),
            "dit_gemm_w8a8_gated_residual": (C.c_int, [vp, vp, vp, vp, i64, i32, i32, vp, i32, vp, i32, vp, vp,
                                                       i32, vp]),
            "dit_gemm_w8a8_swiglu": (C.c_int, [vp, vp, vp, vp, i64, i32, i32, i32, vp, vp]),
            "dit_qkv_rope_w8a8": (C.c_int, [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "dit_attention_workspace_size": (C.c_int, [pd, i32, C.POINTER(sz)]),
            "dit_flash_attention_split": (C.c_int, [pd, vp, vp, vp, vp, i32, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
        if os.environ.get("DIT_TRACE", "0") not in ("", "0"):
            # write the trace the library records under DIT_TRACE before the
            # HIP runtime is torn down (Python's exit handlers run first)
            import atexit
            atexit.register(lambda: L.dit_trace_end(None))
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _p(t: Any) -> Optional[int]:
    """Device/host address of a tensor, array or integer (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):          # numpy array (host helpers only)
        return t.ctypes.data
    raise TypeError(f"cannot take the address of {type(t)}")


def _nbytes(t: Any) -> int:
    if hasattr(t, "element_size"):
        return t.numel() * t.element_size()
    return int(t.nbytes)


def _stream(s: Any) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int):
    if rc != DIT_OK:
        raise DitError(rc, lib().dit_last_error().decode())


def make_desc(batch, seq, hidden, heads, kv_heads, head_dim, ffn, cond_dim, qk_norm=True, rope=DIT_ROPE_INTERLEAVED,
              eps=1e-6, x_dtype=DIT_BF16, norm=DIT_LAYERNORM, w_dtype=DIT_BF16, act=DIT_ACT_SILU,
              gate=DIT_GATE_IDENTITY, mod=DIT_MOD_SHIFT_SCALE_GATE, qk_order=DIT_QK_NORM_ROPE,
              fmt=DIT_FMT_BF16) -> dit_block_desc:
    return dit_block_desc(batch, seq, hidden, heads, kv_heads, head_dim, ffn, cond_dim, int(bool(qk_norm)), norm,
                          rope, eps, x_dtype, w_dtype, act, gate, mod, qk_order, fmt)


def make_weights(tensors: Dict[str, Any]) -> dit_block_weights:
    """dit_block_weights from a name -> tensor mapping (missing / None -> NULL).
    The caller keeps the tensors alive."""
    return dit_block_weights(*[_p(tensors.get(n)) for n in WEIGHT_FIELDS])


# ---------------------------------------------------------------------------
# the C entry points
# ---------------------------------------------------------------------------
def dit_block_workspace_size(desc: dit_block_desc) -> int:
    n = C.c_size_t(0)
    _check(lib().dit_block_workspace_size(C.byref(desc), C.byref(n)))
    return n.value


def dit_block_forward(desc, weights, x, cond, rope_cos, rope_sin, out, ws, stream=None, ws_bytes=None):
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().dit_block_forward(C.byref(desc), C.byref(weights), _p(x), _p(cond), _p(rope_cos), _p(rope_sin),
                                   _p(out), _p(ws), nb, _stream(stream)))


def dit_block_forward_noalloc(desc, weights, x, cond, rope_cos, rope_sin, out, stream=None):
    _check(lib().dit_block_forward_noalloc(C.byref(desc), C.byref(weights), _p(x), _p(cond), _p(rope_cos),
                                           _p(rope_sin), _p(out), _stream(stream)))


def dit_block_forward_noalloc_max_bytes() -> int:
    return int(lib().dit_block_forward_noalloc_max_bytes())


def dit_block_chain_workspace_size(desc: dit_block_desc) -> int:
    n = C.c_size_t(0)
    _check(lib().dit_block_chain_workspace_size(C.byref(desc), C.byref(n)))
    return n.value


def dit_block_chain_forward(desc, blocks: Sequence[dit_block_weights], x, cond, rope_cos, rope_sin, ws,
                            stream=None, side_stream=None, ws_bytes=None):
    arr = (dit_block_weights * len(blocks))(*blocks)
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().dit_block_chain_forward(C.byref(desc), arr, len(blocks), _p(x), _p(cond), _p(rope_cos),
                                         _p(rope_sin), _p(ws), nb, _stream(stream),
                                         None if side_stream is None else _stream(side_stream)))


def make_model(desc: dit_block_desc, blocks: Sequence[dit_block_weights], latent_dim: int, edges: Dict[str, Any]):
    arr = (dit_block_weights * len(blocks))(*blocks)
    m = dit_model(desc, len(blocks), latent_dim, C.cast(arr, C.POINTER(dit_block_weights)),
                  _p(edges["w_in"]), _p(edges["b_in"]), _p(edges["w_fmod"]), _p(edges["b_fmod"]),
                  _p(edges["w_out"]), _p(edges["b_out"]))
    m._keep = arr   # the block array must outlive the struct
    return m


def dit_stack_workspace_size(model: dit_model) -> int:
    n = C.c_size_t(0)
    _check(lib().dit_stack_workspace_size(C.byref(model), C.byref(n)))
    return n.value


def dit_stack_step(model, latent, cond, rope_cos, rope_sin, velocity, ws, stream=None, ws_bytes=None):
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().dit_stack_step(C.byref(model), _p(latent), _p(cond), _p(rope_cos), _p(rope_sin), _p(velocity),
                                _p(ws), nb, _stream(stream)))


def dit_loop_workspace_size(model: dit_model) -> int:
    n = C.c_size_t(0)
    _check(lib().dit_loop_workspace_size(C.byref(model), C.byref(n)))
    return n.value


def dit_loop_create(model, latent, rope_cos, rope_sin, steps, shift, ws, ws_bytes=None) -> int:
    """Returns the loop handle (an opaque address)."""
    h = C.c_void_p(None)
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib().dit_loop_create(C.byref(model), _p(latent), _p(rope_cos), _p(rope_sin), int(steps), float(shift),
                                 _p(ws), nb, C.byref(h)))
    return h.value


def dit_loop_launch_step(loop, step, stream=None):
    _check(lib().dit_loop_launch_step(loop, int(step), _stream(stream)))


def dit_loop_launch(loop, stream=None):
    _check(lib().dit_loop_launch(loop, _stream(stream)))


def dit_loop_destroy(loop):
    _check(lib().dit_loop_destroy(loop))


def euler_flowmatch_update(latent, velocity, n, sigma, sigma_next, stream=None):
    _check(lib().euler_flowmatch_update(_p(latent), _p(velocity), int(n), float(sigma), float(sigma_next),
                                        _stream(stream)))


def dit_timestep_embedding(t, dim, cond_out, stream=None):
    _check(lib().dit_timestep_embedding(float(t), int(dim), _p(cond_out), _stream(stream)))


def dit_sigma_embedding(sigma, dim, cond_out, stream=None):
    _check(lib().dit_sigma_embedding(float(sigma), int(dim), _p(cond_out), _stream(stream)))


def dit_flowmatch_sigmas(steps: int, shift: float):
    import numpy as np
    out = np.zeros(steps + 1, np.float32)
    _check(lib().dit_flowmatch_sigmas(int(steps), float(shift), _p(out)))
    return out


def dit_rope_tables(pos, rope: int, axes: Sequence[int], theta: float, head_dim: int):
    """Host cos/sin tables [seq, head_dim/2] (numpy fp32) for int positions pos [seq, 3]."""
    import numpy as np
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    ax = np.ascontiguousarray(axes, dtype=np.int32)
    seq = pos.shape[0]
    cos = np.zeros((seq, head_dim // 2), np.float32)
    sin = np.zeros((seq, head_dim // 2), np.float32)
    _check(lib().dit_rope_tables(_p(pos), seq, int(rope), _p(ax), len(ax), float(theta), int(head_dim), _p(cos),
                                 _p(sin)))
    return cos, sin


def dit_adaln_modulation(w, b, c, out_dim, in_dim, silu_input, m, stream=None):
    _check(lib().dit_adaln_modulation(_p(w), _p(b), _p(c), int(out_dim), int(in_dim), int(silu_input), _p(m),
                                      _stream(stream)))


def dit_ln_modulate(x, x_dtype, rows, dim, shift, scale, mode, eps, h, stream=None, norm=DIT_LAYERNORM):
    _check(lib().dit_ln_modulate(_p(x), int(x_dtype), int(rows), int(dim), int(norm), _p(shift), _p(scale), int(mode),
                                 float(eps), _p(h), _stream(stream)))


def dit_seq_pad(seq: int) -> int:
    return int(lib().dit_seq_pad(int(seq)))


def dit_qkv_rope(desc, h, w_qkv, q_g, q_b, k_g, k_b, rope_cos, rope_sin, q, k, vt, stream=None):
    _check(lib().dit_qkv_rope(C.byref(desc), _p(h), _p(w_qkv), _p(q_g), _p(q_b), _p(k_g), _p(k_b), _p(rope_cos),
                              _p(rope_sin), _p(q), _p(k), _p(vt), _stream(stream)))


def dit_flash_attention(desc, q, k, vt, out, stream=None):
    _check(lib().dit_flash_attention(C.byref(desc), _p(q), _p(k), _p(vt), _p(out), _stream(stream)))


def dit_attention_workspace_size(desc, nsplit) -> int:
    n = C.c_size_t(0)
    _check(lib().dit_attention_workspace_size(C.byref(desc), int(nsplit), C.byref(n)))
    return n.value


def dit_flash_attention_split(desc, q, k, vt, out, nsplit, ws, stream=None, ws_bytes=None):
    nb = (_nbytes(ws) if ws is not None else 0) if ws_bytes is None else ws_bytes
    _check(lib().dit_flash_attention_split(C.byref(desc), _p(q), _p(k), _p(vt), _p(out), int(nsplit), _p(ws), nb,
                                           _stream(stream)))


def dit_gemm_gated_residual(a, w, M, N, K, resid, resid_dtype, gate, bias, out, out_dtype, stream=None,
                            gate_fn=DIT_GATE_IDENTITY):
    _check(lib().dit_gemm_gated_residual(_p(a), _p(w), int(M), int(N), int(K), _p(resid), int(resid_dtype), _p(gate),
                                         int(gate_fn), _p(bias), _p(out), int(out_dtype), _stream(stream)))


def dit_gemm_swiglu(a, w_gate_up, M, F, K, u, stream=None, act=DIT_ACT_SILU):
    _check(lib().dit_gemm_swiglu(_p(a), _p(w_gate_up), int(M), int(F), int(K), int(act), _p(u), _stream(stream)))


def dit_quantize_h256(x, x_dtype, rows, cols, q, scale, stream=None):
    _check(lib().dit_quantize_h256(_p(x), int(x_dtype), int(rows), int(cols), _p(q), _p(scale), _stream(stream)))


def dit_ln_modulate_h256q(x, x_dtype, rows, dim, shift, scale, mode, eps, q, qscale, stream=None,
                          norm=DIT_LAYERNORM):
    _check(lib().dit_ln_modulate_h256q(_p(x), int(x_dtype), int(rows), int(dim), int(norm), _p(shift), _p(scale),
                                       int(mode), float(eps), _p(q), _p(qscale), _stream(stream)))


def dit_gemm_w8a8_gated_residual(a, a_scale, w, w_scale, M, N, K, resid, resid_dtype, gate, bias, out, out_dtype,
                                 stream=None, gate_fn=DIT_GATE_IDENTITY):
    _check(lib().dit_gemm_w8a8_gated_residual(_p(a), _p(a_scale), _p(w), _p(w_scale), int(M), int(N), int(K),
                                              _p(resid), int(resid_dtype), _p(gate), int(gate_fn), _p(bias), _p(out),
                                              int(out_dtype), _stream(stream)))


def dit_gemm_w8a8_swiglu(a, a_scale, w_gate_up, w_scale, M, F, K, u, stream=None, act=DIT_ACT_SILU):
    _check(lib().dit_gemm_w8a8_swiglu(_p(a), _p(a_scale), _p(w_gate_up), _p(w_scale), int(M), int(F), int(K),
                                      int(act), _p(u), _stream(stream)))


def dit_qkv_rope_w8a8(desc, h, h_scale, w_qkv, w_scale, q_g, q_b, k_g, k_b, rope_cos, rope_sin, q, k, vt,
                      stream=None):
    _check(lib().dit_qkv_rope_w8a8(C.byref(desc), _p(h), _p(h_scale), _p(w_qkv), _p(w_scale), _p(q_g), _p(q_b),
                                   _p(k_g), _p(k_b), _p(rope_cos), _p(rope_sin), _p(q), _p(k), _p(vt),
                                   _stream(stream)))


def dit_trace_begin(capacity: int = 1 << 16):
    _check(lib().dit_trace_begin(int(capacity)))


def dit_trace_end(path: Optional[str] = None):
    _check(lib().dit_trace_end(None if path is None else os.fsencode(path)))


def dit_status_string(status: int) -> str:
    return lib().dit_status_string(int(status)).decode()


def dit_last_error() -> str:
    return lib().dit_last_error().decode()


def dit_version() -> str:
    return lib().dit_version().decode()

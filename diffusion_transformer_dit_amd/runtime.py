"""Device-memory plumbing around the C ABI: torch owns the buffers, libdit.so
does the work.  Used by the tests, the smoke check and the benchmark."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import inputs as I
from . import native as N


def _torch():
    import torch
    return torch


def require_gpu():
    torch = _torch()
    if not torch.cuda.is_available():
        raise RuntimeError("no HIP device visible: the DiT path runs only on the GPU")
    N.lib()


def to_dev_bf16(a: np.ndarray, device="cuda"):
    """Upload fp32 values (already bf16-representable or not) as bf16 (RNE)."""
    torch = _torch()
    bits = I.bf16_bits(np.asarray(a, np.float32))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_f32(a: Optional[np.ndarray], device="cuda"):
    if a is None:
        return None
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def to_host_f32(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def desc_of(cfg: I.DiTConfig, x_dtype: Optional[str] = None) -> N.dit_block_desc:
    xd = cfg.x_dtype if x_dtype is None else x_dtype
    return N.make_desc(cfg.batch, cfg.seq, cfg.hidden, cfg.heads, cfg.kv_heads, cfg.head_dim, cfg.ffn, cfg.cond_dim,
                       qk_norm=cfg.qk_norm,
                       rope=N.DIT_ROPE_INTERLEAVED if cfg.rope == "interleaved3d" else N.DIT_ROPE_HALF,
                       eps=cfg.eps, x_dtype=N.DIT_F32 if xd == "f32" else N.DIT_BF16,
                       w_dtype=N.DIT_F32 if cfg.fmt == "f32" else N.DIT_BF16,
                       norm=N.DIT_RMSNORM if cfg.norm == "rmsnorm" else N.DIT_LAYERNORM,
                       act=N.DIT_ACT_GELU_TANH if cfg.act == "gelu_tanh" else N.DIT_ACT_SILU,
                       gate={"identity": N.DIT_GATE_IDENTITY, "tanh": N.DIT_GATE_TANH,
                             "sigmoid": N.DIT_GATE_SIGMOID}[cfg.gate],
                       mod=N.DIT_MOD_SCALE_GATE if cfg.mod == "scale_gate" else N.DIT_MOD_SHIFT_SCALE_GATE,
                       qk_order=N.DIT_QK_ROPE_NORM if cfg.qk_order == "rope_norm" else N.DIT_QK_NORM_ROPE,
                       fmt=N.DIT_FMT_W8A8_H256 if cfg.fmt == "w8a8_h256" else N.DIT_FMT_BF16)


def rope_tables(cfg: I.DiTConfig, pos: Optional[np.ndarray] = None, device="cuda"):
    """cos/sin tables built by the library's host helper, uploaded to the device."""
    if pos is None:
        pos = I.positions(cfg)
    rope = N.DIT_ROPE_INTERLEAVED if cfg.rope == "interleaved3d" else N.DIT_ROPE_HALF
    cos, sin = N.dit_rope_tables(pos, rope, cfg.rope_axes, cfg.rope_theta, cfg.head_dim)
    return to_dev_f32(cos, device), to_dev_f32(sin, device)


_BF16_KEYS = ("w_ada", "w_qkv", "w_o", "w_gate_up", "w_down")


class DeviceBlock:
    """One block's parameters resident in HBM plus the matching C struct
    (matrices bf16, or fp32 with f32=True for the fp32 path)."""

    def __init__(self, w: Dict[str, Optional[np.ndarray]], device="cuda", tensors=None, f32: bool = False):
        if tensors is None:
            tensors = {}
            for k, v in w.items():
                if v is None:
                    tensors[k] = None
                elif k in _BF16_KEYS and not f32:
                    tensors[k] = to_dev_bf16(v, device)
                else:
                    tensors[k] = to_dev_f32(v, device)
        self.t = tensors
        self.c = N.make_weights(tensors)


PROJECTIONS = {"w_qkv": "s_qkv", "w_o": "s_o", "w_gate_up": "s_gate_up", "w_down": "s_down"}


def quantize_h256(x, stream=None):
    """(int8 codes, fp32 row scales) of a 2-D device tensor (bf16 or fp32) by
    the library's dit_quantize_h256."""
    torch = _torch()
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty(rows, dtype=torch.float32, device=x.device)
    N.dit_quantize_h256(x, N.DIT_F32 if x.dtype == torch.float32 else N.DIT_BF16, rows, cols, q, s, stream)
    return q, s


def quantize_block(blk: DeviceBlock, stream=None) -> DeviceBlock:
    """The W8A8 H256 form of a block: its four projections replaced by their
    int8 codes and row scales, prepared once on the device; every other
    tensor is shared with `blk`."""
    t = dict(blk.t)
    for k, sk in PROJECTIONS.items():
        t[k], t[sk] = quantize_h256(blk.t[k], stream)
    return DeviceBlock({}, tensors=t)


def alloc_ws(nbytes: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def block_forward(cfg: I.DiTConfig, blk: DeviceBlock, x, cond, cos, sin, out=None, ws=None, stream=None):
    """out = block(x, cond) on the device; returns out."""
    torch = _torch()
    desc = desc_of(cfg)
    if out is None:
        out = torch.empty_like(x)
    if ws is None:
        ws = alloc_ws(N.dit_block_workspace_size(desc), x.device)
    N.dit_block_forward(desc, blk.c, x, cond, cos, sin, out, ws, stream)
    return out


class DeviceStack:
    """A stack of blocks with one shared AdaLN linear and the stack edges."""

    def __init__(self, cfg: I.DiTConfig, blocks, edges: Dict[str, object]):
        self.cfg = cfg
        self.blocks = blocks            # list of DeviceBlock
        self.edges = edges              # name -> device tensor
        self.desc = desc_of(cfg, "f32")
        self.model = N.make_model(self.desc, [b.c for b in blocks], cfg.latent_dim, edges)
        self.ws = alloc_ws(N.dit_stack_workspace_size(self.model))

    def step(self, latent, cond, cos, sin, velocity, stream=None):
        N.dit_stack_step(self.model, latent, cond, cos, sin, velocity, self.ws, stream)


def upload_edges(e: Dict[str, np.ndarray], device="cuda", f32: bool = False):
    return {k: (to_dev_bf16(v, device) if k.startswith("w_") and not f32 else to_dev_f32(v, device))
            for k, v in e.items()}


def denoise(stack: DeviceStack, latent, cos, sin, steps: int, shift: float, start: int = 0, stream=None):
    """The flow-match Euler loop on the device (latent updated in place)."""
    torch = _torch()
    sig = N.dit_flowmatch_sigmas(steps, shift)
    cond = torch.empty(stack.cfg.cond_dim, dtype=torch.float32, device=latent.device)
    vel = torch.empty_like(latent)
    for i in range(start, steps):
        N.dit_sigma_embedding(float(sig[i]), stack.cfg.cond_dim, cond, stream)
        stack.step(latent, cond, cos, sin, vel, stream)
        N.euler_flowmatch_update(latent, vel, latent.numel(), float(sig[i]), float(sig[i + 1]), stream)
    return latent


class DeviceLoop:
    """The whole flow-match loop recorded by the library as one HIP graph per
    step (dit_loop_create); each replay updates `latent` in place.  The
    latent, rope tables and the stack's weights must stay alive and in place
    while the loop exists."""

    def __init__(self, stack: DeviceStack, latent, cos, sin, steps: int, shift: float):
        self.stack, self.latent, self.cos, self.sin = stack, latent, cos, sin
        self.steps = steps
        self.ws = alloc_ws(N.dit_loop_workspace_size(stack.model))
        self.handle = N.dit_loop_create(stack.model, latent, cos, sin, steps, shift, self.ws)

    def step(self, i: int, stream=None):
        N.dit_loop_launch_step(self.handle, i, stream)

    def run(self, start: int = 0, stream=None):
        for i in range(start, self.steps):
            self.step(i, stream)
        return self.latent

    def close(self):
        if self.handle:
            _torch().cuda.synchronize()
            N.dit_loop_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


"""Robustness of the device path on normal runs.

* Guard bands: bytes of a known pattern placed right after `out`,
  `velocity` and the workspace stay untouched (ragged row counts, where a
  tile's tail rows are masked, included).
* NaN propagation: a NaN in one token row of one sequence is not masked.
  Attention mixes every key of a sequence into every query, so the oracle
  makes that whole sequence non-finite and leaves the other sequence of the
  batch finite; the GPU output has the same non-finite mask and matches the
  oracle on the finite part (the NaN cascade through the residual stream of
  the ERNIE page, §V Bug 1).
* Outliers: residual channels at +-1e4 (the ERNIE page, §VII Decision 1,
  reports residual values past 14,000) through the fp32 residual stream of
  the stack step, against the oracle.
"""
import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R
from oracle import dit as O

from gpu_helpers import assert_parity, say

pytestmark = pytest.mark.gpu

GUARD = 4096            # bytes after each guarded buffer
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def _sync():
    import torch
    torch.cuda.synchronize()


def _guarded(nbytes):
    """A device byte buffer of nbytes followed by GUARD bytes of PATTERN;
    returns (whole buffer, the first nbytes)."""
    import torch
    big = torch.full((nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
    return big, big[:nbytes]


def _guard_intact(big, nbytes, what):
    tail = big[nbytes:].cpu().numpy()
    bad = int((tail != PATTERN).sum())
    say(f"  guard after {what}: {bad} of {GUARD} bytes changed")
    assert bad == 0, what


@pytest.mark.parametrize("name", ["c1_ragged200", "gqa3_b2_ragged300", "tiny_joint"])
def test_block_guard_bands(name):
    import torch
    from gpu_helpers import SMALL
    cfg = SMALL[name].replace(x_dtype="bf16")
    w = I.block_weights(cfg, 0)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    desc = R.desc_of(cfg)
    blk = R.DeviceBlock(w)
    cos, sin = R.rope_tables(cfg, pos)
    nout = cfg.tokens * cfg.hidden * 2
    obig, ob = _guarded(nout)
    out = ob.view(torch.bfloat16).view(cfg.tokens, cfg.hidden)
    nws = N.dit_block_workspace_size(desc)
    wbig, wsb = _guarded(nws)
    N.dit_block_forward(desc, blk.c, R.to_dev_bf16(x), R.to_dev_f32(c), cos, sin, out, wsb, ws_bytes=nws)
    _sync()
    _guard_intact(obig, nout, f"{name} out")
    _guard_intact(wbig, nws, f"{name} workspace")
    ref = O.block_forward(x, c, w, cfg, pos)
    assert_parity(R.to_host_f32(out), ref, what=f"{name} out")


def _small_stack(cfg, edit_edges=None):
    shared = I.shared_ada(cfg)
    blocks = [I.stack_block_weights(cfg, l, shared) for l in range(cfg.layers)]
    edges = I.stack_edges(cfg)
    if edit_edges:
        edit_edges(edges)
    dev_shared = {"w_ada": R.to_dev_bf16(shared["w_ada"]), "b_ada": R.to_dev_f32(shared["b_ada"])}
    dblocks = []
    for w in blocks:
        t = {k: (None if v is None else (R.to_dev_bf16(v) if k in R._BF16_KEYS else R.to_dev_f32(v)))
             for k, v in w.items() if k not in ("w_ada", "b_ada")}
        t.update(dev_shared)
        dblocks.append(R.DeviceBlock(None, tensors=t))
    return blocks, edges, R.DeviceStack(cfg, dblocks, R.upload_edges(edges))


STK = I.C1.replace(name="stack_ragged", cfg_id=25, x_dtype="f32", layers=2, latent_dim=128, grid=(1, 13, 23))


def test_stack_guard_bands():
    import torch
    cfg = STK                  # 299 tokens: ragged against every row tile
    blocks, edges, stack = _small_stack(cfg)
    pos = I.positions(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    lat = I.latent(cfg)
    cond = torch.empty(cfg.cond_dim, dtype=torch.float32, device="cuda")
    N.dit_sigma_embedding(0.75, cfg.cond_dim, cond)
    nv = cfg.tokens * cfg.latent_dim * 4
    vbig, vb = _guarded(nv)
    vel = vb.view(torch.float32).view(cfg.tokens, cfg.latent_dim)
    nws = N.dit_stack_workspace_size(stack.model)
    wbig, wsb = _guarded(nws)
    N.dit_stack_step(stack.model, R.to_dev_f32(lat), cond, cos, sin, vel, wsb, ws_bytes=nws)
    _sync()
    _guard_intact(vbig, nv, "velocity")
    _guard_intact(wbig, nws, "stack workspace")
    ref = O.stack_step(lat, float(np.float32(0.75)), blocks, edges, cfg, pos)
    assert_parity(R.to_host_f32(vel), ref, what="ragged stack velocity")


def test_nan_row_propagates_within_its_sequence():
    cfg = I.C1.replace(name="c1_nan_b2", cfg_id=26, batch=2, x_dtype="f32")
    w = I.block_weights(cfg, 0)
    x, c, pos = I.block_x(cfg).copy(), I.cond(cfg), I.positions(cfg)
    bad = 37                                     # a row of sequence 0
    x[bad, 5] = np.nan
    with np.errstate(invalid="ignore"):
        ref = O.block_forward(x, c, w, cfg, pos)
    fin_ref = np.isfinite(ref)
    assert not fin_ref[: cfg.seq].any() and fin_ref[cfg.seq:].all()
    blk = R.DeviceBlock(w)
    cos, sin = R.rope_tables(cfg, pos)
    out = R.block_forward(cfg, blk, R.to_dev_f32(x), R.to_dev_f32(c), cos, sin)
    _sync()
    got = R.to_host_f32(out)
    fin = np.isfinite(got)
    say(f"  non-finite rows: GPU {int((~fin).any(1).sum())}, oracle {int((~fin_ref).any(1).sum())}")
    np.testing.assert_array_equal(fin, fin_ref)
    assert_parity(got[cfg.seq:], ref[cfg.seq:], what="the clean sequence")


def test_residual_outlier_channels_stack():
    """Four channels of the fp32 residual stream at +-1e4 (set by the patch
    embedding's bias) through two blocks and the final layer."""
    import torch
    chans = [3, 77, 130, 255]

    def outliers(e):
        e["b_in"] = e["b_in"].copy()
        e["b_in"][chans] = np.array([1e4, -1e4, 1e4, -1e4], np.float32)

    cfg = STK.replace(name="stack_outliers", cfg_id=27, grid=(1, 16, 16))
    blocks, edges, stack = _small_stack(cfg, outliers)
    pos = I.positions(cfg)
    cos, sin = R.rope_tables(cfg, pos)
    lat = I.latent(cfg)
    for sig in (1.0, 0.5):
        cond = torch.empty(cfg.cond_dim, dtype=torch.float32, device="cuda")
        N.dit_sigma_embedding(sig, cfg.cond_dim, cond)
        vel = torch.empty((cfg.tokens, cfg.latent_dim), dtype=torch.float32, device="cuda")
        stack.step(R.to_dev_f32(lat), cond, cos, sin, vel)
        _sync()
        got = R.to_host_f32(vel)
        assert np.isfinite(got).all()
        ref = O.stack_step(lat, sig, blocks, edges, cfg, pos)
        assert_parity(got, ref, what=f"velocity with +-1e4 residual channels, sigma {sig}")

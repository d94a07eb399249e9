"""The library's per-launch tracer: one Chrome-trace "X" event per kernel
launch, in launch order, with positive device durations, and no effect on
the results."""
import json
import os

import numpy as np
import pytest

from diffusion_transformer_dit_amd import inputs as I
from diffusion_transformer_dit_amd import native as N
from diffusion_transformer_dit_amd import runtime as R

pytestmark = pytest.mark.gpu

BLOCK_ORDER = ["adaln_gemv", "ln_modulate", "vt_pad_zero", "gemm_qkv", "flash_attention", "gemm_gated_residual",
               "ln_modulate", "gemm_swiglu", "gemm_gated_residual"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    R.require_gpu()


def test_trace_of_block_forward(tmp_path):
    import torch
    cfg = I.C1.replace(name="trace_block", x_dtype="f32", seq_override=200)   # ragged: split-KV attention
    w = I.block_weights(cfg, 0)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    blk = R.DeviceBlock(w)
    cos, sin = R.rope_tables(cfg, pos)
    xd, cd = R.to_dev_f32(x), R.to_dev_f32(c)
    plain = R.to_host_f32(R.block_forward(cfg, blk, xd, cd, cos, sin))
    path = str(tmp_path / "trace.json")
    N.dit_trace_begin(256)
    try:
        out = R.block_forward(cfg, blk, xd, cd, cos, sin)
        out2 = R.block_forward(cfg, blk, xd, cd, cos, sin)
    finally:
        N.dit_trace_end(path)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(R.to_host_f32(out), plain)
    np.testing.assert_array_equal(R.to_host_f32(out2), plain)
    ev = json.load(open(path))["traceEvents"]
    names = [e["name"] for e in ev]
    print("trace:", [(e["name"], round(e["dur"], 1)) for e in ev[:9]], flush=True)
    assert names == BLOCK_ORDER * 2
    assert all(e["ph"] == "X" and e["dur"] > 0 for e in ev)
    ts = [e["ts"] for e in ev]
    assert all(b >= a for a, b in zip(ts, ts[1:]))              # one stream: launch order is time order
    assert "M=200" in ev[3]["args"]["shape"] and "nsplit=" in ev[4]["args"]["shape"]
    # recording stopped: a later launch leaves no trace and ending again is an error
    R.block_forward(cfg, blk, xd, cd, cos, sin)
    with pytest.raises(N.DitError):
        N.dit_trace_end(path)


def test_trace_records_only_real_launches(tmp_path):
    """At a sequence length that is a multiple of 64 the transposed V has no
    padded key columns, so the pad kernel is not launched and leaves no record."""
    cfg = I.C1.replace(name="trace_block_256", x_dtype="f32", seq_override=256)
    w = I.block_weights(cfg, 0)
    x, c, pos = I.block_x(cfg), I.cond(cfg), I.positions(cfg)
    blk = R.DeviceBlock(w)
    cos, sin = R.rope_tables(cfg, pos)
    xd, cd = R.to_dev_f32(x), R.to_dev_f32(c)
    path = str(tmp_path / "trace256.json")
    N.dit_trace_begin(64)
    try:
        R.block_forward(cfg, blk, xd, cd, cos, sin)
    finally:
        N.dit_trace_end(path)
    names = [e["name"] for e in json.load(open(path))["traceEvents"]]
    assert names == [n for n in BLOCK_ORDER if n != "vt_pad_zero"]

"""GPU parity of the quantizers against the oracle: bit-exact codes and scales.

quantize_nvfp4 (activations and weights), quantize_int4_g128 and fit_lut2,
called through the C ABI on seeded synthetic inputs with the workloads'
shapes, value distributions and outliers.  Every code and every scale is
compared, at every size: at the largest ones the oracle runs over row
chunks in parallel threads (tests/oracle_rows.py), with the tensor scale
taken over the whole tensor.
"""

import numpy as np
import pytest
import torch

from decode_nvfp4_rtn_amd import synth, configs
from oracle import nvfp4, int4, lut2
from tests import oracle_rows as orows
from tests.gpu_common import (require_gpu, say, dev_f32, dev_bf16, host_u8, host_u16)

pytestmark = pytest.mark.gpu


def _check_nvfp4(q, x_host_f32, x_dev, rows=None, static=None):
    ts = None if static is None else torch.tensor([static], dtype=torch.float32, device="cuda")
    codes, scales, st = q.quantize_nvfp4(x_dev, tensor_scale=ts)
    torch.cuda.synchronize()
    ref_st = nvfp4.tensor_scale(x_host_f32) if static is None else np.float32(static)
    assert np.float32(st.item()) == ref_st
    sel = np.arange(x_host_f32.shape[0]) if rows is None else rows
    rc, rs, _ = nvfp4.quantize(x_host_f32[sel], s_t=ref_st)
    gc, gs = host_u8(codes)[sel], host_u8(scales)[sel]
    assert np.array_equal(gs, rs), f"scales differ at {np.argwhere(gs != rs)[:5]}"
    assert np.array_equal(gc, rc), f"codes differ at {np.argwhere(gc != rc)[:5]}"
    return codes, scales, st


def test_quantize_tiny_fp32_activations():
    q = require_gpu()
    x = synth.activations(1, 0, 64, 512, outliers="channels")
    say("quantize tiny fp32 64x512")
    _check_nvfp4(q, x, dev_f32(x))


def test_quantize_tiny_fp32_weights():
    q = require_gpu()
    w = synth.weights(1, 0, 256, 512)
    say("quantize tiny weights 256x512")
    _check_nvfp4(q, w, dev_f32(w))


# The activations the prefill measurements quantize: the Qwen3-8B-like qkv
# (K = 4096) and down (K = 12288) inputs at M = 8192, and the 27B-class qkv
# (K = 5120) and down (K = 17408) inputs up to M = 32768 (1.14 GB of bf16).
@pytest.mark.parametrize("cfg,li,m", [
    (configs.QWEN3_PREFILL, 0, 8192),
    (configs.QWEN3_PREFILL, 3, 8192),
    (configs.BIG27_PREFILL, 3, 4096),
    (configs.BIG27_PREFILL, 0, 32768),
    (configs.BIG27_PREFILL, 3, 32768),
], ids=["qwen3-qkv-8192", "qwen3-down-8192", "27b-down-4096", "27b-qkv-32768",
        "27b-down-32768"])
def test_quantize_bf16_full_size_every_row(cfg, li, m):
    q = require_gpu()
    k = cfg.layers[li].k
    say("quantize bf16 every row", cfg.name, cfg.layers[li].name, m, k)
    bits = orows.activations_bf16(cfg.cid, li, m, k, outliers=cfg.outliers)
    codes, scales, st = q.quantize_nvfp4(dev_bf16(bits))
    torch.cuda.synchronize()
    gc, gs, gt = host_u8(codes), host_u8(scales), np.float32(st.item())
    del codes, scales
    xf = orows.bf16_as_f32(bits)
    del bits
    ref_st = nvfp4.tensor_scale(xf)
    assert gt == ref_st
    rc, rs, _ = orows.nvfp4_quantize(xf, ref_st)
    assert orows.first_mismatch(gs, rs) is None, f"scales differ at {orows.first_mismatch(gs, rs)}"
    assert orows.first_mismatch(gc, rc) is None, f"codes differ at {orows.first_mismatch(gc, rc)}"


@pytest.mark.parametrize("m,k", [(1, 16), (3, 48), (17, 1040), (300, 512), (1000, 64)])
def test_quantize_ragged_shapes(m, k):
    q = require_gpu()
    x = synth.activations(9, m, m, k, outliers="elements")
    say("quantize ragged", m, k)
    _check_nvfp4(q, x, dev_f32(x))
    bits = synth.to_bf16_bits(x)
    _check_nvfp4(q, synth.bf16_bits_as_f32(bits), dev_bf16(bits))


def test_quantize_static_scale_and_saturation():
    q = require_gpu()
    x = synth.activations(9, 1, 128, 256)
    say("quantize static scale")
    _check_nvfp4(q, x, dev_f32(x), static=np.float32(1e-3))   # many groups saturate at 448
    _check_nvfp4(q, x, dev_f32(x), static=np.float32(0.25))   # many groups underflow


def test_quantize_zero_and_signed_zero():
    q = require_gpu()
    x = np.zeros((4, 64), dtype=np.float32)
    x[1, 5] = -0.0
    x[2] = -0.0
    say("quantize zeros")
    _check_nvfp4(q, x, dev_f32(x))
    y = np.zeros((2, 64), dtype=np.float32)
    y[0, 0] = 1000.0
    y[1, 16:] = -1e-9
    _check_nvfp4(q, y, dev_f32(y))


def test_quantize_is_deterministic():
    q = require_gpu()
    bits = synth.activations_bf16(2, 1, 2048, 4096, outliers="channels")
    x = dev_bf16(bits)
    say("quantize determinism")
    a = q.quantize_nvfp4(x)
    b = q.quantize_nvfp4(x)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ------------------------------------------------------------------ INT4 --

@pytest.mark.parametrize("li", range(4))
def test_int4_quantizer_bitexact_every_row(li):
    """The four Qwen3-8B-like decode layers, every row."""
    q = require_gpu()
    cfg = configs.QWEN3_DECODE
    n, k = cfg.layers[li].n, cfg.layers[li].k
    w, rc, rs = orows.int4_layer(cfg.cid, li, n, k)
    say("int4 quantize every row", cfg.layers[li].name, n, k)
    codes, scales = q.quantize_int4_g128(dev_f32(w))
    torch.cuda.synchronize()
    gs, gc = host_u16(scales), host_u8(codes)
    assert orows.first_mismatch(gs, rs) is None, f"scales differ at {orows.first_mismatch(gs, rs)}"
    assert orows.first_mismatch(gc, rc) is None, f"codes differ at {orows.first_mismatch(gc, rc)}"


def test_int4_quantizer_tiny():
    q = require_gpu()
    w = synth.weights(1, 0, 256, 512)
    say("int4 quantize tiny")
    codes, scales = q.quantize_int4_g128(dev_f32(w))
    torch.cuda.synchronize()
    rc, rs = int4.quantize(w)
    assert np.array_equal(host_u16(scales), rs)
    assert np.array_equal(host_u8(codes), rc)


def test_int4_quantizer_edge_groups():
    q = require_gpu()
    w = synth.weights(9, 2, 32, 384)
    w[0, :128] = 0.0
    w[1, :] = 0.3
    w[2, 128:256] = -1e-30
    say("int4 edge groups")
    codes, scales = q.quantize_int4_g128(dev_f32(w))
    torch.cuda.synchronize()
    rc, rs = int4.quantize(w)
    assert np.array_equal(host_u16(scales), rs)
    assert np.array_equal(host_u8(codes), rc)


# ------------------------------------------------------------------ LUT2 --

@pytest.mark.parametrize("li", range(3))
def test_lut2_fit_bitexact_every_row(li):
    """The three Gemma3-12B-like layers (3840 x 3840, 30720 x 3840,
    3840 x 15360), every row."""
    q = require_gpu()
    cfg = configs.GEMMA3_LUT2
    n, k = cfg.layers[li].n, cfg.layers[li].k
    w, ri, rc = orows.lut2_layer(cfg.cid, li, n, k)
    say("lut2 fit every row", cfg.layers[li].name, n, k)
    idx, cent = q.fit_lut2(dev_f32(w))
    torch.cuda.synchronize()
    gcent, gidx = host_u16(cent), host_u8(idx)
    assert orows.first_mismatch(gcent, rc) is None, f"centroids differ at {orows.first_mismatch(gcent, rc)}"
    assert orows.first_mismatch(gidx, ri) is None, f"indices differ at {orows.first_mismatch(gidx, ri)}"


def test_lut2_fit_long_rows():
    """Rows of 15360 and 3840 weights drawn from other seeds than the layers."""
    q = require_gpu()
    for n, k in [(64, 3840), (48, 15360)]:
        w = synth.weights(5, 0, n, k)
        say("lut2 fit", n, k)
        idx, cent = q.fit_lut2(dev_f32(w))
        torch.cuda.synchronize()
        ri, rc = lut2.fit(w)
        assert np.array_equal(host_u16(cent), rc)
        assert np.array_equal(host_u8(idx), ri)


def test_lut2_fit_special_rows():
    q = require_gpu()
    rng = np.random.default_rng(5)
    vals = np.array([-0.375, -0.0625, 0.125, 0.5], dtype=np.float32)
    w = np.stack([rng.permutation(np.repeat(vals, 32)) for _ in range(16)])
    w[3] = 0.0
    w[4, :100] = -0.0
    w[5] = np.abs(w[5])
    say("lut2 special rows")
    idx, cent = q.fit_lut2(dev_f32(w))
    torch.cuda.synchronize()
    ri, rc = lut2.fit(w)
    assert np.array_equal(host_u16(cent), rc)
    assert np.array_equal(host_u8(idx), ri)

"""GPU parity of the quantizers against the oracle: bit-exact codes and scales.

quantize_nvfp4 (activations and weights), quantize_int4_g128 and fit_lut2,
called through the C ABI on seeded synthetic inputs with the workloads'
shapes, value distributions and outliers.  At the largest sizes the oracle
recomputes the tensor scale from the whole tensor and checks a seeded sample
of rows (always including the last).
"""

import numpy as np
import pytest
import torch

from decode_nvfp4_rtn_amd import synth
from oracle import nvfp4, int4, lut2
from tests.gpu_common import (require_gpu, say, dev_f32, dev_bf16, host_u8, host_u16,
                              sample_rows)

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


@pytest.mark.parametrize("m,k,outl,cfg", [
    (8192, 4096, "channels", 2),
    (8192, 12288, "channels", 2),
    (4096, 17408, "elements", 4),
    (32768, 5120, "elements", 4),
])
def test_quantize_bf16_full_size_sampled(m, k, outl, cfg):
    q = require_gpu()
    bits = synth.activations_bf16(cfg, 0, m, k, outliers=outl)
    xf = synth.bf16_bits_as_f32(bits)
    say("quantize bf16", m, k, outl)
    _check_nvfp4(q, xf, dev_bf16(bits), rows=sample_rows(m, 96, m + k))


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

@pytest.mark.parametrize("n,k,cfg", [(256, 512, 1), (6144, 4096, 3), (4096, 12288, 3)])
def test_int4_quantizer_bitexact(n, k, cfg):
    q = require_gpu()
    w = synth.weights(cfg, 0, n, k)
    say("int4 quantize", n, k)
    codes, scales = q.quantize_int4_g128(dev_f32(w))
    torch.cuda.synchronize()
    rows = sample_rows(n, 512, n + k)
    rc, rs = int4.quantize(w[rows])
    assert np.array_equal(host_u16(scales)[rows], rs)
    assert np.array_equal(host_u8(codes)[rows], rc)


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

@pytest.mark.parametrize("n,k", [(64, 3840), (48, 15360), (3840, 3840)])
def test_lut2_fit_bitexact(n, k):
    q = require_gpu()
    w = synth.weights(5, 0, n, k)
    say("lut2 fit", n, k)
    idx, cent = q.fit_lut2(dev_f32(w))
    torch.cuda.synchronize()
    rows = sample_rows(n, 64, n + k)
    ri, rc = lut2.fit(w[rows])
    assert np.array_equal(host_u16(cent)[rows], rc)
    assert np.array_equal(host_u8(idx)[rows], ri)


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

"""Pins for oracle.gemm (products on dequantized operands) and the pass rule."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm, nvfp4, int4, lut2, formats as F
from decode_nvfp4_rtn_amd import synth


def _exact_matmul(a, b):
    """Exact rational A B^T."""
    m, k = a.shape
    n = b.shape[0]
    fa = [[Fraction(float(v)) for v in row] for row in a]
    fb = [[Fraction(float(v)) for v in row] for row in b]
    return [[sum((fa[i][t] * fb[j][t] for t in range(k)), Fraction(0)) for j in range(n)]
            for i in range(m)]


def test_w4a4_brute_force_4x16x32():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    w = (rng.standard_normal((16, 32)) / 4).astype(np.float32)
    ac, as_, at = nvfp4.quantize(x)
    wc, ws, wt = nvfp4.quantize(w)
    y = gemm.w4a4(ac, as_, at, wc, ws, wt)
    assert y.shape == (4, 16)
    ref = _exact_matmul(nvfp4.dequantize(ac, as_, at), nvfp4.dequantize(wc, ws, wt))
    for i in range(4):
        for j in range(16):
            r = ref[i][j]
            assert abs(Fraction(float(y[i, j])) - r) <= abs(r) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


def test_w4a4_is_not_transposed():
    # asymmetric shapes: a transposed operand cannot produce [m, n]
    rng = np.random.default_rng(42)
    x = rng.standard_normal((3, 48)).astype(np.float32)
    w = rng.standard_normal((5, 48)).astype(np.float32)
    y = gemm.w4a4(*nvfp4.quantize(x), *nvfp4.quantize(w))
    assert y.shape == (3, 5)


def test_w4a4_constant_inputs_closed_form():
    x = np.full((2, 64), 0.7, dtype=np.float32)
    w = np.full((3, 64), -0.05, dtype=np.float32)
    ac, as_, at = nvfp4.quantize(x)
    wc, ws, wt = nvfp4.quantize(w)
    y = gemm.w4a4(ac, as_, at, wc, ws, wt)
    xh = 2688.0 * np.float64(at)
    wh = -2688.0 * np.float64(wt)
    assert np.all(y == 64 * xh * wh)


def test_w4a4_one_hot_rows_extract_weight_columns():
    rng = np.random.default_rng(43)
    w = rng.standard_normal((8, 32)).astype(np.float32)
    wc, ws, wt = nvfp4.quantize(w)
    wh = nvfp4.dequantize(wc, ws, wt)
    for k in (0, 7, 16, 31):
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, k] = 6.0          # quantizes to code 7 with scale 448: x_hat = 2688 s_t
        ac, as_, at = nvfp4.quantize(x)
        xh = nvfp4.dequantize(ac, as_, at)
        assert np.count_nonzero(xh) == 1 and xh[0, k] == 2688.0 * np.float64(at)
        y = gemm.w4a4(ac, as_, at, wc, ws, wt)
        assert np.array_equal(y[0], xh[0, k] * wh[:, k])


def test_w4a16_brute_force_and_one_hot():
    rng = np.random.default_rng(44)
    w = (rng.standard_normal((16, 256)) / 16).astype(np.float32)
    wc, ws = int4.quantize(w)
    xb = synth.to_bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    y = gemm.w4a16(xb, wc, ws)
    ref = _exact_matmul(synth.bf16_bits_as_f32(xb), int4.dequantize(wc, ws))
    for i in range(4):
        for j in range(16):
            r = ref[i][j]
            assert abs(Fraction(float(y[i, j])) - r) <= abs(r) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)
    wh = int4.dequantize(wc, ws)
    for k in (0, 127, 128, 255):
        e = np.zeros((1, 256), dtype=np.float32)
        e[0, k] = 1.0
        assert np.array_equal(gemm.w4a16(synth.to_bf16_bits(e), wc, ws)[0], wh[:, k])


def test_lut2_gemm_one_hot_and_constant():
    rng = np.random.default_rng(45)
    w = (rng.standard_normal((8, 64)) / 8).astype(np.float32)
    idx, cb = lut2.fit(w)
    wh = lut2.dequantize(idx, cb)
    for k in (0, 3, 63):
        e = np.zeros((1, 64), dtype=np.float32)
        e[0, k] = 1.0
        assert np.array_equal(gemm.lut2_gemm(synth.to_bf16_bits(e), idx, cb)[0], wh[:, k])
    ones = synth.to_bf16_bits(np.ones((1, 64), dtype=np.float32))
    y = gemm.lut2_gemm(ones, idx, cb)
    assert np.allclose(y[0], wh.sum(axis=1), rtol=1e-14, atol=0)


def test_pass_rule():
    y_ref = np.array([[1.0, -2.0], [0.5, 3.0]])
    rms = np.sqrt(np.mean(y_ref ** 2))
    assert gemm.normalized_max_error(y_ref, y_ref) == 0
    assert gemm.normalized_max_error(y_ref + 0.5e-3 * rms, y_ref) <= 1e-3
    assert gemm.normalized_max_error(y_ref + 2e-3 * rms, y_ref) > 1e-3
    yb = F.rn_bf16(y_ref.astype(np.float32) * np.float32(1.02)).astype(np.float64)
    assert not gemm.bf16_output_ok(yb, y_ref)
    yb = F.rn_bf16((y_ref * (1 + 1e-4)).astype(np.float32)).astype(np.float64)
    assert gemm.bf16_output_ok(yb, y_ref)

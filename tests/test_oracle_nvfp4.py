"""Pins for oracle.nvfp4 (NVFP4 round-to-nearest quantizer)."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4, formats as F
from decode_nvfp4_rtn_amd import synth
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                d[k] = float(v)
    return d


def test_structure_matches_pages():
    g = _golden("nvfp4_structure.txt")
    x = np.random.default_rng(0).standard_normal((3, 64)).astype(np.float32)
    codes, scales, s_t = nvfp4.quantize(x)
    assert nvfp4.GROUP == g["group_size"]
    assert scales.shape == (3, 64 // int(g["group_size"]))
    assert np.ndim(s_t) == 0 and g["tensor_scales_per_tensor"] == 1
    assert codes.shape == (3, 64 * int(g["element_bits"]) // 8)


def _representable_tensor(j, rng, rows=6, groups=5):
    """Elements c * s_g * 2^j; every group holds a +-6 * s_g * 2^j element, and
    one group has s_g = 448, so amax = 2688 * 2^j exactly."""
    mags = F.E2M1_MAGNITUDES
    scale_vals = F.dec_e4m3(np.arange(1, 0x7F))
    x = np.zeros((rows, groups * 16))
    for r in range(rows):
        for g in range(groups):
            s = 448.0 if (r == 0 and g == 0) else rng.choice(scale_vals)
            c = rng.choice(mags, 16) * rng.choice([-1, 1], 16)
            c[rng.integers(16)] = 6.0 * rng.choice([-1, 1])
            x[r, g * 16:(g + 1) * 16] = c * s * 2.0 ** j
    return x.astype(np.float32)


@pytest.mark.parametrize("j", [-20, -7, 0, 3, 10])
def test_exact_preservation_of_representable_tensors(j):
    rng = np.random.default_rng(100 + j)
    x = _representable_tensor(j, rng)
    assert np.array_equal(x.astype(np.float64) * 1, x)  # representable in fp32
    codes, scales, s_t = nvfp4.quantize(x)
    assert s_t == np.float32(2.0 ** j)
    xh = nvfp4.dequantize(codes, scales, s_t)
    assert np.array_equal(xh, x.astype(np.float64))


@pytest.mark.parametrize("c", [0.7, 1.0, 3.14159, 1e-3, 12345.0])
def test_constant_input_closed_form(c):
    x = np.full((4, 64), c, dtype=np.float32)
    codes, scales, s_t = nvfp4.quantize(x)
    assert s_t == F.rn32(np.float64(np.float32(c)) / 2688.0)
    assert np.all(codes == 0x77) and np.all(scales == 0x7E)
    xh = nvfp4.dequantize(codes, scales, s_t)
    assert np.all(xh == 2688.0 * np.float64(s_t))


def test_constant_closed_form_value_for_0_7():
    x = np.full((1, 16), 0.7, dtype=np.float32)
    xh = nvfp4.dequantize(*nvfp4.quantize(x))
    # 2688 * rn32(0.7f / 2688) = 0.699999958...: just below 0.7f, not equal to it
    assert abs(xh[0, 0] - 0.69999996) < 5e-9
    assert xh[0, 0] != np.float64(np.float32(0.7))


def test_nibble_order_even_column_low():
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 6.0, -1.0, 0.5
    codes, scales, s_t = nvfp4.quantize(x)
    # scale 448 -> p = 448 * s_t = 1: the codes are E2M1(6), E2M1(-1), E2M1(.5)
    assert codes[0, 0] == (0xA << 4) | 0x7
    assert codes[0, 1] == 0x1


def test_zero_tensor_and_zero_groups():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 3] = -0.0
    codes, scales, s_t = nvfp4.quantize(x)
    assert s_t == 0 and np.all(scales == 0)
    assert codes[1, 1] == 0x80 and np.count_nonzero(codes) == 1
    xh = nvfp4.dequantize(codes, scales, s_t)
    assert np.all(xh == 0) and not np.any(np.isnan(xh))
    # a group far below the tensor maximum gets scale 0 and sign-only codes
    y = np.zeros((1, 32), dtype=np.float32)
    y[0, 0] = 1000.0
    y[0, 16:] = -1e-9
    codes, scales, s_t = nvfp4.quantize(y)
    assert scales[0, 1] == 0 and np.all(codes[0, 8:] == 0x88)


def test_single_nonzero_element():
    x = np.zeros((3, 48), dtype=np.float32)
    x[2, 37] = -5.5
    codes, scales, s_t = nvfp4.quantize(x)
    xh = nvfp4.dequantize(codes, scales, s_t)
    assert xh[2, 37] == -2688.0 * np.float64(s_t)
    assert np.count_nonzero(xh) == 1


def _brute_cases():
    rng = np.random.default_rng(7)
    cases = []
    a = rng.standard_normal((4, 32)).astype(np.float32)
    a[:, 5] *= 10
    cases.append(a)
    b = (rng.standard_normal((4, 32)) * np.exp2(rng.integers(-12, 12, (4, 32)))).astype(np.float32)
    cases.append(b)
    c = rng.standard_normal((4, 32)).astype(np.float32)
    c[1, :16] = 0.0
    c[2, 16:] *= 1e-6        # group scale underflows to E4M3 subnormal / zero
    c[3, 0] = -0.0
    cases.append(c)
    d = np.round(rng.standard_normal((4, 32)) * 4) / 4   # many exact ties after scaling
    cases.append(d.astype(np.float32))
    return cases


@pytest.mark.parametrize("case", range(4))
def test_brute_force_4x16x32_exact_rationals(case):
    x = _brute_cases()[case]
    codes, scales, s_t = nvfp4.quantize(x)
    ref_codes, ref_scales, ref_st = exact.nvfp4_quantize_exact(x.tolist())
    assert float(s_t) == ref_st
    assert np.array_equal(scales, np.array(ref_scales, dtype=np.uint8))
    assert np.array_equal(nvfp4.unpack_codes(codes), np.array(ref_codes, dtype=np.uint8))


def test_dequantize_is_exact_product():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    codes, scales, s_t = nvfp4.quantize(x)
    xh = nvfp4.dequantize(codes, scales, s_t)
    c = nvfp4.unpack_codes(codes)
    for r in range(4):
        for k in range(32):
            ref = (Fraction(float(F.dec_e2m1(c[r, k])))
                   * Fraction(float(F.dec_e4m3(scales[r, k // 16])))
                   * Fraction(float(s_t)))
            assert Fraction(float(xh[r, k])) == ref


def test_static_tensor_scale_is_used():
    x = np.random.default_rng(9).standard_normal((2, 32)).astype(np.float32)
    codes, scales, s_t = nvfp4.quantize(x, s_t=np.float32(0.01))
    assert s_t == np.float32(0.01)
    codes2, scales2, _ = nvfp4.quantize(x * 2, s_t=np.float32(0.02))
    assert np.array_equal(codes, codes2) and np.array_equal(scales, scales2)


def test_reciprocal_reading_agrees_with_exact_division_on_tiny_config():
    """The oracle scales elements by a rounded reciprocal (x * rn32(1/p));
    the plainest real-number reading divides, x / p, rounded once.  Count the
    codes on which the two readings disagree on the tiny workload."""
    x = synth.activations(1, 0, 64, 512, outliers="channels")
    codes, scales, s_t = nvfp4.quantize(x)
    p = F.rn32(F.dec_e4m3(scales) * np.float64(s_t)).astype(np.float64)
    y_div = F.rn32(x.reshape(64, 32, 16).astype(np.float64) / p[:, :, None])
    alt = F.enc_e2m1(y_div).reshape(64, 512)
    assert np.count_nonzero(alt != nvfp4.unpack_codes(codes)) == 0

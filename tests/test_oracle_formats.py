"""Pins for oracle.formats: E2M1, E4M3, binary32 and bfloat16 rounding."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------- E2M1

def test_e2m1_decode_matches_spec_table():
    for code, val in _read_table("e2m1_values.txt"):
        got = F.dec_e2m1(np.array([int(code)]))[0]
        assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e2m1_roundtrip_all_16_codes():
    codes = np.arange(16, dtype=np.uint8)
    vals = F.dec_e2m1(codes).astype(np.float32)
    assert np.array_equal(F.enc_e2m1(vals), codes)


def test_e2m1_ties_go_to_even_code():
    # midpoint -> expected code (even mantissa bit)
    table = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for mid, code in table.items():
        assert F.enc_e2m1(np.float32(mid)) == code
        assert F.enc_e2m1(np.float32(-mid)) == code | 8
        up = np.nextafter(np.float32(mid), np.float32(np.inf))
        dn = np.nextafter(np.float32(mid), np.float32(0))
        lo_code = [c for c in range(8) if F.E2M1_MAGNITUDES[c] < mid][-1]
        assert F.enc_e2m1(up) == lo_code + 1
        assert F.enc_e2m1(dn) == lo_code


def test_e2m1_saturates_and_keeps_sign_of_zero():
    assert F.enc_e2m1(np.float32(1e30)) == 7
    assert F.enc_e2m1(np.float32(-7.0)) == 15
    assert F.enc_e2m1(np.float32(-0.0)) == 8
    assert F.enc_e2m1(np.float32(-0.1)) == 8
    assert F.enc_e2m1(np.float32(0.0)) == 0


def test_e2m1_brute_force_nearest_exact():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.uniform(-8, 8, 3000), rng.standard_normal(3000) * 2,
        np.exp2(rng.uniform(-30, 4, 2000)) * rng.choice([-1, 1], 2000),
    ]).astype(np.float32)
    got = F.enc_e2m1(v)
    for x, c in zip(v, got):
        ref = exact.nearest_code(abs(Fraction(float(x))), exact.E2M1) | (8 if x < 0 else 0)
        assert c == ref, (x, c, ref)


def test_e2m1_vectorised_nearest_large_sample():
    # 10^6 values in [2^-20, 8): float64 distances to the grid are exact here
    rng = np.random.default_rng(12)
    a = np.exp2(rng.uniform(-20, 3, 1_000_000)).astype(np.float32)
    got = F.enc_e2m1(a).astype(np.int64)
    d = np.abs(a.astype(np.float64)[:, None] - F.E2M1_MAGNITUDES[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates take the even code
    ref = np.where(cand.sum(1) > 1, np.argmax(cand & (np.arange(8) % 2 == 0), 1),
                   np.argmin(d, 1))
    ref = np.where(a > 6, 7, ref)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------- E4M3

def test_e4m3_anchor_values_from_spec():
    for code, val in _read_table("e4m3_anchors.txt"):
        got = F.dec_e4m3(np.array([int(code, 16)]))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e4m3_all_256_bytes_decode_like_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.dec_e4m3(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


def test_e4m3_reencode_all_finite_nonnegative_codes():
    codes = np.arange(0x7F)
    assert np.array_equal(F.enc_e4m3(F.dec_e4m3(codes).astype(np.float32)), codes)


def test_e4m3_matches_torch_cast_up_to_464():
    rng = np.random.default_rng(13)
    q = np.concatenate([
        np.exp2(rng.uniform(-14, np.log2(464), 200_000)),
        rng.uniform(0, 464, 50_000),
        (F.dec_e4m3(np.arange(0x7E)) + F.dec_e4m3(np.arange(1, 0x7F))) / 2,  # midpoints
    ]).astype(np.float32)
    q = q[q <= 464]
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.enc_e4m3(q), ref)


def test_e4m3_saturates_above_448():
    q = np.array([448, 449, 464, 465, 480, 1e6, 3e38], dtype=np.float32)
    assert np.all(F.enc_e4m3(q) == 0x7E)


def test_e4m3_brute_force_nearest_exact():
    rng = np.random.default_rng(14)
    q = np.concatenate([np.exp2(rng.uniform(-12, 9.5, 3000)), [0.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    q = q.astype(np.float32)
    got = F.enc_e4m3(q)
    for x, c in zip(q, got):
        assert c == exact.nearest_code(Fraction(float(x)), exact.E4M3), (x, c)


# ----------------------------------------------------------- bf16 / binary32

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(15)
    v = np.concatenate([rng.standard_normal(100_000) * 10.0 ** rng.uniform(-30, 30, 100_000),
                        rng.standard_normal(10_000)]).astype(np.float32)
    # exact midpoints between bf16 neighbours
    mids = (F.f32_bits(v[:5000]) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    v = np.concatenate([v, F.bits_f32(mids)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.rn_bf16_bits(v), ref)


def test_rn32_matches_exact_rounding():
    rng = np.random.default_rng(16)
    a = rng.standard_normal(2000).astype(np.float32)
    b = (rng.standard_normal(2000) * 3).astype(np.float32)
    for x, y in zip(a, b):
        fx, fy = Fraction(float(x)), Fraction(float(y))
        assert F.rn32(np.float64(x) * np.float64(y)) == exact.frac_to_f32(fx * fy)
        if y != 0:
            assert F.rn32(np.float64(x) / np.float64(y)) == exact.frac_to_f32(fx / fy)

"""Pins for oracle.int4 (symmetric INT4, group 128) and oracle.lut2 (2-bit codebook)."""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int4, lut2, formats as F
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------- INT4

def test_constant_group_gives_plus_minus_7():
    w = np.full((2, 256), 0.3, dtype=np.float32)
    w[1] = -0.3
    codes, scales = int4.quantize(w)
    q = int4.unpack(codes)
    assert np.all(q[0] == 7) and np.all(q[1] == -7)
    # the stored scale is bf16(rn32(0.3f / 7))
    s = F.bf16_bits_to_f32(scales)
    assert np.all(s == F.rn_bf16(F.rn32(np.float64(np.float32(0.3)) / 7)))


def test_representable_group_is_preserved():
    rng = np.random.default_rng(21)
    n, k = 4, 384
    s = F.rn_bf16(np.exp2(rng.uniform(-10, 2, (n, k // 128))).astype(np.float32))
    q = rng.integers(-7, 8, (n, k))
    q[:, ::128] = 7                          # each group reaches +-7 so amax/7 == s
    w = (q * np.repeat(s.astype(np.float64), 128, axis=1)).astype(np.float32)
    codes, scales = int4.quantize(w)
    assert np.array_equal(int4.unpack(codes), q)
    assert np.array_equal(int4.dequantize(codes, scales), w.astype(np.float64))


def test_int4_zero_group_and_range():
    w = np.zeros((1, 256), dtype=np.float32)
    w[0, 200] = 5.0
    codes, scales = int4.quantize(w)
    q = int4.unpack(codes)
    assert scales[0, 0] == 0 and np.all(q[0, :128] == 0)
    assert q[0, 200] == 7 and q.min() >= -7


def test_int4_brute_force_exact_rationals():
    rng = np.random.default_rng(22)
    w = (rng.standard_normal((3, 256)) / 16).astype(np.float32)
    codes, scales = int4.quantize(w)
    q = int4.unpack(codes)
    for r in range(3):
        for g in range(2):
            grp = w[r, g * 128:(g + 1) * 128]
            a = max(abs(Fraction(float(v))) for v in grp)
            s32 = exact.frac_to_f32(a / 7)
            # bf16 round-to-nearest-even of s32 via rationals: keep 8 significant bits
            e = Fraction(s32).numerator.bit_length() - Fraction(s32).denominator.bit_length()
            if Fraction(2) ** e > Fraction(s32):
                e -= 1
            quantum = Fraction(2) ** (e - 7)
            m = Fraction(s32) / quantum
            fl = m.numerator // m.denominator
            rem = m - fl
            if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
                fl += 1
            s = fl * quantum
            assert Fraction(float(F.bf16_bits_to_f32(scales[r, g]))) == s
            for i, v in enumerate(grp):
                t = Fraction(exact.frac_to_f32(Fraction(float(v)) / s))
                fl = t.numerator // t.denominator
                rem = t - fl
                qi = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
                qi = max(-7, min(7, qi))
                assert q[r, g * 128 + i] == qi


def test_marlin_bound_from_storage_layout():
    """Bits per weight of the stored INT4-g128 format against 16-bit weights
    reproduce the ~3.87x bound the MARLIN article quotes."""
    d = {}
    with open(os.path.join(GOLDEN, "marlin_bound.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, v = line.split()
                d[key] = float(v)
    n, k = 64, 1024
    codes, scales = int4.quantize(np.ones((n, k), dtype=np.float32))
    bits = 8 * (codes.nbytes + scales.nbytes) / (n * k)
    assert abs(16.0 / bits - d["bound_approx"]) <= d["tolerance"]


# --------------------------------------------------------------------- LUT2

def test_lut2_four_distinct_bf16_values_reproduced():
    rng = np.random.default_rng(31)
    vals = np.array([-0.375, -0.0625, 0.125, 0.5], dtype=np.float32)  # bf16-exact
    w = np.stack([rng.permutation(np.repeat(vals, 64)) for _ in range(5)])
    idx, cb = lut2.fit(w)
    assert np.array_equal(F.bf16_bits_to_f32(cb), np.tile(vals, (5, 1)))
    assert np.array_equal(lut2.dequantize(idx, cb), w.astype(np.float64))


def test_lut2_centroids_sorted_and_final_assignment_nearest():
    rng = np.random.default_rng(32)
    w = (rng.standard_normal((16, 512)) / np.sqrt(512)).astype(np.float32)
    w[3, :100] = 0.0                       # heavy duplicates
    w[4] = np.abs(w[4])                    # one-sided
    idx, cb = lut2.fit(w)
    c = F.bf16_bits_to_f32(cb).astype(np.float64)
    assert np.all(np.diff(c, axis=1) >= 0)
    ii = lut2.unpack(idx)
    d = np.abs(w.astype(np.float64)[:, :, None] - c[:, None, :])
    chosen = np.take_along_axis(d, ii[:, :, None], axis=2)[:, :, 0]
    assert np.all(chosen <= d.min(axis=2))
    # ties break to the lower index
    lower = np.argmin(d, axis=2)            # argmin returns the first minimum
    assert np.array_equal(ii, lower)


def test_lut2_objective_never_increases():
    rng = np.random.default_rng(33)
    w = (rng.standard_normal((32, 384)) * rng.uniform(0.01, 1, (32, 1))).astype(np.float32)
    _, hist = lut2.lloyd(w)
    h = np.stack(hist)
    assert np.all(np.diff(h, axis=0) <= 1e-12 * h[0])


def test_lut2_converged_centroids_are_cluster_means():
    """At a fixed point each centroid is the mean of the weights nearest to it."""
    rng = np.random.default_rng(34)
    w = np.concatenate([rng.normal(m, 0.01, 40) for m in (-1, -0.2, 0.3, 1.1)])
    w = rng.permutation(w).astype(np.float32)[None, :]
    c, _ = lut2.lloyd(w, iters=30)
    wd = w.astype(np.float64)[0]
    a = np.argmin(np.abs(wd[:, None] - c[0][None, :]), axis=1)
    for j in range(4):
        sel = sorted(Fraction(float(v)) for v in wd[a == j])
        mean = sum(sel, Fraction(0)) / len(sel)
        assert abs(Fraction(float(c[0, j])) - mean) <= abs(mean) * Fraction(1, 2 ** 50)


def test_lut2_initial_centroids_are_quantiles():
    w = np.arange(64, dtype=np.float32)[None, ::-1].copy()
    c = lut2.initial_centroids(w)
    assert np.array_equal(c[0], [8.0, 24.0, 40.0, 56.0])   # floor((2j+1) 64 / 8)


def test_lut2_index_packing_order():
    w = np.array([[0.0, 1.0, 2.0, 3.0] * 2], dtype=np.float32)
    idx, cb = lut2.fit(w)
    assert np.array_equal(F.bf16_bits_to_f32(cb)[0], [0, 1, 2, 3])
    assert idx[0, 0] == (0 | 1 << 2 | 2 << 4 | 3 << 6)


def test_lut2_zero_centroid_is_positive_zero():
    # a quantile that lands on -0.0 and a cluster that stays empty keep +0
    w = np.array([[-0.0] * 60 + [1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
    c = lut2.initial_centroids(w)
    assert c[0, 0] == 0 and not np.signbit(c[0, 0])
    idx, cb = lut2.fit(w)
    assert not np.any(cb == 0x8000)


def test_lut2_lloyd_matches_scikit_learn_kmeans():
    """The ten Lloyd iterations from the quantile start are scikit-learn's
    KMeans(algorithm="lloyd") from the same initial centroids: one init,
    max_iter=10, tol=0, on the row as one-dimensional data.  Rows are drawn
    from continuous distributions (no exact ties) and checked to keep every
    cluster populated, since scikit-learn relocates an empty cluster where
    this reading keeps its centroid (that rule is pinned separately)."""
    import warnings
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(35)
    rows = []
    for k in (64, 128, 512, 3840):
        rows.append(rng.standard_normal(k) / np.sqrt(k))                    # the weight recipe
        rows.append(rng.standard_t(3, k))                                    # heavy tails
        rows.append(np.concatenate([rng.normal(-1, 0.3, k // 2),
                                    rng.normal(2, 0.1, k - k // 2)]))       # two modes
        rows.append(rng.exponential(1.0, k))                                 # one-sided
    checked = 0
    for row in rows:
        w = row.astype(np.float32)[None, :]
        c_or, _ = lut2.lloyd(w)
        init = lut2.initial_centroids(w)[0]
        x = w[0].astype(np.float64)[:, None]
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            km = KMeans(n_clusters=4, init=init[:, None], n_init=1, max_iter=10, tol=0.0,
                        algorithm="lloyd").fit(x)
        if np.bincount(km.labels_, minlength=4).min() == 0:
            continue
        assert np.allclose(c_or[0], km.cluster_centers_[:, 0], rtol=1e-12, atol=1e-15), row[:4]
        checked += 1
    assert checked >= len(rows) - 2

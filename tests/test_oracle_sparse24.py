"""Pins for oracle.sparse24 (2:4 magnitude pruning along k on top of INT4 g128).

The pruning rule is pinned by an independent characterisation checked by brute
force: of the six column pairs of a quad, the kept pair maximises |a| + |b|,
and among maximal pairs it is the lexicographically smallest.  The product is
pinned by a closed form on constant quads.
"""

import itertools

import numpy as np

from oracle import int4, sparse24, gemm, formats as F


def _brute_keep(v):
    v = np.abs(np.asarray(v, dtype=np.float64))
    n, k = v.shape
    out = np.zeros((n, k), dtype=bool)
    for r in range(n):
        for j in range(k // 4):
            quad = v[r, 4 * j:4 * j + 4]
            best = max(itertools.combinations(range(4), 2),
                       key=lambda p: (quad[p[0]] + quad[p[1]], -p[0], -p[1]))
            out[r, 4 * j + best[0]] = out[r, 4 * j + best[1]] = True
    return out


def test_keep_mask_brute_force_with_ties():
    rng = np.random.default_rng(41)
    # small integers: many equal magnitudes, signs, zeros
    v = rng.integers(-3, 4, (24, 64)).astype(np.float32)
    assert np.array_equal(sparse24.keep_mask(v), _brute_keep(v))
    w = rng.standard_normal((8, 128)).astype(np.float32)
    assert np.array_equal(sparse24.keep_mask(w), _brute_keep(w))


def test_keep_mask_examples():
    m = sparse24.keep_mask(np.array([[3, 1, 2, 2, 0, 0, 0, 0, -5, 5, 1, -6]], dtype=np.float32))
    assert m.tolist() == [[True, False, True, False, True, True, False, False,
                           True, False, False, True]]


def test_quantize_invariants():
    rng = np.random.default_rng(42)
    n, k = 16, 512
    w = (rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    codes, scales = sparse24.quantize(w)
    q = int4.unpack(codes)
    nz = (q != 0).reshape(n, k // 4, 4).sum(axis=2)
    assert nz.max() <= 2
    keep = sparse24.keep_mask(w)
    assert not np.any((q != 0) & ~keep)
    a = np.abs(w).reshape(n, k // 4, 4)
    kq = keep.reshape(n, k // 4, 4)
    kept_min = np.where(kq, a, np.inf).min(axis=2)
    drop_max = np.where(~kq, a, -np.inf).max(axis=2)
    assert np.all(kept_min >= drop_max)
    # the group scale is the dense one: the largest magnitude is always kept
    _, dense_scales = int4.quantize(w)
    assert np.array_equal(scales, dense_scales)


def test_prune_is_identity_on_two_four_inputs():
    rng = np.random.default_rng(43)
    w = rng.standard_normal((4, 256)).astype(np.float32)
    w = sparse24.prune(w)
    assert np.array_equal(sparse24.prune(w), w)
    codes, _ = sparse24.quantize(w)
    assert np.array_equal(sparse24.keep_codes(codes), codes)


def test_keep_codes_prunes_dense_codes_by_code_magnitude():
    rng = np.random.default_rng(44)
    w = rng.standard_normal((8, 256)).astype(np.float32)
    codes, _ = int4.quantize(w)          # dense: up to four nonzeros per quad
    q = int4.unpack(codes)
    kept = int4.unpack(sparse24.keep_codes(codes))
    assert np.array_equal(kept, np.where(_brute_keep(q), q, 0))


def test_sparse_product_closed_form():
    """Constant quads keep their first two columns: y = c * sum_{k % 4 < 2} x."""
    rng = np.random.default_rng(45)
    k = 256
    c = 7.0 * 2.0 ** -4                  # group scale bf16(c / 7) = 2^-4 exactly, q = 7
    w = np.full((3, k), c, dtype=np.float32)
    w[1] = -c
    w[2, :] = 0.0
    w[2, 0::4] = c                        # quads (c, 0, 0, -c): columns 0 and 3 kept
    w[2, 3::4] = -c
    codes, scales = sparse24.quantize(w)
    xb = F.rn_bf16_bits(rng.standard_normal((5, k)).astype(np.float32))
    x = F.bf16_bits_to_f32(xb).astype(np.float64)
    y = gemm.w4a16_sp24(xb, codes, scales)
    first_two = x[:, (np.arange(k) % 4) < 2].sum(axis=1)
    assert np.array_equal(y[:, 0], c * first_two)
    assert np.array_equal(y[:, 1], -c * first_two)
    assert np.array_equal(y[:, 2], c * (x[:, 0::4].sum(axis=1) - x[:, 3::4].sum(axis=1)))


def test_sparse_product_differs_from_dense_when_pruning_bites():
    rng = np.random.default_rng(46)
    w = rng.standard_normal((4, 128)).astype(np.float32)
    xb = F.rn_bf16_bits(rng.standard_normal((2, 128)).astype(np.float32))
    c, s = int4.quantize(w)
    cs, ss = sparse24.quantize(w)
    assert not np.allclose(gemm.w4a16(xb, c, s), gemm.w4a16_sp24(xb, cs, ss))

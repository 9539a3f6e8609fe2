"""2:4 structured-sparse INT4 weights, 128-element groups (oracle; test infrastructure).

Source: the MARLIN article (abeam.tech).  Section "データの扱い方" (how data is
handled) names, next to the group-size-128 INT4 format, the official
implementation's combination with 2:4 structured sparsity (Sparse-MARLIN);
section "実験と結果" (experiments) asks how far adding 2:4 sparsity extends the
speed-up, and reports Sparse-MARLIN's larger end-to-end gain.  The pages do
not say how the sparsity pattern is chosen.

Readings (the plainest ones):
* Pattern: magnitude pruning along k.  In every run of four consecutive
  columns 4j .. 4j+3 of a row ("quad"), the two entries of largest |w| are
  kept, ties going to the lower column, and the other two become zero.
* The pruned matrix is quantized by the dense INT4 group-128 quantizer
  (int4.quantize), so every pruned entry has q = 0; dequantization and the
  product are those of the dense format.
* A packed 2:4 blob stores, per quad, two codes and their positions.  From
  canonical codes the packer keeps the two codes of largest |q| (ties to the
  lower column): every nonzero code when the codes come from quantize().
  keep_codes() states that rule; the product of a packed blob is the dense
  product of keep_codes(codes).
"""

import numpy as np

from . import int4


def keep_mask(v):
    """Boolean [n, k]: the two entries of largest |v| in each quad of columns.

    Ranking is by (-|v|, column): a stable sort of -|v| within the quad keeps
    lower columns first among equal magnitudes.
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    n, k = a.shape
    if k % 4:
        raise ValueError("k must be a multiple of 4")
    quads = a.reshape(n, k // 4, 4)
    order = np.argsort(-quads, axis=2, kind="stable")
    mask = np.zeros(quads.shape, dtype=bool)
    np.put_along_axis(mask, order[:, :, :2], True, axis=2)
    return mask.reshape(n, k)


def prune(w):
    """Magnitude-pruned fp32 weights: two of every four consecutive entries kept."""
    w = np.asarray(w, dtype=np.float32)
    return np.where(keep_mask(w), w, np.float32(0.0)).astype(np.float32)


def quantize(w):
    """Prune, then INT4 group-128 quantize -> (codes [n, k/2], scales [n, k/128])."""
    return int4.quantize(prune(w))


def keep_codes(codes):
    """Canonical codes with all but the two largest-|q| codes of each quad set to q = 0."""
    q = int4.unpack(codes)
    qk = np.where(keep_mask(q), q, 0)
    u = (qk + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)

"""2-bit per-row codebook (LUT2) weight fit by K-means (oracle; test infrastructure).

Sources:
* Disaggregated Quantization (singularity-lens): the fully disaggregated
  variant decodes with a 2-bit LUT weight format.
* KLLM article (aibr.jp), sections 1 and 3: K-means (non-uniform)
  quantization splits a tensor into floating-point centroids (a codebook) and
  a matrix of indices.

The pages give only "centroids + index matrix".  The reading taken here, one
codebook of 4 bfloat16 centroids per weight row, fitted by 10 Lloyd
iterations in float64:

1. Initialise at quantiles of the row: c_j = sorted(w)[floor((2j+1) K / 8)],
   j = 0..3.
2. Each iteration: assign every weight to argmin_j |w - c_j| (float64
   distances; ties go to the lower j); replace each c_j by the float64 mean of
   its weights, the sum taken one element at a time in ascending column order
   and then divided by the count; a cluster with no weights keeps its c_j.
   A centroid that is exactly zero is taken as +0 (at initialisation and
   after each mean), so the sign of a zero never depends on sort or
   summation order.
3. Round: C_j = bf16(rn32(c_j)).
4. Final assignment against the rounded C_j (ties to the lower j).
5. Storage: indices 4 per byte, column 4b+i in bits 2i..2i+1; centroids as
   bfloat16 bit patterns [n, 4].

In one dimension Lloyd's step keeps the centroids in ascending order, so the
codebook comes out sorted.
"""

import numpy as np

from .formats import rn32, rn_bf16_bits, bf16_bits_to_f32

NCENT = 4
ITERS = 10


def _assign(w, c):
    """argmin_j |w - c_j| with ties to the lower j; w [n, k], c [n, 4] (float64)."""
    best = np.zeros(w.shape, dtype=np.int64)
    best_d = np.abs(w - c[:, 0:1])
    for j in range(1, NCENT):
        d = np.abs(w - c[:, j:j + 1])
        better = d < best_d
        best = np.where(better, j, best)
        best_d = np.where(better, d, best_d)
    return best


def _sequential_sum(v):
    """Sum along axis 1 one element at a time, in ascending column order."""
    if v.shape[1] == 0:
        return np.zeros(v.shape[0])
    # np.cumsum accumulates left to right; its last column is the sequential sum
    return np.cumsum(v, axis=1)[:, -1]


def initial_centroids(w):
    w = np.asarray(w, dtype=np.float32)
    k = w.shape[1]
    srt = np.sort(w, axis=1).astype(np.float64)
    idx = [((2 * j + 1) * k) // 8 for j in range(NCENT)]
    return srt[:, idx] + 0.0          # -0.0 + 0.0 == +0.0


def lloyd(w, iters=ITERS):
    """Steps 1-2.  Returns the float64 centroids [n, 4] and the per-iteration
    objective (sum of squared distances, evaluated before each update)."""
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    c = initial_centroids(w)
    history = []
    for _ in range(iters):
        idx = _assign(w64, c)
        history.append(np.sum((w64 - np.take_along_axis(c, idx, axis=1)) ** 2, axis=1))
        new = c.copy()
        for j in range(NCENT):
            m = idx == j
            cnt = m.sum(axis=1)
            s = _sequential_sum(np.where(m, w64, 0.0))
            new[:, j] = np.where(cnt > 0, s / np.maximum(cnt, 1) + 0.0, c[:, j])
        c = new
    return c, history


def fit(w, iters=ITERS):
    """Fit fp32 weights [n, k] -> (indices uint8 [n, k/4], centroids uint16 bf16 bits [n, 4])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 4:
        raise ValueError("k must be a multiple of 4")
    c, _ = lloyd(w, iters)
    cb = rn_bf16_bits(rn32(c))                                          # step 3
    cv = bf16_bits_to_f32(cb).astype(np.float64)
    idx = _assign(w.astype(np.float64), cv)                             # step 4
    packed = (idx[:, 0::4] | (idx[:, 1::4] << 2) | (idx[:, 2::4] << 4)
              | (idx[:, 3::4] << 6)).astype(np.uint8)
    return packed, cb.astype(np.uint16)


def unpack(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    n, kb = packed.shape
    idx = np.empty((n, kb * 4), dtype=np.int64)
    for i in range(4):
        idx[:, i::4] = (packed >> (2 * i)) & 3
    return idx


def dequantize(packed, centroids):
    """Exact float64 weights C[n, idx[n, k]]."""
    idx = unpack(packed)
    cv = bf16_bits_to_f32(centroids).astype(np.float64)
    return np.take_along_axis(cv, idx, axis=1)

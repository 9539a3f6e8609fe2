"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module draws random numbers and nothing else: it holds none of the
quantization method's arithmetic.  It is the only code the HIP path and the
CPU oracle have in common.

Recipe
------
* Generator: numpy PCG64 seeded with ``[config_id, layer_id, tensor_id, block]``
  where ``block`` indexes 256-row slabs, so any row range can be regenerated
  without drawing the rows before it.
* Activations: float32 N(0, 1), then the config's outliers, then (for bf16
  workloads) one round-to-nearest-even cast to bfloat16 done by torch on the CPU.
  - channel outliers: round(0.01 K) input channels chosen by a seeded
    permutation are multiplied by 10 (whole columns);
  - element outliers: each element independently (probability 0.001) is
    multiplied by 50.
* Weights: float32 N(0, 1/sqrt(K)) (standard deviation 1/sqrt(K)).

The synthetic layers stand in for the Qwen3-8B, 27B-class and Gemma3-12B
layer shapes the pages name; no model weights or datasets are used.
"""

import numpy as np
import torch

ROW_BLOCK = 256

T_ACT, T_WEIGHT, T_DECODE_X, T_OUTLIER = 0, 1, 2, 3


def _rng(config_id, layer_id, tensor_id, block=0):
    return np.random.default_rng([int(config_id), int(layer_id), int(tensor_id), int(block)])


def _normal_rows(config_id, layer_id, tensor_id, rows, cols, row0=0, std=1.0):
    """Rows [row0, row0+rows) of a seeded float32 N(0, std^2) matrix."""
    out = np.empty((rows, cols), dtype=np.float32)
    r = row0
    while r < row0 + rows:
        blk = r // ROW_BLOCK
        b0 = blk * ROW_BLOCK
        g = _rng(config_id, layer_id, tensor_id, blk)
        slab = g.standard_normal((ROW_BLOCK, cols), dtype=np.float32)
        lo = r - b0
        hi = min(ROW_BLOCK, row0 + rows - b0)
        out[r - row0:r - row0 + (hi - lo)] = slab[lo:hi]
        r = b0 + hi
    if std != 1.0:
        out *= np.float32(std)
    return out


def outlier_channels(config_id, layer_id, k):
    n_out = int(round(0.01 * k))
    perm = _rng(config_id, layer_id, T_OUTLIER).permutation(k)
    return np.sort(perm[:n_out])


def _element_mask_rows(config_id, layer_id, rows, cols, row0):
    out = np.empty((rows, cols), dtype=bool)
    r = row0
    while r < row0 + rows:
        blk = r // ROW_BLOCK
        b0 = blk * ROW_BLOCK
        u = _rng(config_id, layer_id, T_OUTLIER, 1 + blk).random((ROW_BLOCK, cols))
        lo = r - b0
        hi = min(ROW_BLOCK, row0 + rows - b0)
        out[r - row0:r - row0 + (hi - lo)] = u[lo:hi] < 0.001
        r = b0 + hi
    return out


def to_bf16_bits(x):
    """Round float32 -> bfloat16 (torch CPU cast, nearest even); returns uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_as_f32(h):
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(config_id, layer_id, m, k, outliers=None, rows=None):
    """Prefill activations as float32 (before any bfloat16 cast).

    outliers: None, "channels" (1% of K-channels x10) or "elements" (0.1% x50).
    rows: optional (row0, row1) to draw only that row range.
    """
    row0, row1 = (0, m) if rows is None else rows
    x = _normal_rows(config_id, layer_id, T_ACT, row1 - row0, k, row0)
    if outliers == "channels":
        x[:, outlier_channels(config_id, layer_id, k)] *= np.float32(10.0)
    elif outliers == "elements":
        mask = _element_mask_rows(config_id, layer_id, row1 - row0, k, row0)
        x[mask] *= np.float32(50.0)
    elif outliers is not None:
        raise ValueError(outliers)
    return x


def activations_bf16(config_id, layer_id, m, k, outliers=None, rows=None):
    """Prefill activations rounded once to bfloat16; returns uint16 bit patterns."""
    return to_bf16_bits(activations(config_id, layer_id, m, k, outliers, rows))


def decode_x_bf16(config_id, layer_id, m, k):
    """Decode activations: the first m rows of one seeded [32, k] N(0,1) draw, bf16 bits."""
    x = _normal_rows(config_id, layer_id, T_DECODE_X, 32, k)
    return to_bf16_bits(x[:m])


def weights(config_id, layer_id, n, k, rows=None):
    """float32 weights [n, k] ~ N(0, 1/sqrt(k)); rows=(r0, r1) draws a row range."""
    row0, row1 = (0, n) if rows is None else rows
    return _normal_rows(config_id, layer_id, T_WEIGHT, row1 - row0, k, row0,
                        std=1.0 / np.sqrt(k))

"""Full-size parity helpers: the oracle and the seeded draws over row chunks,
in parallel host threads (test infrastructure).

Every quantizer of the method works row by row once the tensor scale is
fixed (NVFP4: per 16-group of a row, given s_t; INT4: per 128-group of a row;
LUT2: per row), so calling the oracle on disjoint row ranges with the same
tensor scale and concatenating gives exactly the oracle's whole-tensor result.
The tensor scale itself is always taken by ``nvfp4.tensor_scale`` over the
whole tensor.  Likewise ``synth`` seeds every 256-row block on its own, so
drawing row ranges separately gives the same tensor as one draw.

numpy releases the interpreter lock inside its array loops, so threads give
a real speed-up on the large tensors (hundreds of millions of elements) the
full-size tests check.
"""

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from decode_nvfp4_rtn_amd import synth
from oracle import nvfp4, int4, lut2, sparse24


def workers():
    """Host threads to use: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _ranges(rows, chunk):
    return [(r, min(rows, r + chunk)) for r in range(0, rows, chunk)]


def _chunk_rows(rows, cols, target_elems=1 << 23):
    """Rows per chunk: about target_elems elements, a multiple of the 256-row
    seed block so each draw regenerates every seed block once."""
    c = max(1, target_elems // max(cols, 1))
    return max(synth.ROW_BLOCK, (c // synth.ROW_BLOCK) * synth.ROW_BLOCK)


def pmap(fn, items):
    with ThreadPoolExecutor(max_workers=workers()) as ex:
        return list(ex.map(fn, items))


# ------------------------------------------------------------- draws --

def activations_bf16(config_id, layer_id, m, k, outliers=None):
    """synth.activations_bf16 of [m, k], drawn in row ranges in parallel."""
    out = np.empty((m, k), dtype=np.uint16)

    def one(rr):
        r0, r1 = rr
        out[r0:r1] = synth.activations_bf16(config_id, layer_id, m, k, outliers=outliers,
                                            rows=(r0, r1))
    pmap(one, _ranges(m, _chunk_rows(m, k)))
    return out


def weights(config_id, layer_id, n, k):
    """synth.weights of [n, k], drawn in row ranges in parallel."""
    out = np.empty((n, k), dtype=np.float32)

    def one(rr):
        r0, r1 = rr
        out[r0:r1] = synth.weights(config_id, layer_id, n, k, rows=(r0, r1))
    pmap(one, _ranges(n, _chunk_rows(n, k)))
    return out


def bf16_as_f32(bits):
    """synth.bf16_bits_as_f32 in row ranges (exact widening)."""
    out = np.empty(bits.shape, dtype=np.float32)

    def one(rr):
        r0, r1 = rr
        out[r0:r1] = synth.bf16_bits_as_f32(bits[r0:r1])
    pmap(one, _ranges(bits.shape[0], _chunk_rows(*bits.shape)))
    return out


# ------------------------------------------------------------ oracle --

def nvfp4_quantize(x_f32, s_t, chunk=512):
    """oracle nvfp4.quantize of every row of x with the given tensor scale."""
    rows, cols = x_f32.shape
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 16), dtype=np.uint8)

    def one(rr):
        r0, r1 = rr
        c, s, _ = nvfp4.quantize(x_f32[r0:r1], s_t=s_t)
        codes[r0:r1] = c
        scales[r0:r1] = s
    pmap(one, _ranges(rows, chunk))
    return codes, scales, np.float32(s_t)


def int4_quantize(w, chunk=512):
    n, k = w.shape
    codes = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // 128), dtype=np.uint16)

    def one(rr):
        r0, r1 = rr
        c, s = int4.quantize(w[r0:r1])
        codes[r0:r1] = c
        scales[r0:r1] = s
    pmap(one, _ranges(n, chunk))
    return codes, scales


def sp24_quantize(w, chunk=512):
    """oracle sparse24.quantize (2:4 pruning along k, then INT4) of every row."""
    n, k = w.shape
    codes = np.empty((n, k // 2), dtype=np.uint8)
    scales = np.empty((n, k // 128), dtype=np.uint16)

    def one(rr):
        r0, r1 = rr
        c, s = sparse24.quantize(w[r0:r1])
        codes[r0:r1] = c
        scales[r0:r1] = s
    pmap(one, _ranges(n, chunk))
    return codes, scales


def lut2_fit(w, chunk=128):
    n, k = w.shape
    idx = np.empty((n, k // 4), dtype=np.uint8)
    cent = np.empty((n, 4), dtype=np.uint16)

    def one(rr):
        r0, r1 = rr
        i, c = lut2.fit(w[r0:r1])
        idx[r0:r1] = i
        cent[r0:r1] = c
    pmap(one, _ranges(n, chunk))
    return idx, cent


def first_mismatch(a, b, chunk_rows=4096):
    """None when a and b are equal; else the first differing [row, col]."""
    for r0 in range(0, a.shape[0], chunk_rows):
        d = a[r0:r0 + chunk_rows] != b[r0:r0 + chunk_rows]
        if d.any():
            rr, cc = np.argwhere(d)[0]
            return int(r0 + rr), int(cc)
    return None


# ------------------------------------------- cached decode layer weights --
# The decode GEMV tests and the weight-quantizer tests of one process share
# the oracle's quantization of the full-size layers.

def _frozen(*arrays):
    for a in arrays:
        a.flags.writeable = False
    return arrays


@functools.lru_cache(maxsize=4)
def int4_layer(config_id, layer_id, n, k):
    """(w fp32 [n, k], oracle INT4 codes, scales) of a seeded decode layer."""
    w = weights(config_id, layer_id, n, k)
    return _frozen(w, *int4_quantize(w))


@functools.lru_cache(maxsize=3)
def lut2_layer(config_id, layer_id, n, k):
    """(w fp32 [n, k], oracle LUT2 indices, centroids) of a seeded decode layer."""
    w = weights(config_id, layer_id, n, k)
    return _frozen(w, *lut2_fit(w))

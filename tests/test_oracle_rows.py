"""The row-chunked, threaded helpers of the full-size GPU tests give exactly
what one whole-tensor call of the oracle (or of synth) gives."""

import numpy as np

from decode_nvfp4_rtn_amd import synth
from oracle import nvfp4, int4, lut2, sparse24
from tests import oracle_rows as orows


def test_chunked_draws_equal_whole_draws():
    # 700 rows: chunks that end inside a 256-row seed block, and a ragged last one
    a = orows.activations_bf16(4, 1, 700, 96, outliers="elements")
    assert np.array_equal(a, synth.activations_bf16(4, 1, 700, 96, outliers="elements"))
    a = orows.activations_bf16(2, 3, 513, 64, outliers="channels")
    assert np.array_equal(a, synth.activations_bf16(2, 3, 513, 64, outliers="channels"))
    w = orows.weights(4, 2, 300, 128)
    assert np.array_equal(w, synth.weights(4, 2, 300, 128))
    assert np.array_equal(orows.bf16_as_f32(a), synth.bf16_bits_as_f32(a))


def test_chunked_oracle_equals_whole_oracle():
    x = synth.bf16_bits_as_f32(synth.activations_bf16(4, 0, 1100, 160, outliers="elements"))
    st = nvfp4.tensor_scale(x)
    c, s, t = orows.nvfp4_quantize(x, st, chunk=96)
    rc, rs, rt = nvfp4.quantize(x)
    assert t == rt and np.array_equal(c, rc) and np.array_equal(s, rs)
    w = synth.weights(3, 0, 530, 256)
    c, s = orows.int4_quantize(w, chunk=64)
    rc, rs = int4.quantize(w)
    assert np.array_equal(c, rc) and np.array_equal(s, rs)
    c, s = orows.sp24_quantize(w, chunk=100)
    rc, rs = sparse24.quantize(w)
    assert np.array_equal(c, rc) and np.array_equal(s, rs)
    w = synth.weights(5, 0, 70, 384)
    i, cb = orows.lut2_fit(w, chunk=16)
    ri, rcb = lut2.fit(w)
    assert np.array_equal(i, ri) and np.array_equal(cb, rcb)


def test_first_mismatch():
    a = np.zeros((10, 4), dtype=np.uint8)
    b = a.copy()
    assert orows.first_mismatch(a, b, chunk_rows=3) is None
    b[7, 2] = 1
    assert orows.first_mismatch(a, b, chunk_rows=3) == (7, 2)

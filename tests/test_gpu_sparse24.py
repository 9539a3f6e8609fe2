"""GPU parity of the 2:4 sparse INT4 path against oracle.sparse24.

* quantize_int4_g128_sp24: codes and scales bit-exact (every row).
* repack (QL_INT4_SP24) + gemm_w4a16_sp24: fp32 outputs within 1e-3 of the
  output RMS of the oracle's fp64 product, bf16 outputs by the bf16 rule; every
  Qwen3-8B-like decode shape and batch (also through the workspace entry
  point, as the benchmark calls it), ragged shapes through both kernels
  (persistent and k-split) and through the k split over blocks, and dense
  (unpruned) codes, which the packer prunes by |q|.
"""

import numpy as np
import pytest
import torch

from decode_nvfp4_rtn_amd import synth, configs
from oracle import int4, sparse24, gemm
from tests import oracle_rows as orows
from tests.gpu_common import (require_gpu, say, dev_f32, dev_bf16, host_f64, host_u8, host_u16,
                              sample_rows)

pytestmark = pytest.mark.gpu
TOL = gemm.TOL


def _sp24_blob(q, w):
    c, s = q.quantize_int4_g128(dev_f32(w), sparse24=True)
    n, k = w.shape
    return q.repack_weights(q.QL_INT4_SP24, n, k, c, s), c, s


def _check(y_gpu, y_ref, bf16):
    if bf16:
        assert gemm.bf16_output_ok(y_gpu, y_ref), gemm.normalized_max_error(y_gpu, y_ref)
    else:
        e = gemm.normalized_max_error(y_gpu, y_ref)
        assert e <= TOL, e


@pytest.mark.parametrize("n,k,cfg", [(256, 512, 1), (6144, 4096, 3), (4096, 12288, 3)])
def test_sp24_quantizer_bitexact(n, k, cfg):
    q = require_gpu()
    w = synth.weights(cfg, 1, n, k)
    w[:, 8:12] = np.float32(0.25)          # an all-equal quad: ties go to the lower columns
    w[:, 12:16] = np.float32([0.0, -0.5, 0.5, -0.0])
    say("sp24 quantize", n, k)
    codes, scales = q.quantize_int4_g128(dev_f32(w), sparse24=True)
    torch.cuda.synchronize()
    rc, rs = orows.sp24_quantize(w)
    gs, gc = host_u16(scales), host_u8(codes)
    assert orows.first_mismatch(gs, rs) is None, f"scales differ at {orows.first_mismatch(gs, rs)}"
    assert orows.first_mismatch(gc, rc) is None, f"codes differ at {orows.first_mismatch(gc, rc)}"


def test_sp24_tiny_decode_and_layout_probe():
    q = require_gpu()
    n, k = 256, 512
    w = synth.weights(1, 0, n, k)
    xb = synth.decode_x_bf16(1, 0, 1, k)
    say("sp24 tiny")
    blob, c, s = _sp24_blob(q, w)
    y = q.gemm_w4a16_sp24(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rc, rs = sparse24.quantize(w)
    _check(host_f64(y), gemm.w4a16_sp24(xb, rc, rs), False)
    # one-hot activations read single weight columns back exactly
    ks = [0, 1, 2, 3, 7, 8, 15, 16, 31, 63, 64, 100, 127, 128, 300, 511]
    x = np.zeros((len(ks), k), dtype=np.float32)
    for i, kk in enumerate(ks):
        x[i, kk] = 1.0
    y = host_f64(q.gemm_w4a16_sp24(dev_bf16(synth.to_bf16_bits(x)), blob, n, k,
                                   out_dtype=torch.float32))
    torch.cuda.synchronize()
    wh = int4.dequantize(rc, rs)
    for i, kk in enumerate(ks):
        assert np.array_equal(y[i], wh[:, kk].astype(np.float32)), kk


@pytest.mark.parametrize("li", range(4))
def test_sp24_qwen3_decode_all_batches(li):
    q = require_gpu()
    cfg = configs.QWEN3_DECODE
    layer = cfg.layers[li]
    n, k = layer.n, layer.k
    w = orows.int4_layer(cfg.cid, li, n, k)[0]
    say("sp24", layer.name, n, k)
    blob, _, _ = _sp24_blob(q, w)
    rc, rs = orows.sp24_quantize(w)
    for m in cfg.ms:
        xb = synth.decode_x_bf16(cfg.cid, li, m, k)
        y16 = q.gemm_w4a16_sp24(dev_bf16(xb), blob, n, k, out_dtype=torch.bfloat16)
        y32 = q.gemm_w4a16_sp24(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref = gemm.w4a16_sp24(xb, rc, rs)
        _check(host_f64(y32), ref, False)
        _check(host_f64(y16), ref, True)
        # the workspace entry point, as the benchmark calls it (k split over
        # blocks where the shape has one)
        nb = q.gemm_w4a16_sp24_workspace(m, n, k)
        if nb:
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            y16 = q.gemm_w4a16_sp24(dev_bf16(xb), blob, n, k, out_dtype=torch.bfloat16,
                                    workspace=ws)
            torch.cuda.synchronize()
            _check(host_f64(y16), ref, True)


@pytest.mark.parametrize("n,k", [(16 * 1031, 3840), (16 * 1537, 2048), (272, 8320), (272, 12288),
                                 (6160, 1152)])
def test_sp24_ragged_shapes_both_kernels(n, k):
    q = require_gpu()
    w = synth.weights(11, 3, n, k)
    say("sp24 ragged", n, k)
    blob, _, _ = _sp24_blob(q, w)
    cols = sample_rows(n, 256, n + k)
    rc, rs = sparse24.quantize(w[cols])
    for m in (1, 7, 16, 25, 40):
        xb = synth.activations_bf16(11, 4, m, k)
        y = q.gemm_w4a16_sp24(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check(host_f64(y)[:, cols], gemm.w4a16_sp24(xb, rc, rs), False)


# The workspace entry point splits k over blocks (S slices of 8 GW groups, P
# tile walkers per slice): a last slice with fewer groups than the others, a
# last slice of one group, tile counts that leave walkers a tile short, one
# and two m-tiles, and every Qwen3-8B-like layer with long k.

@pytest.mark.parametrize("n,k", [(4096, 12288), (272, 8320), (16 * 257, 9088), (6160, 4224),
                                 (16 * 1031, 8192), (12288, 4608)])
def test_sp24_split_ragged(n, k):
    q = require_gpu()
    w = synth.weights(17, k, n, k)
    say("sp24 split", n, k)
    blob, _, _ = _sp24_blob(q, w)
    rc, rs = orows.sp24_quantize(w)
    del w
    ms = (9, 13, 16, 17, 25, 32)
    xs = [synth.activations_bf16(17, m, m, k) for m in ms]
    refs = np.split(gemm.w4a16_sp24(np.concatenate(xs), rc, rs), np.cumsum(ms)[:-1])
    for m, xb, ref in zip(ms, xs, refs):
        nb = q.gemm_w4a16_sp24_workspace(m, n, k)
        assert nb > 0, (m, n, k)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        x = dev_bf16(xb)
        y32 = q.gemm_w4a16_sp24(x, blob, n, k, out_dtype=torch.float32, workspace=ws)
        y16 = q.gemm_w4a16_sp24(x, blob, n, k, out_dtype=torch.bfloat16, workspace=ws)
        y16b = q.gemm_w4a16_sp24(x, blob, n, k, out_dtype=torch.bfloat16, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y16, y16b)
        _check(host_f64(y32), ref, False)
        _check(host_f64(y16), ref, True)


def test_sp24_repack_prunes_dense_codes_by_magnitude():
    q = require_gpu()
    n, k = 64, 1024
    w = synth.weights(12, 0, n, k)
    say("sp24 repack of dense codes")
    c, s = q.quantize_int4_g128(dev_f32(w))          # dense: up to four nonzeros per quad
    blob = q.repack_weights(q.QL_INT4_SP24, n, k, c, s)
    xb = synth.decode_x_bf16(12, 0, 5, k)
    y = q.gemm_w4a16_sp24(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rc, rs = int4.quantize(w)
    _check(host_f64(y), gemm.w4a16_sp24(xb, rc, rs), False)


def test_sp24_deterministic_and_empty():
    q = require_gpu()
    n, k = 6144, 4096
    w = synth.weights(3, 0, n, k)
    blob, _, _ = _sp24_blob(q, w)
    xb = dev_bf16(synth.decode_x_bf16(3, 0, 16, k))
    say("sp24 determinism")
    a = q.gemm_w4a16_sp24(xb, blob, n, k)
    b = q.gemm_w4a16_sp24(xb, blob, n, k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    y0 = q.gemm_w4a16_sp24(xb[:0], blob, n, k)
    assert y0.numel() == 0

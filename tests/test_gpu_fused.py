"""GPU parity of quantize_gemm_w4a4 (NVFP4 quantize folded into the W4A4
GEMM's activation load).

* Against the two-call path on the same inputs: quantize_nvfp4 on bf16 X,
  then gemm_w4a4 without a workspace.  Where gemm_w4a4 runs the kernel whose
  quantizing variant this call runs -- the small-batch kernel (m <= 32) or
  the 128-row-tile kernel (m <= 128, or few 256 x 256 tiles) -- the outputs
  and the tensor scale must be bit-identical; its 256 x 256 kernel
  accumulates each MFMA over another k order, so there only the tensor scale
  is compared exactly.
* Against the oracle (its own quantization of X and W, fp64 product): the
  fp32 and bf16 output bars of the other W4A4 tests, and the tensor scale
  bit for bit.
* A static tensor scale (one launch), ragged m (rows past m in a 64- or
  128-row tile, a wavefront whose rows all lie past m), both tile sizes, and
  a wrong blob, which leaves y and the tensor scale untouched; the static
  scale and the wrong blob through the small-batch kernel as well.
"""

import numpy as np
import pytest
import torch

from decode_nvfp4_rtn_amd import synth, configs
from oracle import nvfp4, gemm
from tests import oracle_rows as orows
from tests.gpu_common import require_gpu, say, dev_f32, dev_bf16, host_f64, rows_f64, sample_rows

pytestmark = pytest.mark.gpu
TOL = gemm.TOL


def _nvfp4_blob(q, w):
    wc, ws, wt = q.quantize_nvfp4(dev_f32(w))
    n, k = w.shape
    return q.repack_weights(q.QL_NVFP4, n, k, wc, ws, wt)


def _check(y_gpu, y_ref, bf16):
    if bf16:
        assert gemm.bf16_output_ok(y_gpu, y_ref), gemm.normalized_max_error(y_gpu, y_ref)
    else:
        e = gemm.normalized_max_error(y_gpu, y_ref)
        assert e <= TOL, e


def _two_calls(q, x, blob, n, dt, ts=None):
    ac, as_, at = q.quantize_nvfp4(x, tensor_scale=ts)
    m, k = x.shape
    return q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=dt), at


def _same_kernel(m, n):
    """gemm_w4a4 (no workspace) runs, on this shape, the kernel whose
    quantizing variant quantize_gemm_w4a4 runs: the small-batch kernel
    (m <= 32) or the 128-row-tile kernel (m <= 128, or few 256 x 256 tiles)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    big = ((m + 255) // 256) * ((n + 255) // 256)
    return m <= 128 or 2 * big <= cus


# m: one token, two m-tiles of the small-batch kernel, a partial first
# wavefront, ragged 64- and 128-row tiles; n: one and two row tiles per
# small-batch block, 64 x 64 tiles (fewer 128 x 128 tiles than CUs) and
# 128 x 128 tiles
@pytest.mark.parametrize("m,n,k", [(1, 256, 512), (3, 4096, 1024), (16, 6144, 4096),
                                   (29, 6160, 12288), (32, 272, 640),
                                   (61, 272, 640), (100, 12288, 1024), (128, 4096, 4096),
                                   (300, 4096, 1024), (1000, 4112, 640), (2048, 6144, 1024)])
def test_fused_matches_two_calls_and_oracle(m, n, k):
    q = require_gpu()
    bits = synth.activations_bf16(21, m, m, k, outliers="channels")
    w = synth.weights(21, n, n, k)
    say("quantize_gemm_w4a4", m, n, k)
    blob = _nvfp4_blob(q, w)
    x = dev_bf16(bits)
    for dt in (torch.float32, torch.bfloat16):
        y, ts = q.quantize_gemm_w4a4(x, blob, n, out_dtype=dt)
        y2, ts2 = _two_calls(q, x, blob, n, dt)
        torch.cuda.synchronize()
        assert torch.equal(ts, ts2)
        if _same_kernel(m, n):
            assert torch.equal(y, y2), dt
        rows = sample_rows(m, 256, m + n)
        xf = orows.bf16_as_f32(bits)
        st = nvfp4.tensor_scale(xf)
        assert np.float32(ts.item()) == st
        ref = gemm.w4a4(*nvfp4.quantize(xf[rows], s_t=st), *nvfp4.quantize(w))
        _check(rows_f64(y, rows), ref, dt == torch.bfloat16)


@pytest.mark.parametrize("m", [77, 20])
def test_fused_static_scale(m):
    """A calibrated tensor scale (QL_STATIC_SCALE): one launch, read not
    written; the per-wave kernel (m = 77) and the small-batch kernel (m = 20)."""
    q = require_gpu()
    n, k = 4096, 2048
    bits = synth.activations_bf16(22, 0, m, k, outliers="channels")
    w = synth.weights(22, 1, n, k)
    blob = _nvfp4_blob(q, w)
    x = dev_bf16(bits)
    xf = orows.bf16_as_f32(bits)
    say("quantize_gemm_w4a4 static scale", m)
    # a scale below the data's (codes saturate at 6 x 448) and one above it
    for st in (np.float32(nvfp4.tensor_scale(xf) * np.float32(0.37)),
               np.float32(nvfp4.tensor_scale(xf) * np.float32(3.0))):
        ts = torch.tensor([st], dtype=torch.float32, device="cuda")
        y, ts_back = q.quantize_gemm_w4a4(x, blob, n, tensor_scale=ts)
        y2, _ = _two_calls(q, x, blob, n, torch.float32, ts=ts)
        torch.cuda.synchronize()
        assert ts_back.item() == st
        assert torch.equal(y, y2)
        ref = gemm.w4a4(*nvfp4.quantize(xf, s_t=st), *nvfp4.quantize(w))
        _check(host_f64(y), ref, False)


@pytest.mark.parametrize("li", range(4))
def test_fused_qwen3_layers_small_batches(li):
    """Every Qwen3-8B-like prefill layer at the batch sizes the benchmark
    times for this call, against the two-call path (bit-identical) and the
    oracle on sampled rows."""
    q = require_gpu()
    cfg = configs.QWEN3_PREFILL
    L = cfg.layers[li]
    n, k = L.n, L.k
    w = orows.weights(cfg.cid, li, n, k)
    wq = orows.nvfp4_quantize(w, nvfp4.tensor_scale(w))
    blob = _nvfp4_blob(q, w)
    del w
    for m in (16, 64, 128, 512):
        bits = orows.activations_bf16(cfg.cid, li, m, k, outliers=cfg.outliers)
        say("quantize_gemm_w4a4", L.name, m, n, k)
        x = dev_bf16(bits)
        y, ts = q.quantize_gemm_w4a4(x, blob, n, out_dtype=torch.bfloat16)
        y2, ts2 = _two_calls(q, x, blob, n, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(ts, ts2)
        if _same_kernel(m, n):
            assert torch.equal(y, y2)
        rows = sample_rows(m, 64, 3 * m + li)
        xf = orows.bf16_as_f32(bits)
        st = nvfp4.tensor_scale(xf)
        ref = gemm.w4a4(*nvfp4.quantize(xf[rows], s_t=st), *wq)
        _check(rows_f64(y, rows), ref, True)


@pytest.mark.parametrize("m", [40, 12])
def test_fused_blob_guard_and_empty(m):
    """A wrong blob leaves y and the tensor scale untouched (per-wave kernel
    at m = 40, small-batch kernel at m = 12); m = 0 is a no-op."""
    q = require_gpu()
    n, k = 256, 512
    w = synth.weights(23, 0, n, k)
    c4, s4 = q.quantize_int4_g128(dev_f32(w))
    i4 = q.repack_weights(q.QL_INT4_G128, n, k, c4, s4)
    right = _nvfp4_blob(q, w)
    wrong = torch.zeros_like(right)
    wrong[: min(i4.numel(), wrong.numel())] = i4[: min(i4.numel(), wrong.numel())]
    x = dev_bf16(synth.activations_bf16(23, 1, m, k))
    say("quantize_gemm_w4a4 blob guard", m)
    y = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
    ts = torch.full((1,), 5.0, dtype=torch.float32, device="cuda")
    q.quantize_gemm_w4a4(x, wrong, n, y=y, ts_out=ts)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and ts.item() == 5.0
    q.quantize_gemm_w4a4(x, right, n, y=y, ts_out=ts)
    torch.cuda.synchronize()
    assert not torch.any(y == 7.0) and ts.item() != 5.0
    y0, _ = q.quantize_gemm_w4a4(x[:0], right, n)
    assert y0.numel() == 0

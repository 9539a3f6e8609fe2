"""GPU parity of the three GEMMs against the oracle's fp64 products.

Bar: max |y - y_ref| / rms(y_ref) <= 1e-3 for fp32 outputs; for bf16 outputs
the per-element rule of oracle.gemm.bf16_output_ok.  The oracle quantizes its
own operands from the same seeded inputs (bit-equality of those codes with the
GPU's is checked in test_gpu_quantize.py).  At full size it computes 1024
seeded rows (always including the last) times every column of each W4A4
output, and every output of the decode GEMMs, in the launch configuration
the benchmark times (the same inputs, and the k-split workspace wherever the
benchmark passes one).
"""

import numpy as np
import pytest
import torch

from decode_nvfp4_rtn_amd import synth, configs
from oracle import nvfp4, int4, lut2, gemm
from tests import oracle_rows as orows
from tests.gpu_common import (require_gpu, say, dev_f32, dev_bf16, host_f64, host_u8, rows_f64,
                              sample_rows)

pytestmark = pytest.mark.gpu
TOL = gemm.TOL


# ------------------------------------------------------------- helpers --

def _nvfp4_blob(q, w):
    wc, ws, wt = q.quantize_nvfp4(dev_f32(w))
    n, k = w.shape
    return q.repack_weights(q.QL_NVFP4, n, k, wc, ws, wt)


def _int4_blob(q, w):
    c, s = q.quantize_int4_g128(dev_f32(w))
    n, k = w.shape
    return q.repack_weights(q.QL_INT4_G128, n, k, c, s)


def _lut2_blob(q, w):
    i, c = q.fit_lut2(dev_f32(w))
    n, k = w.shape
    return q.repack_weights(q.QL_LUT2, n, k, i, c)


def _check(y_gpu, y_ref, bf16):
    if bf16:
        assert gemm.bf16_output_ok(y_gpu, y_ref), gemm.normalized_max_error(y_gpu, y_ref)
    else:
        e = gemm.normalized_max_error(y_gpu, y_ref)
        assert e <= TOL, e


# ---------------------------------------------------------------- W4A4 --

def test_w4a4_tiny_full():
    q = require_gpu()
    x = synth.activations(1, 0, 64, 512, outliers="channels")
    w = synth.weights(1, 0, 256, 512)
    say("w4a4 tiny 64x256x512")
    blob = _nvfp4_blob(q, w)
    ac, as_, at = q.quantize_nvfp4(dev_f32(x))
    y = q.gemm_w4a4(ac, as_, at, blob, 64, 256, 512, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = gemm.w4a4(*nvfp4.quantize(x), *nvfp4.quantize(w))
    _check(host_f64(y), ref, False)


# Small problems without a workspace take the per-wave kernel: 64 x 64 tiles
# while there are fewer 128 x 128 tiles than CUs, 128 x 128 tiles above that
# (1000 x 4112: 264 of them, ragged in M and N).  So does M <= 128 at any N
# (96 x 40976: 161 tiles of 256 x 256, ragged N).
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (5, 48, 256), (130, 272, 384), (257, 128, 1024),
                                   (1000, 4112, 640), (96, 40976, 256)])
def test_w4a4_ragged(m, n, k):
    q = require_gpu()
    x = synth.activations(8, m, m, k, outliers="channels")
    w = synth.weights(8, n, n, k)
    say("w4a4 ragged", m, n, k)
    blob = _nvfp4_blob(q, w)
    ac, as_, at = q.quantize_nvfp4(dev_f32(x))
    ys = {}
    for dt in (torch.float32, torch.bfloat16):
        y = ys[dt] = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=dt)
        torch.cuda.synchronize()
        ref = gemm.w4a4(*nvfp4.quantize(x), *nvfp4.quantize(w))
        _check(host_f64(y), ref, dt == torch.bfloat16)
    # the bf16 epilogue (tiles staged through LDS, stored as whole rows) puts
    # every element where the fp32 one does: the whole bf16 output is the
    # round-to-nearest-even of the same kernel's fp32 output
    assert torch.equal(ys[torch.bfloat16], ys[torch.float32].to(torch.bfloat16))


# Batches of up to 32 tokens take the small-batch kernel (waves split k, one
# or two 16-row tiles and one or two m-tiles per block): one and two m-tiles
# with ragged rows, one row tile per block and two (N >= 6144, odd tile
# count), k from one step (idle waves) to several chunks per wave, both
# output dtypes; and the workspace call, which never splits these batches.
@pytest.mark.parametrize("n,k", [(256, 128), (4112, 640), (6160, 4096), (272, 12288),
                                 (6144, 4224)])
def test_w4a4_small_batches(n, k):
    q = require_gpu()
    w = synth.weights(19, n, n, k)
    say("w4a4 small batches", n, k)
    blob = _nvfp4_blob(q, w)
    wq = nvfp4.quantize(w)
    del w
    for m in (1, 7, 16, 17, 31, 32):
        x = synth.activations(19, m, m, k, outliers="channels")
        ac, as_, at = q.quantize_nvfp4(dev_f32(x))
        assert q.gemm_w4a4_workspace(m, n, k) == 0
        y32 = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.float32)
        y16 = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        ref = gemm.w4a4(*nvfp4.quantize(x), *wq)
        _check(host_f64(y32), ref, False)
        _check(host_f64(y16), ref, True)


# One prefill layer at a time: the oracle's quantization of its weights (every
# row), its GPU blob, and the activations at the largest M of the case list
# (smaller M are their first rows, as the seeded draw is by 256-row block).
_LAYER = {}


def _prefill_layer(q, cfg, li, m_max):
    key = (cfg.cid, li)
    if key not in _LAYER:
        _LAYER.clear()
        L = cfg.layers[li]
        w = orows.weights(cfg.cid, li, L.n, L.k)
        wq = orows.nvfp4_quantize(w, nvfp4.tensor_scale(w))
        blob = _nvfp4_blob(q, w)
        del w
        bits = orows.activations_bf16(cfg.cid, li, m_max, L.k, outliers=cfg.outliers)
        _LAYER[key] = dict(wq=wq, blob=blob, bits=bits)
    return _LAYER[key]


def _w4a4_full_size(q, cfg, li, m, m_max):
    """quantize_nvfp4 + gemm_w4a4 on the benchmark's input of this layer and M
    (with a k-split workspace when the shape has one, as the benchmark does);
    1024 seeded rows x every column against the oracle."""
    L = cfg.layers[li]
    n, k = L.n, L.k
    c = _prefill_layer(q, cfg, li, m_max)
    bits = c["bits"][:m]
    nb = q.gemm_w4a4_workspace(m, n, k)
    say("w4a4 full", cfg.name, L.name, m, n, k, "workspace", nb)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
    ac, as_, at = q.quantize_nvfp4(dev_bf16(bits))
    y32 = q.gemm_w4a4(ac, as_, at, c["blob"], m, n, k, out_dtype=torch.float32, workspace=ws)
    y16 = q.gemm_w4a4(ac, as_, at, c["blob"], m, n, k, out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    rows = sample_rows(m, 1024, 7 * m + n)
    g32, g16 = rows_f64(y32, rows), rows_f64(y16, rows)
    gcodes = host_u8(ac.index_select(0, torch.from_numpy(rows).cuda()))
    del y32, y16, ac, as_, ws
    xf = orows.bf16_as_f32(bits)
    st_a = nvfp4.tensor_scale(xf)
    assert np.float32(at.item()) == st_a
    aq = nvfp4.quantize(xf[rows], s_t=st_a)
    assert np.array_equal(gcodes, aq[0])
    ref = gemm.w4a4(*aq, *c["wq"])
    _check(g32, ref, False)
    _check(g16, ref, True)


@pytest.mark.parametrize("li", range(4))
def test_w4a4_qwen3_prefill_full_size(li):
    q = require_gpu()
    _w4a4_full_size(q, configs.QWEN3_PREFILL, li, 8192, 8192)


# All twelve (layer, M) cases of the 27B-class set, layer by layer.
@pytest.mark.parametrize("li,m", [(li, m) for li in range(4) for m in (4096, 16384, 32768)])
def test_w4a4_27b_prefill_full_size(li, m):
    q = require_gpu()
    cfg = configs.BIG27_PREFILL
    _w4a4_full_size(q, cfg, li, m, max(cfg.ms))


def test_w4a4_one_hot_layout_probe():
    """One-hot NVFP4 activations extract dequantized weight columns exactly."""
    q = require_gpu()
    n, k = 64, 256
    w = synth.weights(7, 0, n, k)
    blob = _nvfp4_blob(q, w)
    ks = [0, 1, 15, 16, 31, 63, 100, 127, 128, 255]
    x = np.zeros((len(ks), k), dtype=np.float32)
    for i, kk in enumerate(ks):
        x[i, kk] = 6.0
    say("w4a4 one-hot probe")
    ac, as_, at = q.quantize_nvfp4(dev_f32(x))
    y = host_f64(q.gemm_w4a4(ac, as_, at, blob, len(ks), n, k, out_dtype=torch.float32))
    torch.cuda.synchronize()
    wh = nvfp4.dequantize(*nvfp4.quantize(w))
    xh = nvfp4.dequantize(*nvfp4.quantize(x))
    for i, kk in enumerate(ks):
        # one exact product, then the fp32 epilogue scale (s_tA * s_tW rounded once)
        ref = xh[i, kk] * wh[:, kk]
        assert np.all(np.abs(y[i] - ref) <= 4 * 2.0 ** -24 * np.abs(ref)), kk
        assert np.array_equal(y[i] == 0, ref == 0)


def test_w4a4_deterministic_and_empty():
    q = require_gpu()
    m, n, k = 1024, 2048, 1024
    bits = synth.activations_bf16(2, 9, m, k, outliers="channels")
    w = synth.weights(2, 9, n, k)
    say("w4a4 determinism")
    blob = _nvfp4_blob(q, w)
    ac, as_, at = q.quantize_nvfp4(dev_bf16(bits))
    a = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.bfloat16)
    b = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    y0 = q.gemm_w4a4(ac, as_, at, blob, 0, n, k, y=torch.empty((0, n), device="cuda"))
    assert y0.numel() == 0


# --------------------------------------------------------------- W4A16 --

def _check_decode_ws(fn, ws_fn, xb, blob, n, k, ref, need_split=False):
    """The workspace entry point (k split over blocks where the shape has
    one) against the oracle, fp32 and bf16 outputs, twice with the same
    workspace (deterministic)."""
    m = xb.shape[0]
    nb = ws_fn(m, n, k)
    if need_split:
        assert nb > 0, (m, n, k)
    if nb == 0:
        return
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    x = dev_bf16(xb)
    y32 = fn(x, blob, n, k, out_dtype=torch.float32, workspace=ws)
    y16 = fn(x, blob, n, k, out_dtype=torch.bfloat16, workspace=ws)
    y16b = fn(x, blob, n, k, out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y16, y16b)
    _check(host_f64(y32), ref, False)
    _check(host_f64(y16), ref, True)


def test_w4a16_tiny_decode():
    q = require_gpu()
    w = synth.weights(1, 0, 256, 512)
    xb = synth.decode_x_bf16(1, 0, 1, 512)
    say("w4a16 tiny")
    blob = _int4_blob(q, w)
    y = q.gemm_w4a16(dev_bf16(xb), blob, 256, 512, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = gemm.w4a16(xb, *int4.quantize(w))
    _check(host_f64(y), ref, False)


@pytest.mark.parametrize("li", range(4))
def test_w4a16_qwen3_decode_all_batches(li):
    """Every output of every Qwen3-8B-like decode layer at every batch size."""
    q = require_gpu()
    cfg = configs.QWEN3_DECODE
    layer = cfg.layers[li]
    n, k = layer.n, layer.k
    w, rc, rs = orows.int4_layer(cfg.cid, li, n, k)
    say("w4a16", layer.name, n, k)
    blob = _int4_blob(q, w)
    for m in cfg.ms:
        xb = synth.decode_x_bf16(cfg.cid, li, m, k)
        y16 = q.gemm_w4a16(dev_bf16(xb), blob, n, k, out_dtype=torch.bfloat16)
        y32 = q.gemm_w4a16(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref = gemm.w4a16(xb, rc, rs)
        _check(host_f64(y32), ref, False)
        _check(host_f64(y16), ref, True)
        _check_decode_ws(q.gemm_w4a16, q.gemm_w4a16_workspace, xb, blob, n, k, ref)


@pytest.mark.parametrize("m", [2, 17, 33, 50, 100])
def test_w4a16_ragged_batches(m):
    q = require_gpu()
    n, k = 272, 1152
    w = synth.weights(8, 1, n, k)
    xb = synth.activations_bf16(8, 2, m, k)
    say("w4a16 ragged", m)
    blob = _int4_blob(q, w)
    y = q.gemm_w4a16(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(host_f64(y), gemm.w4a16(xb, *int4.quantize(w)), False)


# Long K with one row tile per block: the pipelined k-split kernel at M <= 16
# (an odd number of chunks, waves whose last chunk is clamped), the k-split
# kernel with two m-tiles above (ragged second m-tile).
@pytest.mark.parametrize("m,k", [(17, 10240), (25, 8576), (32, 10240), (9, 8576)])
def test_w4a16_pipelined_long_k(m, k):
    q = require_gpu()
    n = 272
    w = synth.weights(9, 1, n, k)
    xb = synth.activations_bf16(9, 2, m, k)
    say("w4a16 pipelined long k", m, k)
    blob = _int4_blob(q, w)
    ref = gemm.w4a16(xb, *int4.quantize(w))
    for dt in (torch.float32, torch.bfloat16):
        y = q.gemm_w4a16(dev_bf16(xb), blob, n, k, out_dtype=dt)
        torch.cuda.synchronize()
        _check(host_f64(y), ref, dt == torch.bfloat16)


def test_w4a16_one_hot_layout_probe():
    q = require_gpu()
    n, k = 48, 384
    w = synth.weights(7, 1, n, k)
    blob = _int4_blob(q, w)
    ks = [0, 1, 7, 8, 31, 32, 127, 128, 200, 383]
    x = np.zeros((len(ks), k), dtype=np.float32)
    for i, kk in enumerate(ks):
        x[i, kk] = 1.0
    say("w4a16 one-hot probe")
    y = host_f64(q.gemm_w4a16(dev_bf16(synth.to_bf16_bits(x)), blob, n, k, out_dtype=torch.float32))
    torch.cuda.synchronize()
    wh = int4.dequantize(*int4.quantize(w))
    for i, kk in enumerate(ks):
        assert np.array_equal(y[i], wh[:, kk].astype(np.float32)), kk


# ---------------------------------------------------------------- LUT2 --

@pytest.mark.parametrize("li", range(3))
def test_lut2_gemma3_decode(li):
    """Every output of every Gemma3-12B-like LUT2 layer at every batch size."""
    q = require_gpu()
    cfg = configs.GEMMA3_LUT2
    layer = cfg.layers[li]
    n, k = layer.n, layer.k
    w, ri, rc = orows.lut2_layer(cfg.cid, li, n, k)
    say("lut2", layer.name, n, k)
    blob = _lut2_blob(q, w)
    for m in cfg.ms:
        xb = synth.decode_x_bf16(cfg.cid, li, m, k)
        y16 = q.gemm_lut2(dev_bf16(xb), blob, n, k, out_dtype=torch.bfloat16)
        y32 = q.gemm_lut2(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref = gemm.lut2_gemm(xb, ri, rc)
        _check(host_f64(y32), ref, False)
        _check(host_f64(y16), ref, True)
        _check_decode_ws(q.gemm_lut2, q.gemm_lut2_workspace, xb, blob, n, k, ref)


def test_lut2_one_hot_layout_probe_and_ragged():
    q = require_gpu()
    n, k = 32, 256
    w = synth.weights(7, 2, n, k)
    blob = _lut2_blob(q, w)
    ks = [0, 1, 3, 4, 7, 8, 31, 32, 127, 128, 255]
    x = np.zeros((len(ks), k), dtype=np.float32)
    for i, kk in enumerate(ks):
        x[i, kk] = 1.0
    say("lut2 one-hot probe")
    y = host_f64(q.gemm_lut2(dev_bf16(synth.to_bf16_bits(x)), blob, n, k, out_dtype=torch.float32))
    torch.cuda.synchronize()
    wh = lut2.dequantize(*lut2.fit(w))
    for i, kk in enumerate(ks):
        assert np.array_equal(y[i], wh[:, kk].astype(np.float32)), kk
    xb = synth.activations_bf16(8, 3, 40, k)
    y = q.gemm_lut2(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check(host_f64(y), gemm.lut2_gemm(xb, *lut2.fit(w)), False)


# ---------------------------------------------- decode k-chunking sweep --
# The decode kernels split k over 8 wavefronts and load each wavefront's
# groups in chunks (2 .. 16 groups) chosen from the group count; these shapes
# reach every chunk size, ragged group counts (idle and partly idle
# wavefronts), both row-tile widths (N >= 6144 uses two 16-row tiles per
# block) and both batch tilings (<= 16 and 17 .. 32 rows, and > 32 rows).

_CHUNK_K = [640, 2176, 5248, 8192, 8320, 15360, 20608]
_CHUNK_CASES = [(272, k) for k in _CHUNK_K] + [(6160, k) for k in _CHUNK_K if k <= 8320]


@pytest.mark.parametrize("fmt", ["int4", "lut2"])
@pytest.mark.parametrize("n,k", _CHUNK_CASES)
def test_decode_k_chunking(fmt, n, k):
    q = require_gpu()
    w = synth.weights(9, k, n, k)
    say("decode chunking", fmt, n, k)
    cols = sample_rows(n, 64, n * 3 + k)
    if fmt == "int4":
        blob = _int4_blob(q, w)
        ref_w = int4.quantize(w[cols])
        fn, ref_fn = q.gemm_w4a16, gemm.w4a16
    else:
        blob = _lut2_blob(q, w)
        ref_w = lut2.fit(w[cols])
        fn, ref_fn = q.gemm_lut2, gemm.lut2_gemm
    del w
    for m in (3, 20, 40):
        xb = synth.activations_bf16(9, m, m, k)
        y = fn(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check(host_f64(y)[:, cols], ref_fn(xb, *ref_w), False)


# --------------------------------------------- decode k split (workspace) --
# The workspace entry points split k over blocks: S slices of NW GW groups,
# P tile walkers per slice.  These shapes give a last slice with fewer groups
# than the others (G not a multiple of the slice), tile counts that leave
# some walkers a tile short (the second tile of a pair computed but not
# stored), ragged batches of one and two m-tiles, and both formats.

@pytest.mark.parametrize("fmt", ["int4", "lut2"])
@pytest.mark.parametrize("n,k", [(4096, 12288), (272, 8320), (3840, 15360), (16 * 257, 9088),
                                 (6160, 4224), (4096, 4096), (16 * 1031, 8192)])
def test_decode_split_ragged(fmt, n, k):
    q = require_gpu()
    w = synth.weights(15, k, n, k)
    say("decode split", fmt, n, k)
    if fmt == "int4":
        blob = _int4_blob(q, w)
        ref_w = orows.int4_quantize(w)
        fn, ws_fn, ref_fn = q.gemm_w4a16, q.gemm_w4a16_workspace, gemm.w4a16
    else:
        blob = _lut2_blob(q, w)
        ref_w = orows.lut2_fit(w)
        fn, ws_fn, ref_fn = q.gemm_lut2, q.gemm_lut2_workspace, gemm.lut2_gemm
    del w
    for m in (9, 13, 16, 17, 25, 32):
        xb = synth.activations_bf16(15, m, m, k)
        _check_decode_ws(fn, ws_fn, xb, blob, n, k, ref_fn(xb, *ref_w), need_split=k > 4096)


def test_decode_split_workspace_sizes():
    q = require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # k <= 4096, batches of at most 8 and above 32 need none
    assert q.gemm_w4a16_workspace(16, 16 * 2 * cus, 4096) == 0
    assert q.gemm_w4a16_workspace(16, 4096, 4096) == 0
    assert q.gemm_lut2_workspace(1, 3840, 15360) == 0
    assert q.gemm_w4a16_workspace(8, 4096, 12288) == 0
    assert q.gemm_w4a16_workspace(33, 4096, 12288) == 0
    assert q.gemm_w4a16_sp24_workspace(16, 4096, 4096) == 0
    assert q.gemm_w4a16_sp24_workspace(8, 4096, 12288) == 0
    assert q.gemm_w4a16_sp24_workspace(33, 4096, 12288) == 0
    # long k with 8 < m <= 32: S slices x m x n fp32 partial sums
    for ws_fn in (q.gemm_w4a16_workspace, q.gemm_lut2_workspace, q.gemm_w4a16_sp24_workspace):
        for m, n, k in ((16, 4096, 12288), (9, 3840, 15360), (32, 272, 8320)):
            nb = ws_fn(m, n, k)
            assert nb > 0 and nb % (4 * m * n) == 0 and 2 <= nb // (4 * m * n) <= k // 128
    # too small a workspace is refused before any launch
    lib = q.raw()
    st = lib.gemm_w4a16_ws(1 << 16, 1 << 17, 16, 4096, 12288, 1 << 18, 1, 1 << 19, 16, None)
    assert st == q.QL_EWORKSPACE
    st = lib.gemm_w4a16_sp24_ws(1 << 16, 1 << 17, 16, 4096, 12288, 1 << 18, 1, 1 << 19, 16, None)
    assert st == q.QL_EWORKSPACE


# ----------------------------------------- persistent decode tile walk --
# M <= 16 and K <= 4096 with at least two 16-row tiles per CU take the
# persistent kernel: each block walks tiles blockIdx.x, + gridDim.x, ...
# These shapes give an odd number of tiles per block (a last tile without a
# partner), a group count that leaves the last wave partly idle (K = 3840:
# 30 groups over 8 waves of 4) and the two-groups-per-wave variant (K = 2048).

@pytest.mark.parametrize("fmt", ["int4", "lut2"])
@pytest.mark.parametrize("n,k", [(16 * 1031, 3840), (16 * 1537, 2048)])
def test_decode_persistent_tile_walk(fmt, n, k):
    q = require_gpu()
    w = synth.weights(10, k, n, k)
    say("decode persistent", fmt, n, k)
    cols = np.unique(np.concatenate([sample_rows(n, 96, n + 7 * k), np.arange(n - 48, n)]))
    if fmt == "int4":
        blob = _int4_blob(q, w)
        ref_w = int4.quantize(w[cols])
        fn, ref_fn = q.gemm_w4a16, gemm.w4a16
    else:
        blob = _lut2_blob(q, w)
        ref_w = lut2.fit(w[cols])
        fn, ref_fn = q.gemm_lut2, gemm.lut2_gemm
    del w
    for m in (1, 7, 16, 25):   # 25: LUT2 takes the two-m-tile persistent kernel
        xb = synth.activations_bf16(10, m, m, k)
        y = fn(dev_bf16(xb), blob, n, k, out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check(host_f64(y)[:, cols], ref_fn(xb, *ref_w), False)


# ------------------------------------------ cooperative W4A4, ragged edges --
# Problems of more than half a round of 256 x 256 tiles (more tiles than
# CUs / 2) take the block-cooperative kernel.  With M and N not multiples of
# 256 its edge blocks read clamped (last valid) rows for the rows past M or
# N; those products must reach no stored output.  Checked on the last rows
# and columns and a sample.

@pytest.mark.parametrize("m,n,k", [(4100, 16400, 512), (8191, 8208, 640),
                                   (2100, 4000, 640),    # 144 tiles: less than one round
                                   (2048, 6144, 1024)])  # 192 tiles
def test_w4a4_cooperative_ragged_edges(m, n, k):
    q = require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 2 * ((m + 255) // 256) * ((n + 255) // 256) > cus
    bits = synth.activations_bf16(11, m, m, k, outliers="channels")
    w = synth.weights(11, n, n, k)
    say("w4a4 coop ragged", m, n, k)
    blob = _nvfp4_blob(q, w)
    ac, as_, at = q.quantize_nvfp4(dev_bf16(bits))
    y32 = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.float32)
    y16 = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(m, 40, m + 3), np.arange(m - 24, m)]))
    cols = np.unique(np.concatenate([sample_rows(n, 40, n + 5), np.arange(n - 24, n)]))
    xf = synth.bf16_bits_as_f32(bits)
    ref = gemm.w4a4(*nvfp4.quantize(xf[rows], s_t=nvfp4.tensor_scale(xf)),
                    *nvfp4.quantize(w[cols], s_t=nvfp4.tensor_scale(w)))
    _check(host_f64(y32)[np.ix_(rows, cols)], ref, False)
    _check(host_f64(y16)[np.ix_(rows, cols)], ref, True)
    # the whole bf16 output (staged through LDS per wave, stored as whole rows)
    # is the round-to-nearest-even of the fp32 output of the same kernel
    assert torch.equal(y16, y32.to(torch.bfloat16))
    # nothing was written past the output: the buffers are exactly [m, n]
    assert y32.shape == (m, n) and y16.shape == (m, n)


# ------------------------------ cooperative W4A4, k split of the last round --
# With a workspace, a last round of tiles that is at most half full, or a
# whole problem of at most half a round, is split along k over the idle CUs
# (fp32 partial tiles, then a fixed-order sum).  The
# oracle checks a sample; the whole output is compared with the unsplit call
# (already pinned to the oracle by the tests above), which differs only in the
# fp32 summation order.

@pytest.mark.parametrize("m,n,k", [
    (4096, 5120, 5120),   # 27B-class o_proj at M = 4096: 320 tiles
    (4096, 5120, 17408),  # 27B-class down at M = 4096 (the benchmarked split shapes)
    (4347, 4096, 2048),   # 17 x 16 tiles, ragged M
    (4352, 4096, 256),    # K = 256: two stage pairs, so at most two slices
    (4096, 5376, 1024),   # 336 tiles: 80 in the last round, 3 slices
    (4096, 4864, 1024),   # 304 tiles: 48 in the last round, 5 slices
    (1024, 5120, 17408),  # 80 tiles, less than one round: 3 slices
    (300, 4096, 1024),    # 32 tiles, ragged M: 8 slices
    (64, 256, 8192),      # a single tile, M <= 128 with long k: 8 slices
])
def test_w4a4_split_last_round(m, n, k):
    q = require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = ((m + 255) // 256) * ((n + 255) // 256)
    tail = tiles % cus
    need = q.gemm_w4a4_workspace(m, n, k)
    splits = min(cus // tail, k // 128, 8) if 0 < tail else 0
    if m <= 128 and not (2 * tiles <= cus and k >= 8192):
        splits = 0   # the per-wave kernel is faster there
    if splits < 2:
        pytest.skip(f"{tiles} tiles on {cus} CUs: no split applies")
    assert need == tail * splits * 256 * 256 * 4
    bits = synth.activations_bf16(12, m, m, k, outliers="channels")
    w = synth.weights(12, n, n, k)
    say("w4a4 split last round", m, n, k, tail, splits)
    blob = _nvfp4_blob(q, w)
    ac, as_, at = q.quantize_nvfp4(dev_bf16(bits))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y32 = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.float32, workspace=ws)
    y16 = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.bfloat16, workspace=ws)
    y16b = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.bfloat16, workspace=ws)
    y32u = q.gemm_w4a4(ac, as_, at, blob, m, n, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y16, y16b)
    a, b = host_f64(y32), host_f64(y32u)
    assert np.max(np.abs(a - b)) <= 1e-4 * np.sqrt(np.mean(b * b))
    rows = np.unique(np.concatenate([sample_rows(m, 40, m + 1), np.arange(m - 16, m)]))
    cols = np.unique(np.concatenate([sample_rows(n, 40, n + 2), np.arange(n - 16, n)]))
    xf = synth.bf16_bits_as_f32(bits)
    ref = gemm.w4a4(*nvfp4.quantize(xf[rows], s_t=nvfp4.tensor_scale(xf)),
                    *nvfp4.quantize(w[cols], s_t=nvfp4.tensor_scale(w)))
    _check(a[np.ix_(rows, cols)], ref, False)
    _check(host_f64(y16)[np.ix_(rows, cols)], ref, True)


def test_w4a4_workspace_not_needed_for_whole_rounds():
    q = require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # whole rounds of tiles on this device, a last round more than half full,
    # a problem of more than half a round, and k too short for two slices
    assert q.gemm_w4a4_workspace(256 * cus, 256, 512) == 0
    assert q.gemm_w4a4_workspace(256 * (cus + cus // 2 + 1), 256, 512) == 0
    assert q.gemm_w4a4_workspace(256 * (cus // 2 + 1), 256, 512) == 0
    assert q.gemm_w4a4_workspace(64, 256, 128) == 0
    # M <= 128 with short k, or above half a round: the per-wave kernel, no split
    assert q.gemm_w4a4_workspace(64, 256, 512) == 0
    assert q.gemm_w4a4_workspace(128, 256 * (cus + cus // 4), 512) == 0
    # a small problem with room for slices needs one
    assert q.gemm_w4a4_workspace(256, 256, 512) == 4 * 256 * 256 * 4
    assert q.gemm_w4a4_workspace(64, 256, 8192) == 8 * 256 * 256 * 4


# ------------------------------------------------------------ blob guard --
# The host cannot read a blob's header without a synchronising copy, so the
# W4A4 kernels check it (magic, version, format, n, k) before any other access
# and return on a mismatch: the output keeps its previous contents and no byte
# past the blob is read.

def test_w4a4_blob_guard_leaves_output_untouched():
    q = require_gpu()
    n, k, m = 256, 512, 4
    w = synth.weights(13, 0, n, k)
    nv, i4, l2 = _nvfp4_blob(q, w), _int4_blob(q, w), _lut2_blob(q, w)
    ac, as_, at = q.quantize_nvfp4(dev_f32(synth.activations(13, 0, m, k)))
    say("w4a4 blob guard")
    # through the C ABI: the Python binding would reject most of these calls
    # on the host already (blob size, operand shapes)
    lib = q.raw()

    def raw_call(blob, nn, kk, y):
        st = lib.gemm_w4a4(ac.data_ptr(), as_.data_ptr(), at.data_ptr(), blob.data_ptr(), m, nn,
                           kk, y.data_ptr(), q.QL_F32, torch.cuda.current_stream().cuda_stream)
        assert st == q.QL_OK, st
    cases = [
        ("an INT4 blob", n, lambda y: raw_call(i4, n, k, y)),
        ("a LUT2 blob", n, lambda y: raw_call(l2, n, k, y)),
        ("n below the packed n", n - 16, lambda y: raw_call(nv, n - 16, k, y)),
        ("k below the packed k", n, lambda y: raw_call(nv, n, 256, y)),
    ]
    for name, nn, fn in cases:
        y = torch.full((m, nn), 7.0, dtype=torch.float32, device="cuda")
        fn(y)
        torch.cuda.synchronize()
        assert torch.all(y == 7.0), name
    y = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
    q.gemm_w4a4(ac, as_, at, nv, m, n, k, y=y)
    torch.cuda.synchronize()
    assert not torch.any(y == 7.0)


# The decode kernels read the header with their first weight loads and test
# it before their first store: a blob of another format or shape, at least as
# large as the expected one (so every read stays inside it), leaves y as it
# was.  Each kernel path: persistent (at least two row tiles per CU,
# k <= 4096), k-split (few row tiles), pipelined long k (m <= 16), and the k
# split over blocks with a workspace (long k, 8 < m <= 32).

@pytest.mark.parametrize("n,k,m", [(16384, 1024, 3), (272, 1024, 5), (272, 8192, 7),
                                   (272, 8192, 12)])
def test_decode_blob_guard_leaves_output_untouched(n, k, m):
    q = require_gpu()
    w = synth.weights(16, 0, n, k)
    nv, i4, l2 = _nvfp4_blob(q, w), _int4_blob(q, w), _lut2_blob(q, w)
    c24, s24 = q.quantize_int4_g128(dev_f32(w), sparse24=True)
    sp = q.repack_weights(q.QL_INT4_SP24, n, k, c24, s24)
    w2 = synth.weights(16, 1, 2 * n, k)
    i4_2n, l2_2n = _int4_blob(q, w2), _lut2_blob(q, w2)        # packed for another n
    w3 = synth.weights(16, 2, n, 2 * k)
    i4_2k = _int4_blob(q, w3)                                  # packed for another k
    xb = dev_bf16(synth.activations_bf16(16, 0, m, k))
    say("decode blob guard", n, k, m)
    ws4 = torch.empty(max(16, q.gemm_w4a16_workspace(m, n, k)), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(max(16, q.gemm_lut2_workspace(m, n, k)), dtype=torch.uint8, device="cuda")
    ws3 = torch.empty(max(16, q.gemm_w4a16_sp24_workspace(m, n, k)), dtype=torch.uint8,
                      device="cuda")
    cases = [
        ("w4a16 given an NVFP4 blob", q.gemm_w4a16, nv, None),
        ("w4a16 given an INT4 blob of 2n rows", q.gemm_w4a16, i4_2n, None),
        ("w4a16 given an INT4 blob of 2k columns", q.gemm_w4a16, i4_2k, None),
        ("w4a16 (workspace) given an INT4 blob of 2k columns", q.gemm_w4a16, i4_2k, ws4),
        ("lut2 given an INT4 blob", q.gemm_lut2, i4, None),
        ("lut2 given a LUT2 blob of 2n rows", q.gemm_lut2, l2_2n, None),
        ("lut2 (workspace) given an INT4 blob", q.gemm_lut2, i4, ws2),
        ("sp24 given an INT4 blob", q.gemm_w4a16_sp24, i4, None),
        ("sp24 (workspace) given an INT4 blob", q.gemm_w4a16_sp24, i4, ws3),
    ]
    for name, fn, blob, ws in cases:
        assert blob.numel() >= q.repack_weights_bytes(
            {q.gemm_w4a16: q.QL_INT4_G128, q.gemm_lut2: q.QL_LUT2,
             q.gemm_w4a16_sp24: q.QL_INT4_SP24}[fn], n, k), name
        y = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
        fn(xb, blob, n, k, y=y, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(y == 7.0), name
    # and the right blobs do write
    for fn, blob in ((q.gemm_w4a16, i4), (q.gemm_lut2, l2), (q.gemm_w4a16_sp24, sp)):
        y = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
        fn(xb, blob, n, k, y=y)
        torch.cuda.synchronize()
        assert not torch.any(y == 7.0)


def test_binding_rejects_undersized_buffers():
    """The Python binding checks operand shapes and blob sizes on the host, so
    a too-small buffer never reaches a kernel."""
    q = require_gpu()
    n, k, m = 256, 512, 4
    w = synth.weights(14, 0, n, k)
    nv, i4 = _nvfp4_blob(q, w), _int4_blob(q, w)
    ac, as_, at = q.quantize_nvfp4(dev_f32(synth.activations(14, 0, m, k)))
    xb = dev_bf16(synth.decode_x_bf16(14, 0, m, k))
    say("binding size checks")
    bad = [
        lambda: q.gemm_w4a4(ac, as_, at, i4, m, n, k),                     # INT4 blob is too small
        lambda: q.gemm_w4a4(ac, as_, at, nv, m, n + 16, k),                # blob for a smaller n
        lambda: q.gemm_w4a4(ac[:, :128].contiguous(), as_, at, nv, m, n, k),
        lambda: q.gemm_w4a4(ac, as_, at, nv, m + 1, n, k),                 # fewer rows than m
        lambda: q.gemm_w4a4(ac, as_, at, nv, m, n, k, y=torch.empty((m, n - 16), device="cuda")),
        lambda: q.gemm_w4a16(xb, i4, n + 16, k),
        lambda: q.gemm_w4a16(xb[:, :256].contiguous(), i4, n, k),
        lambda: q.gemm_lut2(xb, i4[:1024], n, k),
        lambda: q.gemm_w4a16_sp24(xb.float(), i4, n, k),                   # fp32 activations
    ]
    # weight preparation and the quantizer: short outputs, wrong input dtype,
    # short canonical inputs of the repacker
    wd = dev_f32(w)
    wc, ws_, wt = q.quantize_nvfp4(wd)
    c4, s4 = q.quantize_int4_g128(wd)
    u8 = lambda nb: torch.empty(nb, dtype=torch.uint8, device="cuda")
    bad += [
        lambda: q.quantize_nvfp4(wd, codes=u8(n * k // 2 - 16)),
        lambda: q.quantize_nvfp4(wd, scales=u8(n * k // 16 - 16)),
        lambda: q.quantize_nvfp4(wd, ts_out=torch.empty(1, dtype=torch.float64, device="cuda")),
        lambda: q.quantize_nvfp4(wd.reshape(1, n, k)),
        lambda: q.quantize_int4_g128(wd.to(torch.bfloat16)),                 # bf16 read as fp32
        lambda: q.quantize_int4_g128(wd, codes=u8(n * k // 2 - 16)),
        lambda: q.quantize_int4_g128(wd, scales=u8(n * (k // 128) * 2 - 2)),
        lambda: q.fit_lut2(wd.to(torch.bfloat16)),
        lambda: q.fit_lut2(wd, idx=u8(n * k // 4 - 16)),
        lambda: q.repack_weights(q.QL_NVFP4, n, k, wc[:-1], ws_, wt),
        lambda: q.repack_weights(q.QL_NVFP4, n, k, wc, ws_[:-1], wt),
        lambda: q.repack_weights(q.QL_NVFP4, n, k, wc, ws_, None),
        lambda: q.repack_weights(q.QL_INT4_G128, n, k, c4, s4[:-1]),
        lambda: q.repack_weights(q.QL_LUT2, n, k, c4[: n // 4], s4),           # idx rows missing
        lambda: q.repack_weights(q.QL_INT4_G128, n, k, c4, s4, packed=u8(1024)),
        lambda: q.repack_weights(7, n, k, c4, s4),
    ]
    for fn in bad:
        with pytest.raises(ValueError):
            fn()

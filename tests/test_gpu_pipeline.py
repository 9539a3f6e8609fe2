"""Weight streaming from host memory (decode_nvfp4_rtn_amd.pipeline).

The streamed pipeline runs the same kernels on the same inputs as resident
weights, so its outputs must be bit-identical to the resident run's, which
the GEMM parity tests already tie to the oracle; one layer is also checked
against the oracle directly.
"""

import numpy as np
import pytest
import torch

from decode_nvfp4_rtn_amd import synth
from oracle import nvfp4, gemm
from tests.gpu_common import require_gpu, say, dev_f32, dev_bf16, host_f64, sample_rows

pytestmark = pytest.mark.gpu


def test_streamed_weights_match_resident_weights():
    q = require_gpu()
    from decode_nvfp4_rtn_amd.pipeline import PrefillWeightStream
    m = 300
    shapes = [(512, 256), (1024, 384), (272, 512), (768, 256), (256, 640)]   # five layers
    say("pipeline", m, shapes)
    blocks, wts = [], []
    xs, xbits = [], []
    for blk in range(2):   # two blocks with the same shapes and different weights
        blobs, wl = [], []
        for li, (n, k) in enumerate(shapes):
            w = synth.weights(12 + blk, li, n, k)
            wc, wsc, wt = q.quantize_nvfp4(dev_f32(w))
            blobs.append(q.repack_weights(q.QL_NVFP4, n, k, wc, wsc, wt))
            wl.append(w)
        blocks.append(blobs)
        wts.append(wl)
    for li, (n, k) in enumerate(shapes):
        bits = synth.activations_bf16(12, li, m, k, outliers="channels")
        xbits.append(bits)
        xs.append(dev_bf16(bits))
    dev = xs[0].device
    streamer = PrefillWeightStream([[b.cpu().pin_memory() for b in blk] for blk in blocks], dev)
    codes = [torch.empty((m, k // 2), dtype=torch.uint8, device=dev) for _, k in shapes]
    scales = [torch.empty((m, k // 16), dtype=torch.uint8, device=dev) for _, k in shapes]
    tsc = [torch.empty(1, dtype=torch.float32, device=dev) for _ in shapes]
    wsp = [torch.empty(max(16, q.quantize_nvfp4_workspace(m, k)), dtype=torch.uint8, device=dev)
           for _, k in shapes]
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for n, _ in shapes]
    for order in ([0, 1, 0, 1], [1, 0, 1, 1, 0]):   # both buffers reused several times
        streamer.run(order, shapes, xs, ys, codes, scales, tsc, wsp)
        torch.cuda.synchronize()
        last = order[-1]
        for li, (n, k) in enumerate(shapes):
            ac, as_, at = q.quantize_nvfp4(xs[li])
            ref = q.gemm_w4a4(ac, as_, at, blocks[last][li], m, n, k, out_dtype=torch.bfloat16)
            torch.cuda.synchronize()
            assert torch.equal(ys[li].view(torch.int16), ref.view(torch.int16)), (order, li)
    # and one layer of the last block against the oracle
    n, k = shapes[1]
    rows = sample_rows(m, 40, 5)
    xf = synth.bf16_bits_as_f32(xbits[1])
    ref = gemm.w4a4(*nvfp4.quantize(xf[rows], s_t=nvfp4.tensor_scale(xf)),
                    *nvfp4.quantize(wts[0][1]))
    assert gemm.bf16_output_ok(host_f64(ys[1])[rows], ref)


def test_back_to_back_runs_without_host_sync():
    """Two run() calls queued with no synchronisation between them: the second
    call's first copies go into buffers whose blocks the first call's last
    GEMMs still read, so they must wait for them.  Each call writes its own
    outputs; both must equal the resident-weight outputs bit for bit."""
    q = require_gpu()
    from decode_nvfp4_rtn_amd.pipeline import PrefillWeightStream
    m = 2048
    shapes = [(1024, 2048), (2048, 1024), (1024, 4096)]
    say("pipeline back to back", m, shapes)
    blocks = []
    for blk in range(2):
        blobs = []
        for li, (n, k) in enumerate(shapes):
            wc, wsc, wt = q.quantize_nvfp4(dev_f32(synth.weights(20 + blk, li, n, k)))
            blobs.append(q.repack_weights(q.QL_NVFP4, n, k, wc, wsc, wt))
        blocks.append(blobs)
    xs = [dev_bf16(synth.activations_bf16(20, li, m, k, outliers="channels"))
          for li, (_, k) in enumerate(shapes)]
    dev = xs[0].device
    streamer = PrefillWeightStream([[b.cpu().pin_memory() for b in blk] for blk in blocks], dev)

    def bufs():
        return ([torch.empty((m, k // 2), dtype=torch.uint8, device=dev) for _, k in shapes],
                [torch.empty((m, k // 16), dtype=torch.uint8, device=dev) for _, k in shapes],
                [torch.empty(1, dtype=torch.float32, device=dev) for _ in shapes],
                [torch.empty(max(16, q.quantize_nvfp4_workspace(m, k)), dtype=torch.uint8,
                             device=dev) for _, k in shapes],
                [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for n, _ in shapes])
    ref = []
    for blk in range(2):
        ref.append([])
        for li, (n, k) in enumerate(shapes):
            ac, as_, at = q.quantize_nvfp4(xs[li])
            ref[blk].append(q.gemm_w4a4(ac, as_, at, blocks[blk][li], m, n, k,
                                        out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    # run 1 ends with block 0 in buffer 0 and block 1 in buffer 1; run 2
    # copies block 1 into buffer 0 and block 0 into buffer 1
    c1, s1, t1, w1, y1 = bufs()
    c2, s2, t2, w2, y2 = bufs()
    streamer.run([0, 1, 0, 1], shapes, xs, y1, c1, s1, t1, w1)
    streamer.run([1, 0], shapes, xs, y2, c2, s2, t2, w2)
    torch.cuda.synchronize()
    for li in range(len(shapes)):
        assert torch.equal(y1[li].view(torch.int16), ref[1][li].view(torch.int16)), ("run 1", li)
        assert torch.equal(y2[li].view(torch.int16), ref[0][li].view(torch.int16)), ("run 2", li)


def test_stream_rejects_unpinned_blobs():
    require_gpu()
    from decode_nvfp4_rtn_amd.pipeline import PrefillWeightStream
    with pytest.raises(ValueError):
        PrefillWeightStream([[torch.zeros(64, dtype=torch.uint8)]])

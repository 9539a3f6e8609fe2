"""The hot path captured in a HIP graph (torch.cuda.graph over the C ABI).

No entry point allocates, frees, synchronises or clears memory with a memset
(the library contains none of those calls), so the whole path can be
captured: activation quantize and the W4A4 GEMM with its k-split workspace,
the quantize folded into the GEMM, and the three decode GEMMs with their
k-split workspaces.  The graph is replayed several times; between replays
the program runs the same entry points eagerly on other inputs through the
same workspaces (so a replay may not rely on what an earlier run left in
them) and clears the outputs; every replay must reproduce the eager results
bit for bit.
"""

import pytest
import torch

from decode_nvfp4_rtn_amd import synth
from tests.gpu_common import require_gpu, say, dev_f32, dev_bf16

pytestmark = pytest.mark.gpu


def _nvfp4_blob(q, w):
    wc, ws, wt = q.quantize_nvfp4(dev_f32(w))
    n, k = w.shape
    return q.repack_weights(q.QL_NVFP4, n, k, wc, ws, wt)


def test_hot_path_graph_replays_match_eager():
    q = require_gpu()
    dev = "cuda"
    # prefill: 300 tokens (a k split of a small problem), NVFP4 4096 x 1024
    mp, np_, kp = 300, 4096, 1024
    wp = synth.weights(31, 0, np_, kp)
    blob_p = _nvfp4_blob(q, wp)
    xp = dev_bf16(synth.activations_bf16(31, 1, mp, kp, outliers="channels"))
    xp_other = dev_bf16(synth.activations_bf16(31, 2, mp, kp, outliers="channels"))
    codes = torch.empty((mp, kp // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((mp, kp // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    ts_f = torch.empty(1, dtype=torch.float32, device=dev)
    qws = torch.empty(max(16, q.quantize_nvfp4_workspace(mp, kp)), dtype=torch.uint8, device=dev)
    gws_n = q.gemm_w4a4_workspace(mp, np_, kp)
    assert gws_n > 0
    gws = torch.empty(gws_n, dtype=torch.uint8, device=dev)
    # decode: 16 tokens against long-K layers, each with its k-split workspace
    md, nd, kd = 16, 4096, 12288
    wd = synth.weights(31, 3, nd, kd)
    c4, s4 = q.quantize_int4_g128(dev_f32(wd))
    blob4 = q.repack_weights(q.QL_INT4_G128, nd, kd, c4, s4)
    c24, s24 = q.quantize_int4_g128(dev_f32(wd), sparse24=True)
    blob24 = q.repack_weights(q.QL_INT4_SP24, nd, kd, c24, s24)
    nl, kl = 3840, 15360
    wl = synth.weights(31, 4, nl, kl)
    li, lc = q.fit_lut2(dev_f32(wl))
    blobl = q.repack_weights(q.QL_LUT2, nl, kl, li, lc)
    del c4, s4, c24, s24, li, lc
    xd = dev_bf16(synth.decode_x_bf16(31, 5, md, kd))
    xl = dev_bf16(synth.decode_x_bf16(31, 6, md, kl))
    ws4 = torch.empty(q.gemm_w4a16_workspace(md, nd, kd), dtype=torch.uint8, device=dev)
    ws24 = torch.empty(q.gemm_w4a16_sp24_workspace(md, nd, kd), dtype=torch.uint8, device=dev)
    wsl = torch.empty(q.gemm_lut2_workspace(md, nl, kl), dtype=torch.uint8, device=dev)
    assert ws4.numel() > 0 and ws24.numel() > 0 and wsl.numel() > 0

    outs = {"w4a4": torch.empty((mp, np_), dtype=torch.bfloat16, device=dev),
            "fused": torch.empty((mp, np_), dtype=torch.bfloat16, device=dev),
            "w4a16": torch.empty((md, nd), dtype=torch.bfloat16, device=dev),
            "sp24": torch.empty((md, nd), dtype=torch.float32, device=dev),
            "lut2": torch.empty((md, nl), dtype=torch.bfloat16, device=dev)}

    def path(x_pre, x_dec, x_lut):
        q.quantize_nvfp4(x_pre, codes=codes, scales=scales, workspace=qws, ts_out=ts)
        q.gemm_w4a4(codes, scales, ts, blob_p, mp, np_, kp, y=outs["w4a4"], workspace=gws)
        q.quantize_gemm_w4a4(x_pre, blob_p, np_, y=outs["fused"], ts_out=ts_f, workspace=qws)
        q.gemm_w4a16(x_dec, blob4, nd, kd, y=outs["w4a16"], workspace=ws4)
        q.gemm_w4a16_sp24(x_dec, blob24, nd, kd, y=outs["sp24"], workspace=ws24)
        q.gemm_lut2(x_lut, blobl, nl, kl, y=outs["lut2"], workspace=wsl)

    say("graph: eager reference")
    path(xp, xd, xl)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref_ts, ref_ts_f = ts.clone(), ts_f.clone()
    assert torch.equal(ref_ts, ref_ts_f)

    say("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path(xp, xd, xl)
    torch.cuda.synchronize()

    xd_other = dev_bf16(synth.decode_x_bf16(31, 7, md, kd))
    xl_other = dev_bf16(synth.decode_x_bf16(31, 8, md, kl))
    for rep in range(3):
        # eager work between replays: the same entry points on other inputs,
        # through the same workspaces, then cleared outputs
        path(xp_other, xd_other, xl_other)
        torch.cuda.synchronize()
        for v in outs.values():
            v.fill_(0)
        ts.fill_(0)
        ts_f.fill_(0)
        say("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), (rep, k)
        assert torch.equal(ts, ref_ts) and torch.equal(ts_f, ref_ts), rep

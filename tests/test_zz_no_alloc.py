"""quantize_nvfp4_noalloc (the entry point that allocates nothing) against
quantize_nvfp4 with a caller workspace, through the C ABI: codes, scales and
the tensor scale bit for bit, on calls issued back to back on one stream, the
later ones on smaller inputs (so a later call must read only its own partial
maxima, not what the larger call left in the library's array)."""

import ctypes

import numpy as np
import pytest
import torch

from decode_nvfp4_rtn_amd import synth
from oracle import nvfp4
from tests.gpu_common import require_gpu, say, dev_f32, dev_bf16, host_u8

pytestmark = pytest.mark.gpu


def _outputs(rows, cols):
    return (torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
            torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda"),
            torch.empty(1, dtype=torch.float32, device="cuda"))


def _raw(lib, x, codes, scales, ts, flags=0):
    dt = 1 if x.dtype == torch.bfloat16 else 0
    st = lib.quantize_nvfp4_noalloc(
        ctypes.c_void_p(x.data_ptr()), dt, x.shape[0], x.shape[1],
        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
        ctypes.c_void_p(ts.data_ptr()), flags,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st


def test_noalloc_quantize_matches_workspace_entry_point():
    q = require_gpu()
    lib = q.raw()
    # large first (1024 partial maxima, magnitudes x100), then smaller inputs
    # (a few partials, smaller magnitudes): a stale partial would raise s_t
    big = synth.activations_bf16(6, 0, 8192, 4096, outliers="channels")
    big = synth.to_bf16_bits(synth.bf16_bits_as_f32(big) * np.float32(100.0))
    small = synth.activations_bf16(6, 1, 300, 512, outliers="elements")
    tiny32 = synth.activations(6, 2, 3, 48)
    xs = [dev_bf16(big), dev_bf16(small), dev_f32(tiny32)]
    say("noalloc quantize", [tuple(x.shape) for x in xs])
    outs = [_outputs(*x.shape) for x in xs]
    for x, (c, s, t) in zip(xs, outs):          # issued back to back, no sync
        _raw(lib, x, c, s, t)
    refs = [q.quantize_nvfp4(x) for x in xs]     # the workspace entry point
    torch.cuda.synchronize()
    for (c, s, t), (rc, rs, rt) in zip(outs, refs):
        assert torch.equal(t, rt)
        assert torch.equal(s, rs)
        assert torch.equal(c, rc)
    # the smaller call's tensor scale is its own, as the oracle computes it
    assert np.float32(outs[1][2].item()) == nvfp4.tensor_scale(synth.bf16_bits_as_f32(small))
    assert np.float32(outs[2][2].item()) == nvfp4.tensor_scale(tiny32)
    # a second pair of calls in a row, large then small again, after the above
    c2, s2, t2 = _outputs(*xs[1].shape)
    _raw(lib, xs[0], *outs[0])
    _raw(lib, xs[1], c2, s2, t2)
    torch.cuda.synchronize()
    assert torch.equal(t2, refs[1][2]) and torch.equal(s2, refs[1][1]) and torch.equal(c2, refs[1][0])
    assert torch.equal(outs[0][0], refs[0][0])


def test_noalloc_quantize_static_scale_and_binding():
    q = require_gpu()
    x = dev_f32(synth.activations(6, 3, 128, 256))
    say("noalloc quantize static scale")
    ts = torch.tensor([1e-3], dtype=torch.float32, device="cuda")
    c, s, t = q.quantize_nvfp4_noalloc(x, *_outputs(128, 256)[:2], ts.clone(), static_scale=True)
    rc, rs, _ = q.quantize_nvfp4(x, tensor_scale=ts)
    torch.cuda.synchronize()
    assert torch.equal(c, rc) and torch.equal(s, rs) and torch.equal(t, ts)
    c, s, t = q.quantize_nvfp4_noalloc(x, *_outputs(128, 256))
    rc, rs, rt = q.quantize_nvfp4(x)
    torch.cuda.synchronize()
    assert torch.equal(c, rc) and torch.equal(s, rs) and torch.equal(t, rt)
    assert host_u8(c).shape == (128, 128)

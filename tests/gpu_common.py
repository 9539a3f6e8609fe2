"""Helpers shared by the GPU parity tests (marked ``gpu``).

The HIP path is reached only through ``decode_nvfp4_rtn_amd.qlin`` (the C
ABI); expected values come only from ``oracle`` on inputs drawn by
``decode_nvfp4_rtn_amd.synth``.
"""

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    """Skip when no GPU is visible; on a GPU host the library must load."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from decode_nvfp4_rtn_amd import qlin  # raises ImportError if libqlin.so is missing
    return qlin


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def _host(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a if a.flags.writeable else a.copy()   # torch wants writable host arrays


def dev_f32(a):
    return torch.from_numpy(_host(a, np.float32)).cuda()


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> GPU bfloat16 tensor."""
    return torch.from_numpy(_host(bits, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def rows_f64(t, rows):
    """Rows `rows` (numpy indices) of a GPU matrix, as float64 host values."""
    sel = t.index_select(0, torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(t.device))
    return host_f64(sel)


def host_u8(t):
    return t.cpu().numpy().view(np.uint8)


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def host_f64(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def sample_rows(n, count, seed):
    """A fixed seeded sample of row indices that always includes the last row."""
    if n <= count:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(n - 1, count - 1, replace=False))
    return np.concatenate([idx, [n - 1]])

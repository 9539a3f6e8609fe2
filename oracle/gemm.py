"""Linear-layer products on dequantized operands, and the pass rule (oracle).

A linear layer computes Y = X W^T with X [m, k] and W [n, k] (torch Linear
convention; the pages give no layouts).

* W4A4 (prefill; Mix-Quant technical summary, section 2, system-level
  deployment: the prefill worker runs NVFP4 weights and NVFP4 activations):
  Y = X_hat W_hat^T with both operands NVFP4-dequantized.
* W4A16 (decode; Disaggregated Quantization: decode switches to a weight-only
  path that leaves activations unquantized; MARLIN article, "どんな技術か":
  FP16 activations times INT4 weights): Y = X W_hat^T with X in bfloat16.
* W4A16 with 2:4 sparse INT4 weights (MARLIN article, "データの扱い方" and
  "実験と結果": Sparse-MARLIN): the same product on the pruned weights.
* LUT2 (decode with a 2-bit codebook; Disaggregated Quantization, full
  disaggregation; KLLM article section 3): Y = X C[idx]^T.

All three products are float64 BLAS matrix multiplies of exactly
dequantized operands; there is no blocking or reordering beyond the library
call.
"""

import numpy as np

from . import nvfp4, int4, lut2, sparse24
from .formats import bf16_bits_to_f32


def w4a4(a_codes, a_scales, a_st, w_codes, w_scales, w_st):
    xa = nvfp4.dequantize(a_codes, a_scales, a_st)
    wh = nvfp4.dequantize(w_codes, w_scales, w_st)
    return xa @ wh.T


def w4a16(x_bf16_bits, w_codes, w_scales):
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    return x @ int4.dequantize(w_codes, w_scales).T


def w4a16_sp24(x_bf16_bits, w_codes, w_scales):
    """W4A16 with a 2:4 sparse INT4 blob packed from (w_codes, w_scales): the
    dense product of the codes the packer keeps (sparse24.keep_codes)."""
    return w4a16(x_bf16_bits, sparse24.keep_codes(w_codes), w_scales)


def lut2_gemm(x_bf16_bits, w_idx, w_centroids):
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    return x @ lut2.dequantize(w_idx, w_centroids).T


# ---------------------------------------------------------------------------
# pass rule
# ---------------------------------------------------------------------------
TOL = 1e-3  # max |y - y_ref| / rms(y_ref)


def normalized_max_error(y, y_ref):
    """max |y - y_ref| / sqrt(mean(y_ref^2))."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2))
    if rms == 0:
        return float(np.max(np.abs(y - y_ref))) if y.size else 0.0
    return float(np.max(np.abs(y - y_ref)) / rms)


def bf16_ulp(v):
    """Spacing of bfloat16 numbers at |v| (float64); subnormal spacing below 2^-126."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def bf16_output_ok(y_bf16_as_f64, y_ref, tol=TOL):
    """Pass rule for bfloat16 outputs.

    A correctly rounded bfloat16 output already differs from the exact value
    by up to half a bfloat16 ulp (~4e-3 relative), so the fp32 bar is widened
    by that rounding: |y - y_ref| <= tol * rms + ulp_bf16(|y_ref| + tol*rms)/2
    element by element.
    """
    y = np.asarray(y_bf16_as_f64, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref ** 2)) if y_ref.size else 0.0
    bound = tol * rms + 0.5 * bf16_ulp(np.abs(y_ref) + tol * rms)
    return bool(np.all(np.abs(y - y_ref) <= bound))

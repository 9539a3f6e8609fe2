"""NVFP4 round-to-nearest quantizer (oracle; test infrastructure).

Source: Mix-Quant technical summary (gist.science), section 2 "Method",
hybrid-precision strategy, prefill bullet: NVFP4 carries a local scale for
every group of 16 elements plus a tensor-level scale, and plain
round-to-nearest (RTN) quantization is enough for this format.  Both the
weights and the activations of the prefill linear layers are quantized this
way (NVFP4 W4A4; same page, section 2, system-level deployment).

The pages fix neither the binary32 order of operations nor the scale
conventions.  The reading taken here (every step is one correctly rounded
binary32 operation, written rn32(...)):

1. amax_t = max |x| over the whole tensor (exact).
2. s_t = rn32(amax_t / 2688); 2688 = 6 * 448 maps the largest element to the
   largest E2M1 magnitude (6) under the largest E4M3 scale (448).  A given
   (calibrated) s_t may be passed instead.
3. d = rn32(6 * s_t).
4. per 16-group: a_g = max |x| over the group; s_g = E4M3(rn32(a_g / d)),
   or 0 when d == 0.
5. p_g = rn32(s_g * s_t).  If p_g == 0 every code of the group is the sign
   bit alone.  Otherwise inv_g = rn32(1 / p_g), y = rn32(x * inv_g) and the
   code is E2M1(y).
6. Two codes per byte, even column in the low nibble; scales are E4M3 bytes
   laid out [rows, cols/16]; s_t is binary32.
7. Dequantization: x_hat = E2M1(c) * E4M3(s_g) * s_t, exact in float64.
"""

import numpy as np

from .formats import rn32, enc_e2m1, dec_e2m1, enc_e4m3, dec_e4m3

GROUP = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0
TENSOR_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688


def tensor_scale(x):
    """Steps 1-2: the dynamic tensor scale s_t (binary32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float64(np.max(np.abs(x))) if x.size else 0.0
    return np.float32(rn32(amax / TENSOR_DIVISOR))


def quantize(x, s_t=None):
    """Quantize a [rows, cols] binary32 tensor to NVFP4.

    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16],
    s_t float32).  bfloat16 inputs are passed as their exact float32 values.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 16")
    if s_t is None:
        s_t = tensor_scale(x)
    s_t = np.float32(s_t)
    d = rn32(6.0 * np.float64(s_t))                                  # step 3

    g = x.reshape(rows, cols // GROUP, GROUP)
    a_g = np.max(np.abs(g), axis=2).astype(np.float64)               # step 4
    if d == 0:
        s_code = np.zeros(a_g.shape, dtype=np.uint8)
    else:
        s_code = enc_e4m3(rn32(a_g / np.float64(d)))
    s_val = dec_e4m3(s_code)

    p = rn32(s_val * np.float64(s_t)).astype(np.float64)             # step 5
    safe_p = np.where(p == 0, 1.0, p)
    inv = np.where(p == 0, 0.0, rn32(1.0 / safe_p).astype(np.float64))
    y = rn32(g.astype(np.float64) * inv[:, :, None])
    c = enc_e2m1(y)
    sign_only = (np.signbit(g).astype(np.uint8) << 3)
    c = np.where((p == 0)[:, :, None], sign_only, c).reshape(rows, cols)

    codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)       # step 6
    return codes, s_code.astype(np.uint8), np.float32(s_t)


def unpack_codes(codes):
    """[rows, cols/2] packed bytes -> [rows, cols] 4-bit codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def dequantize(codes, scales, s_t):
    """Step 7: exact float64 values of an NVFP4 tensor."""
    c = unpack_codes(codes)
    rows, cols = c.shape
    s = np.repeat(dec_e4m3(scales), GROUP, axis=1)
    return dec_e2m1(c) * s * np.float64(np.float32(s_t))

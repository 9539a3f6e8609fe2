"""Symmetric INT4 weight quantizer, 128-element groups (oracle; test infrastructure).

Source: the MARLIN article (abeam.tech), section "データの扱い方" (how data is
handled): 4-bit weights with a group size of 128 along the input dimension,
consumed by an FP16-activation x INT4-weight kernel (section "どんな技術か").
The pages quantize with GPTQ; calibration is out of scope here, so weights are
quantized by plain round-to-nearest with a symmetric per-group scale equal to
the group's absolute maximum divided by 7, stored as bfloat16.

Reading of the unspecified details:
* s = bf16(rn32(a / 7)) with a = max |w| over the group (double rounding:
  real -> binary32 -> bfloat16, both to nearest even).
* q = clamp(round_half_even(rn32(w / s)), -7, 7); the division uses the
  stored bfloat16 scale.  -8 is never produced.  If s == 0 every q is 0.
* Storage: u = q + 8 (1..15), two per byte, even column in the low nibble;
  scales are bfloat16 bit patterns laid out [n, k/128].
* Dequantization: w_hat = q * s (exact in float64).
"""

import numpy as np

from .formats import rn32, rn_bf16_bits, bf16_bits_to_f32

GROUP = 128


def quantize(w):
    """Quantize fp32 weights [n, k] -> (codes uint8 [n, k/2], scales uint16 [n, k/128])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % GROUP:
        raise ValueError("k must be a multiple of 128")
    g = w.reshape(n, k // GROUP, GROUP).astype(np.float64)
    a = np.max(np.abs(g), axis=2)
    s_bits = rn_bf16_bits(rn32(a / 7.0))
    s = bf16_bits_to_f32(s_bits).astype(np.float64)
    safe = np.where(s == 0, 1.0, s)
    r = rn32(g / safe[:, :, None]).astype(np.float64)
    q = np.clip(np.rint(r), -7, 7)
    q = np.where((s == 0)[:, :, None], 0.0, q).astype(np.int64).reshape(n, k)
    u = (q + 8).astype(np.uint8)
    codes = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    return codes, s_bits.astype(np.uint16)


def unpack(codes):
    """Packed codes [n, k/2] -> signed integers q [n, k]."""
    codes = np.asarray(codes, dtype=np.uint8)
    u = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.int64)
    u[:, 0::2] = codes & 0xF
    u[:, 1::2] = codes >> 4
    return u - 8


def dequantize(codes, scales):
    """Exact float64 weights q * s."""
    q = unpack(codes).astype(np.float64)
    s = bf16_bits_to_f32(scales).astype(np.float64)
    return q * np.repeat(s, GROUP, axis=1)

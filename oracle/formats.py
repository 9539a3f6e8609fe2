"""Number formats used by the quantized linear layer (oracle; test infrastructure).

Sources
-------
* NVFP4 is a 4-bit floating-point element format with a local scale per
  16-element group and one tensor-level scale (Mix-Quant technical summary,
  gist.science, section 2 "Method", hybrid-precision bullet on prefill).  The
  pages do not print the bit layouts.
* E2M1 element and E4M3 scale layouts follow the public OCP specifications:
  OCP Microscaling Formats (MX) v1.0, element type FP4 (E2M1); OCP 8-bit
  Floating Point (OFP8) v1.0, E4M3 (the "FN" variant: no infinities, one NaN
  mantissa pattern, maximum 448).
* bfloat16 is the top 16 bits of binary32; conversion rounds to nearest even.

Every function here works on numpy arrays and is written for clarity, not speed.
"""

import numpy as np

# ---------------------------------------------------------------------------
# binary32 / bfloat16 rounding
# ---------------------------------------------------------------------------


def rn32(v):
    """Round float64 value(s) to binary32, ties to even (IEEE 754 default)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def f32_bits(v):
    return np.asarray(v, dtype=np.float32).view(np.uint32)


def bits_f32(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def rn_bf16_bits(v):
    """bfloat16 bit patterns (uint16) of binary32 value(s), round to nearest even.

    Finite inputs only.  bfloat16 keeps the sign, the 8 exponent bits and the
    top 7 mantissa bits; the dropped 16 bits are rounded half-to-even on the
    integer bit pattern, which carries into the exponent when needed.
    """
    u = f32_bits(v).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(h):
    """Exact binary32 value(s) of bfloat16 bit patterns."""
    return bits_f32(np.asarray(h, dtype=np.uint32) << 16)


def rn_bf16(v):
    """Round binary32 value(s) to bfloat16 and return them as float32."""
    return bf16_bits_to_f32(rn_bf16_bits(v))


# ---------------------------------------------------------------------------
# E2M1 (FP4) element format
# ---------------------------------------------------------------------------
# Layout s e1 e0 m, exponent bias 1.  Codes 0..7 are the magnitudes below;
# code | 8 is the negative of the same magnitude (code 8 is -0).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def dec_e2m1(codes):
    """Values (float64) of 4-bit E2M1 codes."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def enc_e2m1(y):
    """Encode binary32 value(s) to E2M1 codes: round to nearest, ties to even.

    The magnitude is placed on the grid {0, .5, 1, 1.5, 2, 3, 4, 6} by
    comparing against the midpoints between neighbours; at an exact midpoint
    the code with an even mantissa bit (the even code) wins.  Magnitudes above
    6 saturate to 6 (there is no infinity).  The sign bit is copied from the
    input, so a negative value that rounds to zero encodes as 0b1000.
    NaN inputs are outside the method's domain.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    grid = E2M1_MAGNITUDES
    code = np.zeros(a.shape, dtype=np.int64)
    for i in range(7):
        lo, hi = grid[i], grid[i + 1]
        mid = (lo + hi) / 2.0  # exact: at most 3 significant bits
        # the upper neighbour wins above the midpoint, and at the midpoint when
        # its code (i + 1) is even
        up = (a > mid) | ((a == mid) & ((i + 1) % 2 == 0))
        code = np.where(up, i + 1, code)
    sign = np.signbit(y).astype(np.int64)
    return (code | (sign << 3)).astype(np.uint8)


# ---------------------------------------------------------------------------
# E4M3 (OCP E4M3FN) scale format
# ---------------------------------------------------------------------------
# Layout s e3 e2 e1 e0 m2 m1 m0, exponent bias 7.  Normal values are
# 2^(e-7) * (1 + m/8) for e = 1..15 (except the NaN pattern e=15, m=7);
# subnormals are m * 2^-9.  Largest finite value 448 (0x7E).


def dec_e4m3(codes):
    """Values (float64) of E4M3 bytes; 0x7F / 0xFF give NaN."""
    b = np.asarray(codes).astype(np.int64)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where((b & 0x80) != 0, -mag, mag)


# The 127 non-negative finite E4M3 values in code order (codes 0x00..0x7E);
# they are increasing, so code order is value order.
_E4M3_GRID = dec_e4m3(np.arange(0x7F))


def enc_e4m3(q):
    """Encode non-negative binary32 value(s) to E4M3 bytes.

    Round to nearest, ties to even code; values at or above 448 saturate to
    0x7E (448).  Only non-negative inputs occur in the method (group scales are
    ratios of magnitudes).
    """
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    if np.any(q < 0) or np.any(np.isnan(q)):
        raise ValueError("enc_e4m3 expects non-negative, non-NaN inputs")
    grid = _E4M3_GRID
    # index of the first grid value >= q (clamped to the last value)
    hi = np.searchsorted(grid, np.minimum(q, grid[-1]), side="left")
    lo = np.maximum(hi - 1, 0)
    g_lo, g_hi = grid[lo], grid[hi]
    mid = (g_lo + g_hi) / 2.0  # exact in float64
    pick_hi = (q > mid) | ((q == mid) & (hi % 2 == 0))
    code = np.where(hi == lo, hi, np.where(pick_hi, hi, lo))
    code = np.where(q >= grid[-1], 0x7E, code)
    return code.astype(np.uint8)

"""Exact-rational brute-force references used to pin the oracle.

Everything here works on ``fractions.Fraction`` and Python integers, so it
shares no mechanism with the oracle (which evaluates binary32 steps in
float64 and rounds with numpy).  Grids are enumerated from the OCP format
definitions directly (value = 2^(e-bias) * (1 + m/2^mbits), subnormals
m * 2^(1-bias-mbits)).
"""

from fractions import Fraction
import struct


def f32_to_frac(x):
    """Exact rational value of a Python float that holds a binary32 value."""
    return Fraction(float(x))


def frac_to_f32(q):
    """Round a rational to binary32, nearest-even, by integer arithmetic.

    Returns a Python float holding the binary32 value (inf on overflow).
    """
    q = Fraction(q)
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # subnormals share the quantum 2^-149
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = Fraction(fl) * quantum
    if v >= Fraction(2) ** 128:
        r = float("inf")
    else:
        r = float(v)                       # exact: v has <= 24 significant bits
    # sanity: the result must be a binary32 value
    assert r == struct.unpack("f", struct.pack("f", r))[0] or r == float("inf")
    return -r if neg else r


def e2m1_grid():
    """Non-negative E2M1 values by code 0..7 (bias 1, one mantissa bit)."""
    out = []
    for e in range(4):
        for m in range(2):
            if e == 0:
                out.append(Fraction(m, 2))
            else:
                out.append(Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)))
    return out


def e4m3_grid():
    """Non-negative finite E4M3 values by code 0x00..0x7E (bias 7, three mantissa bits)."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            out.append(Fraction(m, 8) * Fraction(2) ** -6)
        else:
            out.append(Fraction(2) ** (e - 7) * (1 + Fraction(m, 8)))
    return out


def nearest_code(value, grid):
    """Nearest grid code to a non-negative rational, ties to the even code,
    saturating at the last grid value."""
    value = Fraction(value)
    if value >= grid[-1]:
        return len(grid) - 1
    best, best_d = 0, abs(value - grid[0])
    for c in range(1, len(grid)):
        d = abs(value - grid[c])
        if d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


E2M1 = e2m1_grid()
E4M3 = e4m3_grid()


def nvfp4_quantize_exact(rows):
    """Brute-force NVFP4 quantizer on a list of rows of binary32 floats.

    Same reading as the oracle (each binary32 step rounded once), computed
    with rationals and integer rounding.  Returns (codes [r][c], scales
    [r][c/16], s_t float).
    """
    amax = max(abs(f32_to_frac(v)) for row in rows for v in row)
    s_t = frac_to_f32(amax / 2688)
    d = frac_to_f32(6 * Fraction(s_t))
    codes, scales = [], []
    for row in rows:
        crow, srow = [], []
        for g0 in range(0, len(row), 16):
            grp = row[g0:g0 + 16]
            a_g = max(abs(f32_to_frac(v)) for v in grp)
            if d == 0:
                sc = 0
            else:
                sc = nearest_code(Fraction(frac_to_f32(a_g / Fraction(d))), E4M3)
            srow.append(sc)
            p = frac_to_f32(E4M3[sc] * Fraction(s_t))
            for v in grp:
                sign = 1 if (v < 0 or (v == 0 and struct.pack("f", v)[3] & 0x80)) else 0
                if p == 0:
                    crow.append(sign << 3)
                    continue
                inv = frac_to_f32(1 / Fraction(p))
                y = frac_to_f32(f32_to_frac(v) * Fraction(inv))
                crow.append(nearest_code(abs(Fraction(y)), E2M1) | (sign << 3))
        codes.append(crow)
        scales.append(srow)
    return codes, scales, s_t

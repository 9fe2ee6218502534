"""Exact number-format codecs for the oracle (bf16, FP4 E2M1, FP8 E4M3).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FP4 main KV cache stores every latent value as an E2M1 code with one
E4M3 scale per 16 channels and no second, global scale [P1 section
效率组件四件, item 4 "FP4 主 KV Cache"; P4, the CSA2 paragraph].  The pages
name the formats only; the bit-level definitions below are the standard ones:

* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/NaN.
  Magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E4M3 (the OCP "E4M3FN" variant used by NVFP4-style block scaling, which
  the pages name as the model for this cache): 1 sign bit, 4 exponent bits
  (bias 7), 3 mantissa bits, subnormal quantum 2^-9, largest finite 448
  (0x7E), 0x7F / 0xFF are NaN, no infinities.
* bf16: the upper 16 bits of an IEEE binary32.

Encoders are brute force over the finite code points ("nearest value, ties to
the even code"), which is the plain definition of round-to-nearest-even for a
small format.  Distances are formed in float64; the comments at each encoder
say why that is exact where it matters.
"""

import numpy as np

# ---------------------------------------------------------------- bf16


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 / int16 array) -> float64 values, exactly.

    A bf16 value is the binary32 whose upper half is the pattern and whose
    lower half is zero; binary32 -> float64 is exact.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits_exact(x):
    """float64 values that are exactly representable in bf16 -> bit patterns.

    Raises if any value would need rounding: the oracle only ever converts
    values it knows to be bf16-exact (test fixtures).
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x, equal_nan=True):
        raise ValueError("value not representable in binary32")
    u = f.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("value not representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- E2M1


def e2m1_decode(codes):
    """4-bit E2M1 codes (0..15) -> float64 values (sign kept, -0 for 0x8)."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    # subnormal (e == 0): m * 0.5 ; normal: 2^(e-1) * (1 + m/2)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.copysign(mag, np.where(s == 1, -1.0, 1.0))


# magnitude of each 3-bit E2M1 magnitude code, from the decoder above
def _e2m1_grid():
    return e2m1_decode(np.arange(8))


def e2m1_encode_magnitude(y_abs, sigma):
    """Magnitude code (0..7) of |x| for block scale ``sigma``.

    The code is the E2M1 magnitude nearest to |x| / sigma, ties to the even
    code, saturating at 6 (code 7).  sigma == 0 gives code 0.

    Distances are |sigma * g - |x||: sigma * g is exact (<= 6 significant
    bits), |x| is a bf16 value, and when |x| < 6 * sigma the two operands of
    every subtraction that can decide the minimum are within a few binades of
    each other, so the float64 difference is exact.  |x| >= 6 * sigma is the
    saturating branch and is taken before any distance is compared.
    """
    y = np.asarray(y_abs, dtype=np.float64)
    sg = np.broadcast_to(np.asarray(sigma, dtype=np.float64), y.shape)
    grid = _e2m1_grid()                                   # [8]
    d = np.abs(sg[..., None] * grid - y[..., None])       # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    is_min = d == best
    # among the (at most two, adjacent) minimisers prefer the even code
    even = (np.arange(8) % 2) == 0
    pick_even = np.any(is_min & even, axis=-1)
    code_even = np.argmax(is_min & even, axis=-1)
    code_any = np.argmax(is_min, axis=-1)
    code = np.where(pick_even, code_even, code_any)
    code = np.where(y >= 6.0 * sg, 7, code)
    code = np.where(sg == 0.0, 0, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- E4M3


def e4m3_decode(codes):
    """8-bit E4M3FN codes -> float64 values (0x7F / 0xFF -> NaN)."""
    b = np.asarray(codes).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.copysign(mag, np.where(s == 1, -1.0, 1.0))


def _e4m3_nonneg_values():
    """Values of the 127 non-negative finite codes 0x00..0x7E, increasing."""
    return e4m3_decode(np.arange(127))


def _nearest_even_code(dist):
    """Index of the smallest distance along the last axis, ties -> even index."""
    best = dist.min(axis=-1, keepdims=True)
    is_min = dist == best
    n = dist.shape[-1]
    even = (np.arange(n) % 2) == 0
    pick_even = np.any(is_min & even, axis=-1)
    return np.where(pick_even, np.argmax(is_min & even, axis=-1), np.argmax(is_min, axis=-1))


def e4m3_encode(t):
    """Non-negative reals (float64, taken as exact) -> E4M3 code, RNE, saturating.

    Nearest finite E4M3 value, ties to the even code (= even mantissa), values
    above 448 saturate to 0x7E.  Used by the pins against torch's cast.
    """
    t = np.asarray(t, dtype=np.float64)
    if np.any(t < 0) or np.any(np.isnan(t)):
        raise ValueError("e4m3_encode takes non-negative, non-NaN values")
    out = np.empty(t.shape, dtype=np.uint8)
    vals = _e4m3_nonneg_values()
    flat_t = t.reshape(-1)
    flat_o = out.reshape(-1)
    for lo in range(0, flat_t.size, 1 << 15):
        tt = flat_t[lo:lo + (1 << 15)]
        code = _nearest_even_code(np.abs(vals[None, :] - tt[:, None]))
        code = np.where(tt >= 448.0, 126, code)
        flat_o[lo:lo + (1 << 15)] = code
    return out


def e4m3_scale_code_for_amax(amax):
    """Block-scale code for a group whose largest magnitude is ``amax``.

    The scale is the E4M3 value nearest to amax / 6 (6 = largest E2M1
    magnitude, so the largest element lands on the top of the FP4 grid), ties
    to the even code, saturating at 448 (0x7E); the sign bit is 0.

    Distances are |6 * v - amax| so no division is rounded: 6 * v is exact
    (<= 6 significant bits), amax is a bf16 value, and below the saturation
    point (amax < 6 * 448) the deciding subtractions are exact in float64.
    """
    a = np.asarray(amax, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint8)
    vals6 = 6.0 * _e4m3_nonneg_values()
    flat_a = a.reshape(-1)
    flat_o = out.reshape(-1)
    for lo in range(0, flat_a.size, 1 << 15):
        aa = flat_a[lo:lo + (1 << 15)]
        code = _nearest_even_code(np.abs(vals6[None, :] - aa[:, None]))
        code = np.where(aa >= 6.0 * 448.0, 126, code)
        flat_o[lo:lo + (1 << 15)] = code
    return out

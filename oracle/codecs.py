"""Number codecs of the oracle: BF16 and OCP FP8 E4M3, written from their definitions.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module.

Sources:
  * "Cloudflare quantizes Kimi and GLM caches for 41% faster inference", KV cache
    quantization paragraph: the KV cache is stored as FP8 "e4m3" instead of BF16.
  * The OCP 8-bit floating point format (OFP8) E4M3: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite
    value 448, smallest subnormal 2^-9.
  * BF16: the upper 16 bits of an IEEE binary32.

Readings taken where the pages are silent (listed in the design notes as well):
  * e4m3 means the OCP "fn" variant (max 448), not the FNUZ variant (max 240).
  * fp32 -> e4m3 rounds to nearest, ties to even; magnitudes above 448 saturate
    to 448; the sign survives underflow (-tiny -> 0x80); NaN -> 0x7F.

Every routine works on numpy arrays and is vectorised only over elements; the
arithmetic is exact (fp64 holds every fp32 and every e4m3 value exactly, and
scaling by a power of two is exact).
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


# ---------------------------------------------------------------- bf16
def bf16_to_f64(bits):
    """BF16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_from_f32_rne(x):
    """float32 values -> BF16 bit patterns, round to nearest, ties to even.

    The 16 dropped bits are compared against one half of the kept LSB; NaN maps
    to the canonical quiet NaN 0x7FC0 (sign kept).
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    round_up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    out = (hi + round_up.astype(np.uint64)).astype(np.uint32)
    nan = np.isnan(f)
    out = np.where(nan, (hi & np.uint64(0x8000)).astype(np.uint32) | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


# ---------------------------------------------------------------- e4m3
def _e4m3_table():
    """Value of each of the 256 codes (fp64); NaN for the two NaN codes."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if (c & 0x80) else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:                       # subnormal: m/8 * 2^(1-7)
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:                              # normal: (1 + m/8) * 2^(e-7)
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_to_f64(codes):
    """e4m3 codes (uint8) -> float64, exact."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_from_f32_rne_sat(x):
    """float32 values -> e4m3 codes: saturate |v| > 448 to 448, then RNE.

    For a magnitude a (exact in fp64):
      * a < 2^-6 is in the subnormal range, spaced 2^-9: the code is the
        integer rint(a / 2^-9) in 0..8 (8 is the smallest normal 2^-6, whose
        code is also 0x08);
      * otherwise a = f * 2^k with f in [1, 2); the mantissa field is
        rint((f - 1) * 8), and a carry to 8 bumps the exponent.
    numpy's rint rounds halves to even.
    """
    f = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(f)
    a = np.abs(f)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    codes = np.zeros(a.shape, dtype=np.int64)

    sub = a < 2.0 ** -6
    codes[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)

    nrm = ~sub
    mant, expo = np.frexp(a[nrm])          # a = mant * 2^expo, mant in [0.5, 1)
    k = expo - 1                           # a = (2*mant) * 2^k, 2*mant in [1, 2)
    m = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    k = np.where(carry, k + 1, k)
    m = np.where(carry, 0, m)
    codes[nrm] = ((k + 7) << 3) | m

    codes = codes | np.where(neg, 0x80, 0)
    codes = np.where(nan, E4M3_NAN, codes)
    return codes.astype(np.uint8)

"""Pins for the oracle's number codecs (CPU only).

Each codec is tied to something other than its own formula: the OCP E4M3
reference points (tests/golden/e4m3_points.txt), torch's float8_e4m3fn and
bfloat16 conversions (library routines), and a brute-force nearest-value
search with the tie rule written as a search rule.
"""
import os

import numpy as np
import pytest
import torch

from oracle import (
    E4M3_VALUES,
    bf16_from_f32_rne,
    bf16_to_f64,
    e4m3_from_f32_rne_sat,
    e4m3_to_f64,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_points():
    pts = []
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            pts.append((int(c, 16), float(v)))
    return pts


def test_e4m3_decode_golden_points():
    for code, val in _golden_points():
        got = e4m3_to_f64(np.uint8(code))
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert nan.sum() == 2  # 0x7F and 0xFF only


def test_e4m3_positive_codes_monotone_and_distinct():
    v = E4M3_VALUES[:0x7F]
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 448.0 and v[1] == 2.0 ** -9


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3_to_f64(codes).astype(np.float32)
    assert np.array_equal(e4m3_from_f32_rne_sat(vals), codes)


def _brute_force_e4m3(x32):
    """Nearest finite code of the same sign; ties -> even code; |x| > 448 -> 448."""
    x = x32.astype(np.float64)
    out = np.empty(x.shape, np.uint8)
    pos_codes = np.arange(0, 0x7F)                 # 0x00 .. 0x7E
    pos_vals = E4M3_VALUES[pos_codes]
    a = np.minimum(np.abs(x), 448.0)
    for lo in range(0, x.size, 1 << 16):
        aa = a[lo:lo + (1 << 16)]
        d = np.abs(aa[:, None] - pos_vals[None, :])
        best = d.min(axis=1, keepdims=True)
        is_best = d == best
        n_best = is_best.sum(axis=1)
        first = np.argmax(is_best, axis=1)
        # a tie has exactly two neighbours: take the one with an even code
        tie = n_best == 2
        pick = first.copy()
        pick[tie] = np.where(first[tie] % 2 == 0, first[tie], first[tie] + 1)
        out[lo:lo + (1 << 16)] = pos_codes[pick]
    neg = np.signbit(x)
    return (out | np.where(neg, 0x80, 0)).astype(np.uint8)


def _test_values(rng):
    # random fp32 bit patterns spanning 2^-14 .. 2^10, both signs
    exps = rng.integers(127 - 14, 127 + 10, size=600_000)
    mant = rng.integers(0, 1 << 23, size=600_000)
    sign = rng.integers(0, 2, size=600_000)
    bits = (sign << 31) | (exps << 23) | mant
    r = bits.astype(np.uint32).view(np.float32)
    # exact midpoints between neighbouring codes and their fp32 neighbours
    v = E4M3_VALUES[:0x7F]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    around = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                             np.nextafter(mids, np.float32(0))])
    special = np.array([0.0, -0.0, 448.0, 449.0, 464.0, 465.0, 1e30, -1e30,
                        2.0 ** -10, -2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 1e-30, -1e-30,
                        np.float32(np.finfo(np.float32).tiny)], np.float32)
    allv = np.concatenate([r, around, -around, special, np.tile(special, 1)]).astype(np.float32)
    return np.concatenate([allv, rng.standard_normal(400_000).astype(np.float32) * 100])


def test_e4m3_encode_matches_brute_force():
    rng = np.random.default_rng(123)
    x = _test_values(rng)
    assert x.size >= 1_000_000
    got = e4m3_from_f32_rne_sat(x)
    ref = _brute_force_e4m3(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_e4m3_encode_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn rounds to nearest even; it returns NaN instead
    # of saturating at |x| >= 464, so compare only |x| <= 448.
    rng = np.random.default_rng(7)
    x = _test_values(rng)
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3_from_f32_rne_sat(x)
    assert np.array_equal(got, ref)


def test_e4m3_special_readings():
    enc = lambda v: int(e4m3_from_f32_rne_sat(np.array([v], np.float32))[0])  # noqa: E731
    assert enc(1e9) == 0x7E and enc(-1e9) == 0xFE          # saturation
    assert enc(-1e-30) == 0x80 and enc(1e-30) == 0x00      # sign kept on underflow
    assert enc(2.0 ** -10) == 0x00                         # tie to even (0)
    assert enc(3 * 2.0 ** -10) == 0x02                     # tie 1.5 ulp -> 2 (even)
    assert enc(float("nan")) == 0x7F


def _brute_force_bf16(x32):
    """Nearest bf16 by searching the two truncation neighbours; ties -> even."""
    u = x32.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)
    hi = lo + 1
    vlo = bf16_to_f64(lo.astype(np.uint16))
    vhi = bf16_to_f64(hi.astype(np.uint16))
    x = x32.astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def test_bf16_encode_matches_brute_force_and_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    exps = (bits >> 23) & 0xFF
    x = bits[(exps > 0) & (exps < 254)].view(np.float32)           # finite, away from overflow
    ties = ((rng.integers(0, 2 ** 16, 1000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], rng.standard_normal(10000).astype(np.float32)])
    got = bf16_from_f32_rne(x)
    assert np.array_equal(got, _brute_force_bf16(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_decode_known_values():
    assert bf16_to_f64(np.uint16(0x3F80)) == 1.0
    assert bf16_to_f64(np.uint16(0xC000)) == -2.0
    assert bf16_to_f64(np.uint16(0x3E00)) == 0.125
    assert np.isnan(bf16_to_f64(np.uint16(0x7FC0)))


@pytest.mark.parametrize("v", [0.1, -3.3, 1e-3, 300.0])
def test_bf16_encode_is_within_half_ulp(v):
    b = bf16_from_f32_rne(np.array([v], np.float32))[0]
    back = bf16_to_f64(b)
    ulp = 2.0 ** (np.floor(np.log2(abs(v))) - 7)
    assert abs(back - np.float32(v)) <= ulp / 2

"""Pins of the oracle's 4-bit float block product (e2m1 elements, one E8M0
scale per 32 k) -- the 4-bit float block format the specialised-runtime spec
("spec: specialized model runtimes", section "Target package and artifact")
puts after groupwise-int weights, read as the public microscaling definition
with 32-element blocks.  CPU only.

The pages print no values for it.  What pins it:
  * E8M0 scales: all 256 bytes against torch's float8_e8m0fnu decoding (an
    independent implementation);
  * e2m1 elements: the properties that single the format out -- 8 distinct
    magnitudes from 0 to 6 with smallest positive 0.5, magnitude increasing
    with the code, the sign in bit 3, and the exponent step doubling the
    value -- which a mistaken bias, sign bit or mantissa weight breaks;
  * closed forms, exact rational brute force on small tiles, and a float64
    library matmul of the dequantised weights.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic


def test_e8m0_matches_torch_decoding():
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0_value(int(b)) for b in bits])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0


def test_e2m1_element_set():
    v = np.array([oracle.e2m1_value(c) for c in range(16)])
    pos = v[:8]
    assert pos[0] == 0.0 and not np.signbit(pos[0])
    assert np.all(np.diff(pos) > 0)                      # magnitude grows with the code
    assert pos[1] == 0.5 and pos[7] == 6.0               # smallest positive, largest
    assert len(set(pos.tolist())) == 8
    # sign in bit 3, magnitude in bits 2..0
    assert np.array_equal(v[8:], -pos) and np.signbit(v[8])
    # codes 2e + m for e >= 1: one exponent step doubles the value
    for e in (1, 2):
        for m in (0, 1):
            assert pos[2 * (e + 1) + m] == 2 * pos[2 * e + m]
    # the mantissa bit adds half of the exponent's power, in the subnormal
    # range too (0 -> 0.5 is that half of 1.0)
    assert pos[3] - pos[2] == 0.5 and pos[1] - pos[0] == 0.5


def test_dequant_and_library_matmul():
    c = synthetic.mx_case(11, 3, 40, 192)
    w = oracle.mx_dequant(c.w_q, c.w_e)
    e2 = np.array([oracle.e2m1_value(k) for k in range(16)])
    # nibble order: k = 2j is the low nibble of byte j
    lo, hi = c.w_q & 0x0F, c.w_q >> 4
    codes = np.empty((40, 192), dtype=np.int64)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    sc = np.ldexp(1.0, c.w_e.astype(np.int64) - 127)
    assert np.array_equal(w, e2[codes] * np.repeat(sc, 32, axis=1))
    y, t = oracle.mx_matmul(c.x, c.w_q, c.w_e)
    xf = (c.x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = xf @ w.T
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(xf) @ np.abs(w).T) + 1e-300)
    assert np.allclose(t, np.abs(xf) @ np.abs(w).T, rtol=1e-12, atol=0)


def test_closed_forms():
    K, N = 256, 3
    x = np.full((1, K), 0x3FC0, dtype=np.uint16)          # 1.5
    w_q = np.full((N, K // 2), 0x77, dtype=np.uint8)      # element 7 = 6.0
    w_e = np.full((N, K // 32), 125, dtype=np.uint8)      # 2^-2
    y, t = oracle.mx_matmul(x, w_q, w_e)
    assert np.all(y == K * 1.5 * 6.0 * 0.25) and np.all(t == y)
    w_q[:] = 0xF9                                         # elements -0.5 (even k), -6 (odd k)
    y, t = oracle.mx_matmul(x, w_q, w_e)
    assert np.all(y == (K // 2) * 1.5 * (-0.5 - 6.0) * 0.25)
    w_q[:] = 0x08                                         # +0 and -0
    y, t = oracle.mx_matmul(x, w_q, w_e)
    assert np.all(y == 0) and np.all(t == 0)
    w_q[:] = 0x22
    w_e[:, 1] = 255                                       # one NaN scale poisons the row
    y, _ = oracle.mx_matmul(x, w_q, w_e)
    assert np.all(np.isnan(y))


def test_exact_rational_brute_force():
    c = synthetic.mx_case(12, 4, 6, 64, e_lo=100, e_hi=140)
    y, t = oracle.mx_matmul(c.x, c.w_q, c.w_e)

    def frac_bf16(b):
        f = float((np.uint32(b) << np.uint32(16)).view(np.float32))
        return Fraction(f)

    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
           Fraction(4), Fraction(6)]
    for m in range(4):
        for n in range(6):
            acc, ab = Fraction(0), Fraction(0)
            for k in range(64):
                byte = int(c.w_q[n, k // 2])
                code = byte & 15 if k % 2 == 0 else byte >> 4
                wv = (-1 if code & 8 else 1) * mag[code & 7] * Fraction(2) ** (int(c.w_e[n, k // 32]) - 127)
                p = frac_bf16(c.x[m, k]) * wv
                acc += p
                ab += abs(p)
            assert abs(Fraction(y[m, n]) - acc) <= 64 * Fraction(2) ** -52 * ab
            assert abs(Fraction(t[m, n]) - ab) <= 64 * Fraction(2) ** -52 * ab


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.mx_matmul(np.zeros((1, 64), np.uint16), np.zeros((2, 32), np.uint8),
                         np.zeros((2, 3), np.uint8))
    with pytest.raises(ValueError):
        oracle.mx_matmul(np.zeros((1, 32), np.uint16), np.zeros((2, 32), np.uint8),
                         np.zeros((2, 2), np.uint8))

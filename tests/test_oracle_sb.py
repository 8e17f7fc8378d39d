"""Pins of the oracle's super-block (two-level) scale format, CPU only:
w[n,k] = (c[n,k] - 8) * d[n, k/256] * sc[n, k/32], with fp16 d and unsigned
8-bit sc -- the two-level block-scale structure of the K-quant profiles the
layer-package spec names, on this library's codes.  Pinned against the base
format (when d * sc is an fp16 value the two must agree exactly), exact
rational brute force, closed forms and a numpy float64 product."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def test_agrees_with_the_base_format():
    """d with at most 3 significant bits and sc < 32 keep d * sc an fp16
    value: the base format with s = d * sc gives the same result bit for bit."""
    rng = np.random.default_rng(40)
    M, N, K = 3, 50, 512
    c = synthetic.sb_case(41, M, N, K)
    d = np.ldexp(rng.integers(4, 8, size=(N, K // 256)).astype(np.float64),
                 rng.integers(-12, -8, size=(N, K // 256)))
    w_d = d.astype(np.float16).view(np.uint16)
    w_sc = rng.integers(0, 32, size=(N, K // 32)).astype(np.uint8)
    s = np.repeat(d, 8, axis=1) * w_sc
    w_s = s.astype(np.float16)
    assert np.array_equal(w_s.astype(np.float64), s)
    y, t = oracle.sb_matmul(c.x, c.w_q, w_d, w_sc)
    yb, tb = oracle.matmul(c.x, c.w_q, w_s.view(np.uint16))
    assert np.array_equal(y, yb) and np.array_equal(t, tb)
    assert np.array_equal(oracle.sb_dequant(c.w_q, w_d, w_sc),
                          oracle.dequant_f32(c.w_q, w_s.view(np.uint16)).astype(np.float64))


def test_exact_rational_brute_force():
    c = synthetic.sb_case(42, 2, 4, 256)
    y, t = oracle.sb_matmul(c.x, c.w_q, c.w_d, c.w_sc)
    xf = (c.x.astype(np.uint32) << 16).view(np.float32)
    for m in range(2):
        for n in range(4):
            acc = Fraction(0)
            for k in range(256):
                byte = int(c.w_q[n, k // 2])
                code = byte & 15 if k % 2 == 0 else byte >> 4
                w = Fraction(code - 8) * Fraction(float(_f16(c.w_d[n, k // 256]))) \
                    * int(c.w_sc[n, k // 32])
                acc += Fraction(float(xf[m, k])) * w
            assert abs(y[m, n] - float(acc)) <= 256 * 2.0 ** -53 * t[m, n]


def test_closed_forms():
    K, N = 512, 6
    x = np.full((2, K), 0x3FC0, np.uint16)                       # 1.5
    w_q = np.full((N, K // 2), 0xDD, np.uint8)                    # code 13: +5
    w_d = np.full((N, K // 256), np.float16(2.0 ** -6).view(np.uint16), np.uint16)
    w_sc = np.full((N, K // 32), 3, np.uint8)
    y, _ = oracle.sb_matmul(x, w_q, w_d, w_sc)
    assert np.all(y == K * 1.5 * 5 * 3 * 2.0 ** -6)
    w_sc[:, ::2] = 0                                              # half the blocks off
    y, t = oracle.sb_matmul(x, w_q, w_d, w_sc)
    assert np.all(y == K / 2 * 1.5 * 5 * 3 * 2.0 ** -6)
    w_sc[:] = 0
    y, t = oracle.sb_matmul(x, w_q, w_d, w_sc)
    assert np.all(y == 0) and np.all(t == 0)


def test_against_numpy_float64():
    c = synthetic.sb_case(43, 5, 70, 1024)
    y, t = oracle.sb_matmul(c.x, c.w_q, c.w_d, c.w_sc)
    lo, hi = (c.w_q & 15).astype(np.int64), (c.w_q >> 4).astype(np.int64)
    codes = np.empty((70, 1024), np.int64)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    w = (codes - 8) * np.repeat(_f16(c.w_d), 256, axis=1) * np.repeat(c.w_sc.astype(np.float64), 32, axis=1)
    assert np.array_equal(oracle.sb_dequant(c.w_q, c.w_d, c.w_sc), w)
    xf = (c.x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(y - xf @ w.T) <= 1e-12 * t)


def test_shape_errors():
    c = synthetic.sb_case(44, 1, 4, 256)
    with pytest.raises(ValueError):
        oracle.sb_matmul(c.x, c.w_q, c.w_d[:, :0], c.w_sc)
    with pytest.raises(ValueError):
        synthetic.sb_case(45, 1, 4, 288)

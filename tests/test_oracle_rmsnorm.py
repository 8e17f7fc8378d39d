"""Pins of the oracle's RMSNorm prologue (CPU only).

The pages name "one quantized GEMM plus fused RMSNorm" as the first measured
kernel ("spec: specialized model runtimes", "Feasibility gate") without
defining RMSNorm; the oracle takes the usual definition
    x'[m,k] = x[m,k] * gamma[k] / sqrt(mean_k x[m,k]^2 + eps)
and these tests pin it against closed forms, exact powers-of-two invariants,
a 60-digit decimal evaluation, and numpy's float64 product."""
from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic

BF16_ONE = 0x3F80


def bf16(v: float) -> int:
    return int(synthetic.f32_to_bf16_bits(np.array([v], np.float32))[0])


def bf16_value(b: int) -> float:
    return float(np.array([b << 16], np.uint32).view(np.float32)[0])


def test_constant_row_normalises_to_its_sign():
    K = 64
    for a in (1.5, -3.0, 0.0078125, 1e30):
        x = np.full((1, K), bf16(a), np.uint16)
        g = np.full(K, BF16_ONE, np.uint16)
        xn = oracle.rmsnorm(x, g, 0.0)
        assert np.allclose(xn, np.sign(bf16_value(bf16(a))), rtol=2e-16, atol=0)


def test_constant_row_with_eps():
    K, a, eps = 32, 0.5, 0.25
    x = np.full((2, K), bf16(a), np.uint16)
    g = np.full(K, BF16_ONE, np.uint16)
    xn = oracle.rmsnorm(x, g, eps)
    assert np.allclose(xn, a / np.sqrt(a * a + eps), rtol=1e-15, atol=0)


def test_one_hot_row_and_its_product():
    K, N, j, a, eps = 256, 40, 77, 3.0, 1e-6
    d = synthetic.dense_case(11, 1, N, K)
    x = np.zeros((1, K), np.uint16)
    x[0, j] = bf16(a)
    g = synthetic.rms_case(12, 1, 1, K).gamma
    xn = oracle.rmsnorm(x, g, eps)
    expect = a / np.sqrt(a * a / K + eps) * bf16_value(int(g[j]))
    assert np.count_nonzero(xn) == 1
    assert xn[0, j] == pytest.approx(expect, rel=1e-15)
    y, t, u = oracle.rmsnorm_matmul(x, g, eps, d.w_q, d.w_s)
    w = oracle.dequant_f32(d.w_q, d.w_s).astype(np.float64)
    assert np.allclose(y[0], xn[0, j] * w[:, j], rtol=1e-15, atol=0)
    assert np.allclose(t[0], np.abs(xn[0, j] * w[:, j]), rtol=1e-15, atol=0)


def test_power_of_two_invariants():
    """eps = 0: scaling x by 2^e leaves x' unchanged bit for bit; doubling
    gamma doubles x' exactly."""
    c = synthetic.rms_case(13, 3, 1, 512)
    base = oracle.rmsnorm(c.x, c.gamma, 0.0)
    xf = (c.x.astype(np.uint32) << 16).view(np.float32)
    for e in (-20, 7):
        xs = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** e))
        assert np.array_equal(oracle.rmsnorm(xs, c.gamma, 0.0), base)
    gf = (c.gamma.astype(np.uint32) << 16).view(np.float32)
    g2 = synthetic.f32_to_bf16_bits(gf * np.float32(2.0))
    assert np.array_equal(oracle.rmsnorm(c.x, g2, 0.0), 2 * base)


def test_against_a_decimal_evaluation():
    """Sum of squares exactly (fractions), square root and products at 60
    digits: the double oracle agrees to a few units in the last place."""
    getcontext().prec = 60
    c = synthetic.rms_case(14, 2, 1, 160)
    eps = 1e-6
    xn = oracle.rmsnorm(c.x, c.gamma, eps)
    K = c.x.shape[1]
    for m in range(2):
        vals = [Fraction(bf16_value(int(b))) for b in c.x[m]]
        ms = sum(v * v for v in vals) / K + Fraction(eps)
        r = Decimal(1) / (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
        for k in range(K):
            exact = Decimal(float(vals[k])) * r * Decimal(bf16_value(int(c.gamma[k])))
            assert abs(float(exact) - xn[m, k]) <= 4e-16 * abs(float(exact)) + 1e-300


def test_product_against_numpy_float64():
    c = synthetic.rms_case(15, 5, 70, 640)
    y, t, u = oracle.rmsnorm_matmul(c.x, c.gamma, c.eps, c.w_q, c.w_s)
    xn = oracle.rmsnorm(c.x, c.gamma, c.eps)
    w = oracle.dequant_f32(c.w_q, c.w_s).astype(np.float64)
    assert np.all(np.abs(y - xn @ w.T) <= 1e-12 * t)
    assert np.allclose(t, np.abs(xn) @ np.abs(w).T, rtol=1e-12, atol=0)


def _half_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 2.0 ** -134)


def test_rounding_allowance():
    """u = sum_k hulp(x'_k) |w_k|, hulp from the bf16 format (8 significant
    bits): checked against a log2-based evaluation, and against the actual
    effect of rounding x' to bf16 (never larger than u)."""
    for v, h in ((1.0, 2.0 ** -8), (1.99, 2.0 ** -8), (2.0, 2.0 ** -7), (-0.75, 2.0 ** -9),
                 (2.0 ** -130, 2.0 ** -134)):
        assert oracle.bf16_half_ulp(v) == h
    c = synthetic.rms_case(16, 4, 50, 512)
    y, t, u = oracle.rmsnorm_matmul(c.x, c.gamma, c.eps, c.w_q, c.w_s)
    xn = oracle.rmsnorm(c.x, c.gamma, c.eps)
    w = oracle.dequant_f32(c.w_q, c.w_s).astype(np.float64)
    assert np.allclose(u, _half_ulp(xn) @ np.abs(w).T, rtol=1e-12, atol=0)
    xr = (synthetic.f32_to_bf16_bits(xn.astype(np.float32)).astype(np.uint32) << 16).view(np.float32)
    yr = xr.astype(np.float64) @ w.T
    # rounding through float32 first can add one float32 ulp per element
    assert np.all(np.abs(yr - y) <= u * (1 + 2.0 ** -15) + 1e-12 * t)


def test_sampled_equals_full():
    c = synthetic.rms_case(17, 6, 33, 320)
    y, t, u = oracle.rmsnorm_matmul(c.x, c.gamma, c.eps, c.w_q, c.w_s)
    ms = np.array([0, 5, 3, 5, 1])
    ns = np.array([0, 32, 17, 1, 9])
    ys, ts, us = oracle.rmsnorm_matmul_sampled(c.x, c.gamma, c.eps, c.w_q, c.w_s, ms, ns)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(ts, t[ms, ns])
    assert np.array_equal(us, u[ms, ns])


def test_shape_errors():
    c = synthetic.rms_case(18, 2, 4, 64)
    with pytest.raises(ValueError):
        oracle.rmsnorm(c.x, c.gamma[:-1], 1e-6)
    with pytest.raises(ValueError):
        oracle.rmsnorm_matmul(c.x[:, :32], c.gamma[:32], 1e-6, c.w_q, c.w_s)

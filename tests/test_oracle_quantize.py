"""Pins of the oracle's quantiser (bf16 weights -> 4-bit codes + fp16 block
scales), CPU only.

Reading (the pages name a convert step but no method): per 32-element block,
s = fp16(m / -8) with m the largest-magnitude element (first on ties), |s|
clamped to 65504; codes clamp(rint(w / s) + 8, 0, 15) with the quotient and
its rounding in fp32.  Pinned by: exact round trips of blocks the format
represents, sign and power-of-two symmetries, the error bound, special
blocks, and an independent numpy evaluation."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic


def bf16_bits(a):
    return synthetic.f32_to_bf16_bits(np.asarray(a, np.float32))


def bf16_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def _unpack(wq):
    lo, hi = wq & 0x0F, wq >> 4
    out = np.empty(wq.shape[:-1] + (wq.shape[-1] * 2,), np.int64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return out


def numpy_quantize(w_bits):
    """The reading, in numpy float32 / float16 arithmetic."""
    w = bf16_f32(w_bits).reshape(w_bits.shape[0], -1, 32)
    idx = np.argmax(np.abs(w), axis=2)                         # first max
    m = np.take_along_axis(w, idx[..., None], axis=2)[..., 0]
    d = (m.astype(np.float64) / -8.0)
    d = np.clip(d, -65504.0, 65504.0)
    s = d.astype(np.float16)                                   # nearest-even
    sf = s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(w / sf[..., None])
    c = np.where(sf[..., None] != 0, np.clip(q + 8, 0, 15), 8).astype(np.uint8)
    c = c.reshape(w_bits.shape)
    wq = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return wq, s.view(np.uint16)


def test_against_numpy():
    rng = np.random.default_rng(1)
    w = bf16_bits(rng.standard_normal((300, 512)) * 0.03)
    wq, ws = oracle.quantize(w)
    nq, ns = numpy_quantize(w)
    assert np.array_equal(ws, ns)
    assert np.array_equal(wq, nq)


def test_against_numpy_subnormal_scales():
    """Blocks small enough that m / -8 falls in fp16's subnormal range, where
    the scale is rounded to a multiple of 2^-24."""
    rng = np.random.default_rng(5)
    w = bf16_bits(rng.standard_normal((100, 256)) * 3e-6)
    wq, ws = oracle.quantize(w)
    nq, ns = numpy_quantize(w)
    assert np.array_equal(ws, ns)
    assert np.array_equal(wq, nq)
    assert np.any((ws & 0x7C00) == 0)          # some scales are fp16 subnormals


def test_round_trip_of_representable_blocks():
    """Blocks (c - 8) * s with s of at most 5 significant bits (so every
    weight is a bf16 value) and a code 0 in each block: the quantiser gives
    back exactly those codes and scales."""
    rng = np.random.default_rng(2)
    N, K = 64, 256
    codes = rng.integers(1, 16, size=(N, K)).astype(np.int64)
    codes[np.arange(N)[:, None], rng.integers(0, 32, size=(N, K // 32)) + 32 * np.arange(K // 32)] = 0
    mant = rng.integers(16, 32, size=(N, K // 32))
    expo = rng.integers(-14, 6, size=(N, K // 32))
    sign = rng.choice([-1.0, 1.0], size=(N, K // 32))
    s = sign * np.ldexp(mant.astype(np.float64), expo - 4)
    w = (codes - 8) * np.repeat(s, 32, axis=1)
    wb = bf16_bits(w)
    assert np.array_equal(bf16_f32(wb).astype(np.float64), w)
    wq, ws = oracle.quantize(wb)
    assert np.array_equal(_unpack(wq), codes)
    assert np.array_equal(ws.view(np.float16).astype(np.float64), s)


def test_sign_and_scale_symmetries():
    rng = np.random.default_rng(3)
    wf = rng.standard_normal((40, 320)).astype(np.float32) * 0.02
    wq, ws = oracle.quantize(bf16_bits(wf))
    nq, ns = oracle.quantize(bf16_bits(-wf))
    assert np.array_equal(nq, wq)
    assert np.array_equal(ns.view(np.float16), -ws.view(np.float16))
    q8, s8 = oracle.quantize(bf16_bits(wf * np.float32(8.0)))
    assert np.array_equal(q8, wq)
    assert np.array_equal(s8.view(np.float16).astype(np.float64),
                          8.0 * ws.view(np.float16).astype(np.float64))


def test_error_bound():
    """Every weight lies within half a step of its code's value, except the
    ones clamped at +7 (value exactly -m), which lie within one step."""
    rng = np.random.default_rng(4)
    wb = bf16_bits(rng.standard_normal((200, 512)) * 0.05)
    wq, ws = oracle.quantize(wb)
    w = bf16_f32(wb).astype(np.float64)
    deq = oracle.dequant_f32(wq, ws).astype(np.float64)
    s = np.abs(np.repeat(ws.view(np.float16).astype(np.float64), 32, axis=1))
    err = np.abs(w - deq)
    clamped = _unpack(wq) == 15
    assert np.all(err[~clamped] <= s[~clamped] * (0.5 + 2.0 ** -10))
    assert np.all(err <= s * (1.0 + 2.0 ** -10))


def test_special_blocks():
    K = 64
    w = np.zeros((4, K), np.uint16)
    w[1] = bf16_bits(np.full(K, 2.0 ** -130))           # far below fp16: s = 0
    w[2] = bf16_bits(np.linspace(-1e6, 1e6, K))         # past fp16 range: |s| = 65504
    w[3, :32] = bf16_bits(np.full(32, 0.5))             # ties: first max, m = 0.5
    w[3, 5] = bf16_bits([-0.5])[0]
    wq, ws = oracle.quantize(w)
    s = ws.view(np.float16).astype(np.float64)
    assert np.all(s[0] == 0) and np.all(_unpack(wq[0]) == 8)
    assert np.all(s[1] == 0) and np.all(_unpack(wq[1]) == 8)
    assert np.all(np.abs(s[2]) == 65504.0)
    assert s[3, 0] == -0.0625 and np.all(_unpack(wq[3])[:32][np.arange(32) != 5] == 0)
    assert _unpack(wq[3])[5] == 15                      # -0.5 / -0.0625 = 8, clamped


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 48), np.uint16))

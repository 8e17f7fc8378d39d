"""Pins of the oracle's routed expert FFN (gate/up, SwiGLU, down, weighted
sum) -- "Layer Package Repository Spec", the MoE fixture paragraph under
"Policy Resolution" (routed gate/up/down expert matmuls, fused SwiGLU split,
weighted sum).  CPU only."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synthetic


def _const_case(T, topk, E, H, F, x_bits, gate_code, gate_s, up_code, up_s, down_code, down_s):
    x = np.full((T, H), x_bits, dtype=np.uint16)
    w13_q = np.empty((E, 2 * F, H // 2), dtype=np.uint8)
    w13_s = np.empty((E, 2 * F, H // 32), dtype=np.uint16)
    w13_q[:, 0::2] = gate_code | (gate_code << 4)
    w13_q[:, 1::2] = up_code | (up_code << 4)
    w13_s[:, 0::2] = gate_s
    w13_s[:, 1::2] = up_s
    w2_q = np.full((E, H, F // 2), down_code | (down_code << 4), dtype=np.uint8)
    w2_s = np.full((E, H, F // 32), down_s, dtype=np.uint16)
    return x, w13_q, w13_s, w2_q, w2_s


def test_closed_form_saturated_gate():
    """x = 1, gate weight 7 (code 15, scale 1), up weight 0.5 (code 9, scale
    0.5), down weight 2^-9 (code 10, scale 2^-10), H = 64, F = 32:
    gate = 448, silu(448) = 448 in double, up = 32, a = 14336,
    o = F * a * 2^-9 = 896; gates 0.25 + 0.75 -> y = 896 exactly."""
    T, topk, E, H, F = 2, 2, 3, 64, 32
    args = _const_case(T, topk, E, H, F, 0x3F80, 15, 0x3C00, 9, 0x3800, 10, 0x1400)
    ids = np.array([[0, 2], [1, 0]], dtype=np.int32)
    gates = np.array([[0.25, 0.75], [0.5, 0.5]], dtype=np.float32)
    y, b = oracle.moe_ffn(*args, ids, gates)
    assert np.all(y == 896.0)
    assert np.all(b > 0)


def test_closed_form_negative_gate_is_off():
    """gate = -448: silu(-448) = -448 / (1 + e^448) is below 1e-190."""
    T, topk, E, H, F = 1, 1, 1, 64, 32
    args = _const_case(T, topk, E, H, F, 0x3F80, 1, 0x3C00, 9, 0x3800, 10, 0x1400)
    y, _ = oracle.moe_ffn(*args, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32))
    assert np.all(np.abs(y) < 1e-180)
    assert np.all(y <= 0)


def test_bound_closed_form_when_up_cancels():
    """Up weights alternate +0.5 / -0.5 (codes 9 / 7, scale 0.5) so up = 0
    exactly while its |.|-sum is 32; gate = 448 as above.  Then y = 0 and
    the bound is sum_j |g_j| * F * 2^-9 * silu(448) * 32 = 896 for F = 32."""
    T, topk, E, H, F = 1, 2, 2, 64, 32
    x, w13_q, w13_s, w2_q, w2_s = _const_case(T, topk, E, H, F, 0x3F80, 15, 0x3C00, 9, 0x3800,
                                              10, 0x1400)
    w13_q[:, 1::2] = 0x79            # k even: code 9 (+1), k odd: code 7 (-1)
    y, b = oracle.moe_ffn(x, w13_q, w13_s, w2_q, w2_s, np.array([[0, 1]], np.int32),
                          np.array([[0.25, 0.75]], np.float32))
    assert np.all(y == 0)
    assert np.all(b == 896.0)


def test_zero_up_rows_give_exact_zero_and_zero_bound():
    c = synthetic.moe_ffn_case(11, 3, 2, 4, 64, 64)
    w13_q = c.w13_q.copy()
    w13_q[:, 1::2] = 0x88          # every up weight 0
    y, b = oracle.moe_ffn(c.x, w13_q, c.w13_s, c.w2_q, c.w2_s, c.ids, c.gates)
    assert np.all(y == 0) and np.all(b == 0)


def test_top1_unit_gate_is_the_composition_of_dense_products():
    """One expert with gate 1: y = (silu(x W_gate^T) * (x W_up^T)) W_down^T,
    built from the pinned dense oracle and numpy's float64 matmul."""
    c = synthetic.moe_ffn_case(12, 3, 1, 5, 96, 64)
    gates = np.ones_like(c.gates)
    y, _ = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.ids, gates)
    for t in range(3):
        e = int(c.ids[t, 0])
        h, _ = oracle.matmul(c.x[t:t + 1], c.w13_q[e], c.w13_s[e])
        g, u = h[0, 0::2], h[0, 1::2]
        a = g / (1.0 + np.exp(-g)) * u
        w2 = oracle.dequant_f32(c.w2_q[e], c.w2_s[e]).astype(np.float64)
        ref = w2 @ a
        assert np.all(np.abs(y[t] - ref) <= 1e-12 * (np.abs(w2) @ np.abs(a)))


def _brute(x, w13_q, w13_s, w2_q, w2_s, ids, gates):
    """Scalar loops: nibble unpack, numpy's fp16 decode, Python floats."""
    E, F2, Hh = w13_q.shape
    F, H = F2 // 2, Hh * 2

    def w(q, s, n, k):
        byte = int(q[n, k // 2])
        c = (byte >> 4) if k % 2 else (byte & 15)
        return (c - 8) * float(s[n, k // 32:k // 32 + 1].view(np.float16)[0])

    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    T, topk = ids.shape
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            a = []
            for f in range(F):
                g = sum(xf[t, k] * w(w13_q[e], w13_s[e], 2 * f, k) for k in range(H))
                u = sum(xf[t, k] * w(w13_q[e], w13_s[e], 2 * f + 1, k) for k in range(H))
                a.append(g / (1.0 + math.exp(-g)) * u)
            for h in range(H):
                o = sum(a[f] * w(w2_q[e], w2_s[e], h, f) for f in range(F))
                y[t, h] += float(gates[t, j]) * o
    return y


def test_brute_force_tiny():
    c = synthetic.moe_ffn_case(13, 2, 2, 3, 32, 32)
    ids = c.ids.copy()
    ids[1, 1] = 7                   # out of range: adds nothing
    y, b = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, ids, c.gates)
    yb = _brute(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, ids, c.gates)
    np.testing.assert_allclose(y, yb, rtol=1e-9, atol=1e-9 * np.max(np.abs(yb)))
    assert np.all(b >= np.abs(y) * 0.999)


def test_repeated_id_sums_and_invalid_id_adds_nothing():
    c = synthetic.moe_ffn_case(14, 2, 3, 4, 64, 32)
    ids = np.array([[1, 1, -1], [2, 9, 2]], dtype=np.int32)
    gates = np.array([[0.25, 0.5, 0.125], [0.5, 0.75, 0.25]], dtype=np.float32)
    y, _ = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, ids, gates)
    ids1 = np.array([[1], [2]], dtype=np.int32)
    y1, _ = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, ids1,
                           np.array([[0.75], [0.75]], dtype=np.float32))
    np.testing.assert_allclose(y, y1, rtol=1e-12, atol=1e-12)


def test_shape_errors():
    c = synthetic.moe_ffn_case(15, 1, 1, 2, 64, 32)
    with pytest.raises(ValueError):
        oracle.moe_ffn(c.x[:, :32], c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.ids, c.gates)
    with pytest.raises(ValueError):
        oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q[:, :32], c.w2_s, c.ids, c.gates)

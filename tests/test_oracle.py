"""Pins of the CPU oracle against things other than itself.

Every check here runs on the CPU.  What pins what:

* dequantisation -- exhaustive: all 16 codes x all 65,536 fp16 scale bit
  patterns, expected values from numpy's own float16 decoding (fp32 output)
  and torch's float32 -> bfloat16 rounding (bf16 output), bit for bit;
* nibble order and scale block index -- hand-worked fixtures in
  tests/golden/ (values computed by hand from the layout rules);
* the k-ordered double sum -- exact rational brute force (fractions) on
  8 x 64 tiles, closed forms on constant / alternating inputs, and a float64
  library matmul of the dequantised matrix (catches transposed operands and
  index mix-ups on non-square shapes);
* the MoE weighted sum -- reductions to the dense case and an exact rational
  brute force on a tiny routed case.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from helpers import load_golden

# ---------------------------------------------------------------- decoding


def _fp16(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


def test_scalar_decoders_match_struct():
    for b in range(0, 65536, 7):
        a, e = oracle.fp16_value(b), _fp16(b)
        assert (a == e) or (np.isnan(a) and np.isnan(e)), hex(b)
        a, e = oracle.bf16_value(b), _bf16(b)
        assert (a == e) or (np.isnan(a) and np.isnan(e)), hex(b)
        if not (np.isnan(a) or np.isinf(a)):
            assert np.signbit(a) == np.signbit(e)


def exhaustive_case():
    """N = 4096 rows, K = 512: 65,536 blocks, block i has scale pattern i,
    and every block holds codes 0..15 twice (k = 0..31 -> code k % 16)."""
    N, K = 4096, 512
    block = np.array([(2 * j) % 16 | (((2 * j + 1) % 16) << 4) for j in range(16)],
                     dtype=np.uint8)
    w_q = np.tile(block, (N, K // 32))
    w_s = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(N, K // 32)
    codes = np.tile(np.arange(32) % 16, K // 32)
    return w_q, w_s, codes


def test_dequant_f32_exhaustive():
    w_q, w_s, codes = exhaustive_case()
    got = oracle.dequant_f32(w_q, w_s)
    s = w_s.view(np.float16).astype(np.float64)                # numpy's decoding
    s_full = np.repeat(s, 32, axis=1)
    with np.errstate(invalid="ignore"):
        exp = ((codes - 8)[None, :] * s_full).astype(np.float32)
    nan = np.isnan(exp)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got.view(np.uint32)[~nan], exp.view(np.uint32)[~nan])


def test_dequant_bf16_exhaustive():
    torch = pytest.importorskip("torch")
    w_q, w_s, codes = exhaustive_case()
    got = oracle.dequant_bf16_bits(w_q, w_s)
    s = np.repeat(w_s.view(np.float16).astype(np.float64), 32, axis=1)
    with np.errstate(invalid="ignore"):
        f32 = ((codes - 8)[None, :] * s).astype(np.float32)
    exp = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f32)
    got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    assert np.array_equal(got_nan, nan)
    assert np.array_equal(got[~nan], exp[~nan])


def test_bf16_round_scalar_ties_and_limits():
    # exact ties between bf16 neighbours go to the even significand
    one = 1.0
    ulp = 2.0 ** -7
    assert oracle.bf16_round_bits(one + ulp / 2) == 0x3F80          # tie -> even (1.0)
    assert oracle.bf16_round_bits(one + 3 * ulp / 2) == 0x3F82      # tie -> even (1+2ulp)
    assert oracle.bf16_round_bits(one + ulp / 2 + 2 ** -30) == 0x3F81
    # largest finite bf16 and overflow
    big = (2 - 2 ** -7) * 2.0 ** 127
    assert oracle.bf16_round_bits(big) == 0x7F7F
    assert oracle.bf16_round_bits(big + 2.0 ** 119) == 0x7F80         # tie at the top -> inf
    # subnormal quantum 2^-133
    assert oracle.bf16_round_bits(2.0 ** -133) == 0x0001
    assert oracle.bf16_round_bits(2.0 ** -134) == 0x0000              # tie -> even (0)
    assert oracle.bf16_round_bits(-3 * 2.0 ** -134) == 0x8002         # tie -> even (2)


# ------------------------------------------------------- hand-worked values


@pytest.mark.parametrize("name", ["nibble_order.txt", "two_blocks.txt"])
def test_golden_dequant_and_matmul(name):
    g = load_golden(name)
    got = oracle.dequant_f32(g["w_q"], g["w_s"])
    assert np.array_equal(got.astype(np.float64), g["w"])
    y, t = oracle.matmul(g["x"], g["w_q"], g["w_s"])
    for m, n, v in g["y"]:
        assert y[m, n] == v, (m, n, y[m, n], v)


# ------------------------------------------------------------ closed forms


@pytest.mark.parametrize("code,a_bits,s_bits", [(0, 0x3F80, 0x3C00), (15, 0xC040, 0x2E66),
                                                (3, 0x3E00, 0x0001), (12, 0x4120, 0x7BFF)])
def test_closed_form_constant(code, a_bits, s_bits):
    """x = a everywhere, every code c, every scale s: y = K * a * (c-8) * s."""
    M, N, K = 2, 3, 256
    x = np.full((M, K), a_bits, dtype=np.uint16)
    w_q = np.full((N, K // 2), code | (code << 4), dtype=np.uint8)
    w_s = np.full((N, K // 32), s_bits, dtype=np.uint16)
    y, t = oracle.matmul(x, w_q, w_s)
    exp = K * _bf16(a_bits) * (code - 8) * _fp16(s_bits)
    assert np.all(y == exp)
    assert np.all(t == abs(exp))


def test_closed_form_zero_codes():
    """Every code 8 is the zero weight: y = 0 and the bound is 0."""
    d = synthetic.dense_case(11, 3, 5, 96)
    w_q = np.full_like(d.w_q, 0x88)
    y, t = oracle.matmul(d.x, w_q, d.w_s)
    assert np.all(y == 0) and np.all(t == 0)


def test_closed_form_alternating():
    """Codes 0,15,0,15,... and x = 1: each pair is -8 + 7 = -1, each block
    -16: y = -16 * sum of the row's scales."""
    N, K = 4, 160
    d = synthetic.dense_case(12, 1, N, K)
    w_q = np.full((N, K // 2), 0xF0, dtype=np.uint8)
    x = np.full((1, K), 0x3F80, dtype=np.uint16)
    y, t = oracle.matmul(x, w_q, d.w_s)
    exp = -16 * d.w_s.view(np.float16).astype(np.float64).sum(axis=1)
    assert np.array_equal(y[0], exp)


def test_closed_form_single_block():
    """Only block b has a non-zero scale: y = s_b * sum_{k in b} x_k (c_k - 8)."""
    N, K, b = 3, 256, 5
    d = synthetic.dense_case(13, 2, N, K)
    w_s = np.zeros_like(d.w_s)
    w_s[:, b] = d.w_s[:, b]
    y, _ = oracle.matmul(d.x, d.w_q, w_s)
    for m in range(2):
        for n in range(N):
            acc = Fraction(0)
            for k in range(32 * b, 32 * b + 32):
                byte = int(d.w_q[n, k // 2])
                c = (byte & 15) if k % 2 == 0 else (byte >> 4)
                acc += Fraction(_bf16(int(d.x[m, k]))) * (c - 8)
            exp = acc * Fraction(_fp16(int(w_s[n, b])))
            assert abs(Fraction(y[m, n]) - exp) <= abs(exp) * Fraction(1, 2 ** 50)


# -------------------------------------------------------------- brute force


def _exact_matmul(x, w_q, w_s):
    M, K = x.shape
    N = w_q.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    t = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        w = []
        for k in range(K):
            byte = int(w_q[n, k // 2])
            c = (byte & 15) if k % 2 == 0 else (byte >> 4)
            w.append((c - 8) * Fraction(_fp16(int(w_s[n, k // 32]))))
        for m in range(M):
            for k in range(K):
                p = Fraction(_bf16(int(x[m, k]))) * w[k]
                y[m][n] += p
                t[m][n] += abs(p)
    return y, t


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_brute_force_8x64(seed):
    M, N, K = 8, 8, 64
    d = synthetic.dense_case(seed, M, N, K)
    y, t = oracle.matmul(d.x, d.w_q, d.w_s)
    ye, te = _exact_matmul(d.x, d.w_q, d.w_s)
    for m in range(M):
        for n in range(N):
            slack = K * Fraction(2) ** -53 * te[m][n]
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= slack
            assert abs(Fraction(t[m, n]) - te[m][n]) <= slack


def test_matches_float64_library_matmul():
    """Non-square shapes: oracle vs numpy float64 matmul of the dequantised W."""
    M, N, K = 3, 70, 96
    d = synthetic.dense_case(31, M, N, K)
    y, t = oracle.matmul(d.x, d.w_q, d.w_s)
    xf = (d.x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = oracle.dequant_f32(d.w_q, d.w_s).astype(np.float64)
    ref = xf @ w.T
    tref = np.abs(xf) @ np.abs(w).T
    assert np.allclose(t, tref, rtol=1e-13, atol=0)
    assert np.all(np.abs(y - ref) <= 4 * K * 2.0 ** -53 * tref)


def test_bf16_weights_option():
    """bf16_weights=True is the same sum over the bf16-rounded weights."""
    M, N, K = 2, 9, 64
    d = synthetic.dense_case(32, M, N, K)
    y, _ = oracle.matmul(d.x, d.w_q, d.w_s, bf16_weights=True)
    wb = oracle.dequant_bf16_bits(d.w_q, d.w_s)
    wf = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = (d.x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = xf @ wf.T
    tref = np.abs(xf) @ np.abs(wf).T
    assert np.all(np.abs(y - ref) <= 4 * K * 2.0 ** -53 * tref)


def test_sampled_matches_full():
    M, N, K = 5, 33, 128
    d = synthetic.dense_case(33, M, N, K)
    y, t = oracle.matmul(d.x, d.w_q, d.w_s)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    ys, ts = oracle.matmul_sampled(d.x, d.w_q, d.w_s, ms, ns)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(ts, t[ms, ns])


# --------------------------------------------------------------------- MoE


def test_moe_top1_unit_gate_is_dense():
    T, E, N, K = 4, 6, 10, 64
    c = synthetic.moe_case(41, T, 1, E, N, K)
    gates = np.ones((T, 1), dtype=np.float32)
    y, t = oracle.moe(c.x, c.w_q, c.w_s, c.ids, gates)
    for tok in range(T):
        e = int(c.ids[tok, 0])
        yd, td = oracle.matmul(c.x[tok:tok + 1], c.w_q[e], c.w_s[e])
        assert np.array_equal(y[tok], yd[0]) and np.array_equal(t[tok], td[0])


def test_moe_permutation_invariant():
    T, topk, E, N, K = 3, 3, 7, 8, 64
    c = synthetic.moe_case(42, T, topk, E, N, K)
    y, t = oracle.moe(c.x, c.w_q, c.w_s, c.ids, c.gates)
    perm = np.random.default_rng(1).permutation(E)
    inv = np.argsort(perm)
    y2, t2 = oracle.moe(c.x, c.w_q[perm], c.w_s[perm], inv[c.ids].astype(np.int32), c.gates)
    assert np.array_equal(y, y2) and np.array_equal(t, t2)


def test_moe_identical_experts_reduce_to_dense():
    T, topk, E, N, K = 3, 4, 5, 6, 96
    c = synthetic.moe_case(43, T, topk, E, N, K)
    w_q = np.repeat(c.w_q[:1], E, axis=0)
    w_s = np.repeat(c.w_s[:1], E, axis=0)
    y, t = oracle.moe(c.x, w_q, w_s, c.ids, c.gates)
    yd, td = oracle.matmul(c.x, w_q[0], w_s[0])
    gsum = c.gates.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.allclose(y, yd * gsum, rtol=0, atol=1e-12 * td.max())


def test_moe_out_of_range_ids_contribute_nothing():
    T, topk, E, N, K = 2, 3, 4, 5, 64
    c = synthetic.moe_case(44, T, topk, E, N, K)
    ids = c.ids.copy()
    ids[0, 1] = E
    ids[1, 2] = -1
    y, _ = oracle.moe(c.x, c.w_q, c.w_s, ids, c.gates)
    keep = np.ones_like(c.gates)
    keep[0, 1] = 0
    keep[1, 2] = 0
    y2, _ = oracle.moe(c.x, c.w_q, c.w_s, np.where(keep > 0, ids, 0).astype(np.int32),
                       (c.gates * keep).astype(np.float32))
    assert np.allclose(y, y2, rtol=0, atol=1e-15)


def test_moe_brute_force():
    T, topk, E, N, K = 2, 3, 5, 4, 64
    c = synthetic.moe_case(45, T, topk, E, N, K)
    y, t = oracle.moe(c.x, c.w_q, c.w_s, c.ids, c.gates)
    for tok in range(T):
        for n in range(N):
            acc, mag = Fraction(0), Fraction(0)
            for j in range(topk):
                e = int(c.ids[tok, j])
                ye, te = _exact_matmul(c.x[tok:tok + 1], c.w_q[e, n:n + 1], c.w_s[e, n:n + 1])
                g = Fraction(float(c.gates[tok, j]))
                acc += g * ye[0][0]
                mag += abs(g) * te[0][0]
            slack = (K + topk + 2) * Fraction(2) ** -52 * mag
            assert abs(Fraction(y[tok, n]) - acc) <= slack
            assert abs(Fraction(t[tok, n]) - mag) <= slack


# --------------------------------------------------------------- generator


def test_generator_deterministic_and_distributed():
    a = synthetic.dense_case(5, 2, 64, 512)
    b = synthetic.dense_case(5, 2, 64, 512)
    c = synthetic.dense_case(6, 2, 64, 512)
    assert all(np.array_equal(u, v) for u, v in ((a.x, b.x), (a.w_q, b.w_q), (a.w_s, b.w_s)))
    assert not np.array_equal(a.w_q, c.w_q)
    d = synthetic.dense_case(7, 64, 512, 1024)
    lo = d.w_q & 15
    hi = d.w_q >> 4
    for nib in (lo, hi):
        counts = np.bincount(nib.ravel(), minlength=16)
        assert counts.min() > 0.9 * nib.size / 16
    s = d.w_s.view(np.float16).astype(np.float64)
    assert np.all(s >= 0)
    assert abs(s.mean() - 0.02 * np.sqrt(2 / np.pi)) < 5e-4
    xf = (d.x.astype(np.uint32) << 16).view(np.float32)
    assert abs(xf.mean()) < 0.02 and abs(xf.std() - 1) < 0.02


def test_moe_router_distinct_and_normalised():
    c = synthetic.moe_case(4, 8, 8, 128, 4, 64)
    for tok in range(8):
        assert len(set(c.ids[tok].tolist())) == 8
        assert abs(float(c.gates[tok].astype(np.float64).sum()) - 1) < 1e-6
    assert c.ids.min() >= 0 and c.ids.max() < 128

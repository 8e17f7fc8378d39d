"""Parity of q4_rmsnorm_matmul (the quantised matmul behind an RMSNorm
prologue) with the oracle, through the C ABI.

Bar per output: |y - y_ref| <= 1e-3 * sum_k |x'_k w_k| + u, u = sum_k
hulp(x'_k) |w_k| (what rounding the normalised activations x' to bf16, the
matrix cores' operand type, can move y by), plus half a bf16 ulp of y_ref
for bf16 outputs.  The fused decode form keeps x' in fp32 and meets the bar
without u; it is held to the same bar."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import DEV, dev, host
from helpers import RTOL, assert_parity, bf16_half_ulp, stratified_outputs

pytestmark = pytest.mark.gpu

import quantized_q4_block_amd as q4  # noqa: E402

F32, BF16 = torch.float32, torch.bfloat16


def _run(c, out_dtype=F32, workspace="auto"):
    y = q4.q4_rmsnorm_matmul(dev(c.x), dev(c.gamma), c.eps, dev(c.w_q), dev(c.w_s),
                             out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return host(y)


def _check(c, out_dtype=F32, what="", workspace="auto"):
    y = _run(c, out_dtype, workspace)
    y_ref, t, u = oracle.rmsnorm_matmul(c.x, c.gamma, c.eps, c.w_q, c.w_s)
    extra = u + (bf16_half_ulp(y_ref) if out_dtype == BF16 else 0.0)
    assert_parity(y, y_ref, t, RTOL, extra, what=what)
    return y


# M <= 2 with K up to 8192: the fused matrix-vector form (no workspace);
# K = 8224 leaves it (normalised activations in the workspace, then the
# matrix-vector path cut into slices).
@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("N,K", [(1, 32), (77, 640), (300, 5120), (65, 8192), (40, 8224)])
def test_decode_forms(M, N, K):
    assert (q4.q4_rmsnorm_matmul_workspace_bytes(M, N, K) == 0) == (K <= 8192)
    c = synthetic.rms_case(20000 + M * 100 + N, M, N, K)
    _check(c, what=f"rms decode M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(3, 100, 640), (16, 257, 2048 + 32), (33, 300, 4096),
                                   (129, 257, 1024), (300, 77, 2048 + 32), (512, 640, 5120)])
def test_prologue_forms(M, N, K):
    assert q4.q4_rmsnorm_matmul_workspace_bytes(M, N, K) >= M * K * 2
    c = synthetic.rms_case(21000 + M + N, M, N, K)
    _check(c, what=f"rms M={M} N={N} K={K}")
    _check(c, BF16, what=f"rms bf16 M={M} N={N} K={K}")


def test_workspace_of_only_the_activations():
    """A workspace holding only the normalised activations: the product runs
    uncut, with the same result as with the full workspace (K slices)."""
    M, N, K = 512, 640, 5120
    c = synthetic.rms_case(21500, M, N, K)
    full = q4.q4_rmsnorm_matmul_workspace_bytes(M, N, K)
    act = (M * K * 2 + 255) // 256 * 256
    assert full > act
    small = torch.full((act,), 0x7F, dtype=torch.uint8, device=DEV)
    y = _run(c, workspace=small)
    y_ref, t, u = oracle.rmsnorm_matmul(c.x, c.gamma, c.eps, c.w_q, c.w_s)
    assert_parity(y, y_ref, t, RTOL, u, what="activations-only workspace")


@pytest.mark.parametrize("M", [1, 2, 200])
@pytest.mark.parametrize("kind", ["huge", "tiny", "constant"])
def test_activation_ranges(M, kind):
    """Rows scaled by 2^100 or 2^-100 (the squares would overflow or
    underflow fp32; the sums are in double), and constant rows (x' = +-1 at
    gamma = 1, eps = 0)."""
    N, K = 130, 1024
    c = synthetic.rms_case(22000 + M, M, N, K)
    xf = (c.x.astype(np.uint32) << 16).view(np.float32)
    if kind == "huge":
        c.x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** 100))
    elif kind == "tiny":
        c.x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** -100))
    else:
        c.x = np.repeat(c.x[:, :1], K, axis=1)
        c.gamma = np.full(K, 0x3F80, np.uint16)
        c.eps = 0.0
    _check(c, what=f"rms {kind} M={M}")


def test_full_decode_gate_up():
    cfg = synthetic.RMS_CONFIGS["rms_decode_gate_up"]
    c = synthetic.rms_case(cfg["seed"], cfg["M"], cfg["N"], cfg["K"])
    _check(c, what="rms_decode_gate_up")


def test_full_prefill_stratified():
    cfg = synthetic.RMS_CONFIGS["rms_prefill"]
    M, N = cfg["M"], cfg["N"]
    c = synthetic.rms_case(cfg["seed"], M, N, cfg["K"])
    y = _run(c, BF16)
    assert np.isfinite(y).all()
    ms, ns = stratified_outputs(M, N)
    y_ref, t, u = oracle.rmsnorm_matmul_sampled(c.x, c.gamma, c.eps, c.w_q, c.w_s, ms, ns)
    assert_parity(y[ms, ns], y_ref, t, RTOL, u + bf16_half_ulp(y_ref), what="rms_prefill")


def test_run_to_run_identical():
    for M in (1, 200):
        c = synthetic.rms_case(23000 + M, M, 500, 2048)
        x, g, wq, ws = dev(c.x), dev(c.gamma), dev(c.w_q), dev(c.w_s)
        a = q4.q4_rmsnorm_matmul(x, g, c.eps, wq, ws)
        b = q4.q4_rmsnorm_matmul(x, g, c.eps, wq, ws)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), M


def test_errors_leave_output_untouched():
    c = synthetic.rms_case(23500, 200, 64, 256)
    x, g, wq, ws = dev(c.x), dev(c.gamma), dev(c.w_q), dev(c.w_s)
    y = torch.full((200, 64), 3.0, device=DEV)
    P = ctypes.c_void_p
    args = lambda eps, gp, work, nbytes: (P(x.data_ptr()), P(gp), ctypes.c_float(eps),  # noqa: E731
                                          P(wq.data_ptr()), P(ws.data_ptr()), P(y.data_ptr()),
                                          q4.Q4_F32, 200, 64, 256, P(work), nbytes, None)
    assert q4.lib.q4_rmsnorm_matmul(*args(1e-6, g.data_ptr(), 0, 0)) == q4.Q4_ERR_WORKSPACE
    assert q4.lib.q4_rmsnorm_matmul(*args(-1.0, g.data_ptr(), 0, 0)) == q4.Q4_ERR_SHAPE
    assert q4.lib.q4_rmsnorm_matmul(*args(float("nan"), g.data_ptr(), 0, 0)) == q4.Q4_ERR_SHAPE
    assert q4.lib.q4_rmsnorm_matmul(*args(1e-6, g.data_ptr() + 2, 0, 0)) == q4.Q4_ERR_ALIGN
    assert q4.lib.q4_rmsnorm_matmul(*args(1e-6, 0, 0, 0)) == q4.Q4_ERR_NULL
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)

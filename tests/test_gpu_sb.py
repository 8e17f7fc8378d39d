"""Parity of q4_sb_matmul (super-block scales: w = (c - 8) * d[k/256] *
sc[k/32]) with the oracle, through the C ABI: every path (matrix-vector,
few-row and tiled matrix cores, with and without K slices) against the
exact-weight oracle at 1e-3 * sum|x w| (+ half a bf16 ulp for bf16 out)."""
from __future__ import annotations

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


def _run(x, c, out_dtype=F32, workspace="auto"):
    y = q4.q4_sb_matmul(dev(x), dev(c.w_q), dev(c.w_d), dev(c.w_sc), out_dtype=out_dtype,
                        workspace=workspace)
    torch.cuda.synchronize()
    return host(y)


def _check(c, out_dtype=F32, what="", workspace="auto"):
    y = _run(c.x, c, out_dtype, workspace)
    y_ref, t = oracle.sb_matmul(c.x, c.w_q, c.w_d, c.w_sc)
    extra = bf16_half_ulp(y_ref) if out_dtype == BF16 else 0.0
    assert_parity(y, y_ref, t, RTOL, extra, what=what)


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 300, 5120), (2, 77, 8192), (1, 65, 8448),
                                   (3, 100, 768), (16, 257, 2048), (33, 300, 4096),
                                   (129, 257, 1024), (300, 77, 2304), (512, 640, 5120)])
def test_paths(M, N, K):
    c = synthetic.sb_case(41000 + M + N, M, N, K)
    _check(c, what=f"sb M={M} N={N} K={K}")
    if M > 2:
        _check(c, BF16, what=f"sb bf16 M={M} N={N} K={K}")


def test_scales_only_workspace():
    """A workspace of only the expanded scales: the tiled product runs
    uncut and agrees with the oracle."""
    M, N, K = 512, 640, 5120
    c = synthetic.sb_case(41500, M, N, K)
    nbytes = (N * K // 32 * 4 + 255) // 256 * 256
    assert q4.q4_sb_matmul_workspace_bytes(M, N, K) > nbytes
    _check(c, what="scales-only workspace",
           workspace=torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV))


def test_identity_activations_give_exact_weights():
    K, N = 256, 96
    c = synthetic.sb_case(42000, 1, N, K)
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    w = oracle.sb_dequant(c.w_q, c.w_d, c.w_sc)
    assert np.array_equal(_run(eye, c), w.T)                     # tiled
    for m0 in (0, 40, 254):                                       # matrix-vector, M = 2
        assert np.array_equal(_run(eye[m0:m0 + 2], c), w[:, m0:m0 + 2].T)
    assert np.array_equal(_run(eye[:8], c), w[:, :8].T)           # few-row


def test_zero_multipliers_and_closed_form():
    K, N = 512, 70
    c = synthetic.sb_case(42500, 200, N, K)
    c.x = np.full((200, K), 0x3FC0, np.uint16)                   # 1.5
    c.w_q = np.full((N, K // 2), 0xDD, np.uint8)                  # code 13: +5
    c.w_d = np.full((N, K // 256), np.float16(2.0 ** -6).view(np.uint16), np.uint16)
    c.w_sc = np.full((N, K // 32), 3, np.uint8)
    c.w_sc[:, ::2] = 0
    for M in (1, 8, 200):
        y = _run(c.x[:M], c)
        assert np.all(y == K / 2 * 1.5 * 5 * 3 * 2.0 ** -6), M


def test_full_decode_gate_up():
    cfg = synthetic.SB_CONFIGS["sb_decode_gate_up"]
    _check(synthetic.sb_case(cfg["seed"], cfg["M"], cfg["N"], cfg["K"]), what="sb_decode_gate_up")


def test_full_prefill_stratified():
    cfg = synthetic.SB_CONFIGS["sb_prefill"]
    M, N = cfg["M"], cfg["N"]
    c = synthetic.sb_case(cfg["seed"], M, N, cfg["K"])
    y = _run(c.x, c, BF16)
    ms, ns = stratified_outputs(M, N)
    got, ref, bound = np.empty(N), np.empty(N), np.empty(N)
    for m in range(M):
        cols = ns[ms == m]
        y_ref, t = oracle.sb_matmul(c.x[m:m + 1], c.w_q[cols], c.w_d[cols], c.w_sc[cols])
        got[cols], ref[cols], bound[cols] = y[m, cols], y_ref[0], t[0]
    assert_parity(got, ref, bound, RTOL, bf16_half_ulp(ref), what="sb_prefill stratified")


def test_errors():
    c = synthetic.sb_case(43000, 4, 64, 512)
    with pytest.raises(q4.Q4Error):
        q4.q4_sb_matmul(dev(c.x), dev(c.w_q), dev(c.w_d), dev(c.w_sc),
                        workspace=torch.empty(16, dtype=torch.uint8, device=DEV))

"""GPU parity of the 4-bit float block product (q4_mx_matmul, through the C
ABI) with the oracle: e2m1 elements, one E8M0 scale per 32 k.  Every weight
enters exactly, so the bar is the matmul tolerance |y - y_ref| <= 1e-3 *
sum_k |x_k w_k| per output (plus half a bf16 ulp of y_ref for bf16 outputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from helpers import RTOL, assert_parity, bf16_half_ulp, stratified_outputs

pytestmark = pytest.mark.gpu

import quantized_q4_block_amd as q4  # noqa: E402

DEV = "cuda:0"


def _mx(x, w_q, w_e, out_dtype=torch.float32):
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)
    y = q4.q4_mx_matmul(xd, torch.from_numpy(np.ascontiguousarray(w_q)).to(DEV),
                        torch.from_numpy(np.ascontiguousarray(w_e)).to(DEV), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check(c, what, out_dtype=torch.float32):
    y = _mx(c.x, c.w_q, c.w_e, out_dtype)
    y_ref, t = oracle.mx_matmul(c.x, c.w_q, c.w_e)
    extra = 0.0 if out_dtype == torch.float32 else 2.0 ** -9 * np.abs(y_ref)
    assert_parity(y, y_ref, t, RTOL, extra=extra, what=what)


# M from 1 to 8; N with ragged task tails; K of one block to several stages,
# with leftover stages split between the half-waves (<= 32 blocks) or not
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("N,K", [(1, 32), (7, 64), (65, 2048 + 32 * 5), (300, 4096 + 32 * 40),
                                 (131, 5120), (96, 17408)])
def test_mx_parity_shapes(M, N, K):
    c = synthetic.mx_case(9000 + 13 * M + N + K, M, N, K)
    _check(c, f"mx M={M} N={N} K={K}")


# from 3 rows on: the few-row matrix-core kernel, one or more slabs of 32 rows
@pytest.mark.parametrize("M", [3, 5, 16, 17, 33, 70])
@pytest.mark.parametrize("N,K", [(40, 96), (130, 2048 + 32 * 3), (512, 5120)])
def test_mx_few_rows(M, N, K):
    c = synthetic.mx_case(9400 + M + N + K, M, N, K)
    _check(c, f"mx few-row M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 5, 40])
def test_mx_bf16_output(M):
    c = synthetic.mx_case(9100 + M, M, 200, 3072)
    _check(c, f"mx bf16 M={M}", out_dtype=torch.bfloat16)


# many rows with K a multiple of 64: the tiled matrix-core kernel (128 x 128
# tiles, ragged in M and N); K = 96 and 2080 keep the few-row slabs
@pytest.mark.parametrize("M,N,K", [(129, 130, 64), (200, 300, 2048 + 64), (256, 256, 5120),
                                   (1000, 72, 1024), (150, 100, 96), (300, 50, 2080)])
def test_mx_tiled(M, N, K):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_MFMA
    c = synthetic.mx_case(9500 + M + N + K, M, N, K)
    _check(c, f"mx tiled M={M} N={N} K={K}")
    _check(c, f"mx tiled bf16 M={M} N={N} K={K}", out_dtype=torch.bfloat16)


def test_mx_full_prefill_stratified():
    """The prefill shape (512 x 34816 x 5120, bf16 out) on the tiled kernel,
    against the oracle on one output of every column, spread so that every
    row and every 128 x 128 output tile is hit."""
    cfg = synthetic.MX_CONFIGS["mx_prefill"]
    M, N = cfg["M"], cfg["N"]
    c = synthetic.mx_case(cfg["seed"], M, N, cfg["K"])
    y = _mx(c.x, c.w_q, c.w_e, torch.bfloat16)
    assert np.isfinite(y).all()
    ms, ns = stratified_outputs(M, N)
    assert len(set(ms.tolist())) == M
    assert len(set(zip((ms // 128).tolist(), (ns // 128).tolist()))) == (M // 128) * (N // 128)
    got = np.empty(N)
    ref = np.empty(N)
    bound = np.empty(N)
    for m in range(M):
        cols = ns[ms == m]
        y_ref, t = oracle.mx_matmul(c.x[m:m + 1], c.w_q[cols], c.w_e[cols])
        got[cols], ref[cols], bound[cols] = y[m, cols], y_ref[0], t[0]
    assert_parity(got, ref, bound, RTOL, extra=bf16_half_ulp(ref), what="mx_prefill stratified")


def _mx_ex(x, w_q, w_e, out_dtype=torch.float32, workspace="auto"):
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)
    y = q4.q4_mx_matmul_ex(xd, torch.from_numpy(np.ascontiguousarray(w_q)).to(DEV),
                           torch.from_numpy(np.ascontiguousarray(w_e)).to(DEV),
                           out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


# K slices of the tiled path through q4_mx_matmul_ex (2 to 58 slices, ragged
# last slice; M * N = 60000 and 33153 take the combine kernel's 16-byte and
# scalar forms)
@pytest.mark.parametrize("M,N,K", [(200, 300, 2048 + 64), (129, 257, 1024), (200, 128, 64 * 520)])
def test_mx_tiled_split(M, N, K):
    assert q4.q4_mx_matmul_workspace_bytes(M, N, K) >= 2 * M * N * 4
    c = synthetic.mx_case(9600 + M + N, M, N, K)
    y_ref, t = oracle.mx_matmul(c.x, c.w_q, c.w_e)
    y = _mx_ex(c.x, c.w_q, c.w_e)
    assert_parity(y, y_ref, t, RTOL, what=f"mx split M={M} N={N} K={K}")
    yb = _mx_ex(c.x, c.w_q, c.w_e, torch.bfloat16)
    assert_parity(yb, y_ref, t, RTOL, extra=2.0 ** -9 * np.abs(y_ref), what=f"mx split bf16 M={M}")
    y0 = _mx_ex(c.x, c.w_q, c.w_e, workspace=None)
    assert_parity(y0, y_ref, t, RTOL, what=f"mx unsplit M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(64, 4096, 4096 + 64 * 3), (128, 2048, 8192)])
def test_mx_slab_shapes_with_a_workspace(M, N, K):
    """33..128 rows on large weights: the tiled kernel cut along K with a
    workspace, the few-row slabs without; both exact."""
    assert q4.q4_matmul_path_ex(M, N, K, True) == q4.Q4_PATH_MFMA
    assert q4.q4_mx_matmul_workspace_bytes(M, N, K) > 0
    c = synthetic.mx_case(9800 + M, M, N, K)
    y_ref, t = oracle.mx_matmul(c.x, c.w_q, c.w_e)
    assert_parity(_mx_ex(c.x, c.w_q, c.w_e), y_ref, t, RTOL, what=f"mx slab shape tiled M={M}")
    assert_parity(_mx_ex(c.x, c.w_q, c.w_e, workspace=None), y_ref, t, RTOL,
                  what=f"mx slab shape slabs M={M}")


def test_mx_split_down_projection_sampled_and_deterministic():
    """512 x 5120 x 17408 (160 tiles, 4 slices) with junk workspace contents:
    two calls agree bit for bit; sampled rows and columns against the oracle."""
    M, N, K = 512, 5120, 17408
    c = synthetic.mx_case(9700, M, N, K)
    x = torch.from_numpy(c.x.view(np.int16)).to(DEV)
    wq, we = torch.from_numpy(c.w_q).to(DEV), torch.from_numpy(c.w_e).to(DEV)
    need = q4.q4_mx_matmul_workspace_bytes(M, N, K)
    work = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    y1 = q4.q4_mx_matmul_ex(x, wq, we, out_dtype=torch.bfloat16, workspace=work)
    y2 = q4.q4_mx_matmul_ex(x, wq, we, out_dtype=torch.bfloat16, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y = y1.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(78)
    ms = np.unique(np.concatenate([rng.integers(0, M, 30), [0, M - 1]]))
    ns = np.unique(np.concatenate([rng.integers(0, N, 200), [0, N - 1]]))
    y_ref, t = oracle.mx_matmul(c.x[ms], c.w_q[ns], c.w_e[ns])
    assert_parity(y[np.ix_(ms, ns)], y_ref, t, RTOL, extra=2.0 ** -9 * np.abs(y_ref),
                  what="mx down split sampled")


def test_mx_full_decode_gate_up():
    cfg = synthetic.MX_CONFIGS["mx_decode_gate_up"]
    c = synthetic.mx_case(cfg["seed"], cfg["M"], cfg["N"], cfg["K"])
    _check(c, "mx_decode_gate_up")


def test_mx_scale_extremes_and_nan():
    """E8M0 bytes 0 (2^-127, an fp32 subnormal), 254 and 255 (NaN)."""
    c = synthetic.mx_case(9200, 2, 64, 512)
    _extremes(c)
    _extremes(synthetic.mx_case(9201, 7, 64, 512))        # few-row path
    _extremes(synthetic.mx_case(9202, 200, 64, 512))      # tiled path


def _extremes(c):
    w_e = c.w_e.copy()
    w_e[0::3, :] = 0
    w_e[1::3, 0] = 254
    xs = c.x.copy()
    xs[:] = 0x3C00                     # 2^-7: keeps the 2^127 blocks finite
    y = _mx(xs, c.w_q, w_e)
    y_ref, t = oracle.mx_matmul(xs, c.w_q, w_e)
    assert_parity(y, y_ref, t, RTOL, what="E8M0 extremes")
    # a NaN scale poisons its row only (the other blocks keep ordinary scales)
    w_e = c.w_e.copy()
    w_e[5, 2] = 255
    y = _mx(c.x, c.w_q, w_e)
    assert np.all(np.isnan(y[:, 5]))
    others = np.delete(np.arange(w_e.shape[0]), 5)
    assert np.all(np.isfinite(y[:, others]))


def test_mx_exact_zeros_and_closed_form():
    K, N = 1024, 40
    x = np.full((3, K), 0x3FC0, dtype=np.uint16)            # 1.5
    w_q = np.full((N, K // 2), 0x08, dtype=np.uint8)        # +0, -0
    w_e = np.full((N, K // 32), 127, dtype=np.uint8)
    assert np.all(_mx(x, w_q, w_e) == 0)
    w_q[:] = 0x77                                           # 6.0 everywhere
    w_e[:] = 125                                            # 2^-2
    assert np.all(_mx(x, w_q, w_e) == K * 1.5 * 6.0 * 0.25)


def test_mx_deterministic():
    c = synthetic.mx_case(9300, 1, 4096, 5120)
    a = _mx(c.x, c.w_q, c.w_e)
    b = _mx(c.x, c.w_q, c.w_e)
    assert np.array_equal(a, b)

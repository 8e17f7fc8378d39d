"""Parity of the HIP path with the CPU oracle, element by element.

All calls go through the C ABI (via the binding).  The bars:
  * dequantisation: bit-exact (fp32 output = the exact (c-8)*s; bf16 output
    = that value rounded nearest-even);
  * matmul: |y - y_ref| <= 1e-3 * sum_k |x_k * w_k| per output, with y_ref
    the oracle's double result; a bf16 output adds half a bf16 ulp of y_ref
    (the rounding of the store itself);
  * every path, the tiled matrix-core one included, is compared with the
    exact-weight oracle (the weights (c-8)*s unrounded);
  * integer-valued special cases (identity activations, zero codes, closed
    forms) are compared exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import DEV, dev, host, matmul, matmul_ex, moe
from helpers import RTOL, assert_parity, bf16_half_ulp, load_golden, stratified_outputs

pytestmark = pytest.mark.gpu

import quantized_q4_block_amd as q4  # noqa: E402

F32, BF16 = torch.float32, torch.bfloat16


def _check_dense(d, out_dtype=F32, what=""):
    M, K = d.x.shape
    N = d.w_q.shape[0]
    y = matmul(d.x, d.w_q, d.w_s, out_dtype)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    extra = bf16_half_ulp(y_ref) if out_dtype == BF16 else 0.0
    assert_parity(y, y_ref, t, RTOL, extra, what=what)
    return y, y_ref, t


# ------------------------------------------------------------ dequantise


def _exhaustive():
    N, K = 4096, 512
    block = np.array([(2 * j) % 16 | (((2 * j + 1) % 16) << 4) for j in range(16)], np.uint8)
    w_q = np.tile(block, (N, K // 32))
    w_s = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(N, K // 32)
    return w_q, w_s


def test_dequant_f32_exhaustive_bit_exact():
    w_q, w_s = _exhaustive()
    got = q4.q4_dequantize(dev(w_q), dev(w_s), out_dtype=F32).cpu().numpy()
    exp = oracle.dequant_f32(w_q, w_s)
    nan = np.isnan(exp)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got.view(np.uint32)[~nan], exp.view(np.uint32)[~nan])


def test_dequant_bf16_exhaustive_bit_exact():
    w_q, w_s = _exhaustive()
    got = q4.q4_dequantize(dev(w_q), dev(w_s), out_dtype=BF16).view(torch.int16).cpu().numpy()
    got = got.view(np.uint16)
    exp = oracle.dequant_bf16_bits(w_q, w_s)
    isnan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)  # noqa: E731
    nan = isnan(exp)
    assert np.array_equal(isnan(got), nan)
    assert np.array_equal(got[~nan], exp[~nan])


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (77, 640), (1000, 4096)])
def test_dequant_random_shapes(N, K):
    d = synthetic.dense_case(100 + N, 1, N, K)
    got = q4.q4_dequantize(dev(d.w_q), dev(d.w_s), out_dtype=F32).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.dequant_f32(d.w_q, d.w_s).view(np.uint32))


# --------------------------------------------------------- hand-worked


@pytest.mark.parametrize("name", ["nibble_order.txt", "two_blocks.txt"])
def test_golden_through_both_paths(name):
    g = load_golden(name)
    y = matmul(g["x"], g["w_q"], g["w_s"])                 # GEMV (M = 2)
    for m, n, v in g["y"]:
        assert y[m, n] == v, (m, n, y[m, n], v)
    # matrix-core path: pad to 16 rows by repeating the fixture rows
    x16 = np.tile(g["x"], (8, 1))
    y16 = matmul(x16, g["w_q"], g["w_s"])
    for m, n, v in g["y"]:
        for rep in range(8):
            assert y16[m + rep * len(g["x"]), n] == v


# ---------------------------------------------------------------- tiny


def test_tiny_gemv_config():
    c = synthetic.CONFIGS["tiny_gemv"]
    d = synthetic.dense_case(c["seed"], c["M"], c["N"], c["K"])
    _check_dense(d, what="tiny_gemv")


# -------------------------------------------------------- decode (GEMV)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("N,K", [(1, 32), (7, 96), (65, 2048 + 32 * 7), (300, 4096 + 32)])
def test_gemv_parity(M, N, K):
    d = synthetic.dense_case(1000 * M + N, M, N, K)
    _check_dense(d, F32, what=f"gemv M={M} N={N} K={K}")


# Long rows cut into slices (q4_matmul_ex with a workspace, matrix-vector
# path): two-stage slices of 86 (K = 8224), 108/109 (17408) and 128 (16384)
# blocks; K = 258080 (8065 blocks) takes one-stage slices; K = 5696 (178
# blocks, 3 stages) fits one workgroup and is not cut.  At M = 3, 4 the call
# takes the few-row matrix-core path: with a workspace, one K slice per 32
# blocks (the 8065-block rows, too many slices, keep the few-row kernel's
# plan).
@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(37, 8192 + 32), (300, 17408), (65, 5696), (17, 16384),
                                 (5, 258080)])
def test_gemv_split_parity(M, N, K):
    d = synthetic.dense_case(5000 + 10 * M + N, M, N, K)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    y = matmul_ex(d.x, d.w_q, d.w_s, F32)
    assert_parity(y, y_ref, t, RTOL, what=f"split M={M} N={N} K={K}")
    yb = matmul_ex(d.x, d.w_q, d.w_s, BF16)
    assert_parity(yb, y_ref, t, RTOL, bf16_half_ulp(y_ref), what=f"split bf16 M={M} N={N} K={K}")
    # without a workspace the same call takes the unsplit path
    y0 = matmul_ex(d.x, d.w_q, d.w_s, F32, workspace=None)
    assert_parity(y0, y_ref, t, RTOL, what=f"unsplit M={M} N={N} K={K}")


def test_gemv_split_deterministic_and_workspace_reuse():
    d = synthetic.dense_case(5100, 2, 300, 17408)
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    need = q4.q4_matmul_workspace_bytes(2, 300, 17408)
    assert need > 0
    work = torch.full((need,), 0x7F, dtype=torch.uint8, device=x.device)   # junk contents
    y1 = q4.q4_matmul_ex(x, wq, ws, workspace=work)
    y2 = q4.q4_matmul_ex(x, wq, ws, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # a smaller problem in the same workspace
    e = synthetic.dense_case(5101, 1, 50, 9216)
    y3 = host(q4.q4_matmul_ex(dev(e.x), dev(e.w_q), dev(e.w_s), workspace=work))
    y_ref, t = oracle.matmul(e.x, e.w_q, e.w_s)
    assert_parity(y3, y_ref, t, RTOL, what="reused workspace")
    with pytest.raises(q4.Q4Error):
        q4.q4_matmul_ex(x, wq, ws, workspace=work[: need - 16])


@pytest.mark.parametrize("M", [1, 4, 8])
def test_gemv_bf16_output(M):
    d = synthetic.dense_case(2000 + M, M, 257, 1024)
    _check_dense(d, BF16, what=f"gemv bf16 M={M}")


# ------------------------------------- few rows (exact-weight matrix cores)


# 16-row weight groups with a ragged last one (N = 1, 37, 65, 300), rows of
# 1 block, of 7 and 257 blocks (not a whole number of 4-block groups), of 129
# blocks and of 544 blocks (several groups per wavefront); M covers one and
# two 16-row activation groups with ragged ends.
@pytest.mark.parametrize("M", [3, 5, 16, 17, 32])
@pytest.mark.parametrize("N,K", [(1, 32), (37, 224), (65, 8224), (300, 4096 + 32), (64, 17408)])
def test_small_parity(M, N, K):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_SMALL
    d = synthetic.dense_case(6000 + 10 * M + N, M, N, K)
    _check_dense(d, F32, what=f"small M={M} N={N} K={K}")


# Past 32 rows while the tiled path would have fewer tiles than compute
# units: slabs of 32 activation rows (the last one ragged).
@pytest.mark.parametrize("M", [33, 64, 100, 128])
@pytest.mark.parametrize("N,K", [(300, 640), (31, 2048 + 32)])
def test_small_slab_parity(M, N, K):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_SMALL
    d = synthetic.dense_case(6500 + M + N, M, N, K)
    _check_dense(d, F32, what=f"small slabs M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [4, 24])
def test_small_bf16_output(M):
    d = synthetic.dense_case(6800 + M, M, 257, 1024)
    _check_dense(d, BF16, what=f"small bf16 M={M}")


# K slices on the few-row path (q4_matmul_ex with a workspace): slices of
# whole and ragged 4-block groups, a last slice shorter than the others, one
# and two 16-row activation groups, and slabs past 32 rows.
@pytest.mark.parametrize("M,N,K", [(4, 300, 17408), (3, 65, 8224), (16, 37, 4096 + 32),
                                   (17, 300, 2048), (32, 1, 17408), (64, 300, 2048 + 96)])
def test_small_split_parity(M, N, K):
    assert q4.q4_matmul_path_ex(M, N, K, True) == q4.Q4_PATH_SMALL
    need = q4.q4_matmul_workspace_bytes(M, N, K)
    assert need > 0
    d = synthetic.dense_case(6900 + M + N, M, N, K)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    y = matmul_ex(d.x, d.w_q, d.w_s, F32)
    assert_parity(y, y_ref, t, RTOL, what=f"small split M={M} N={N} K={K}")
    yb = matmul_ex(d.x, d.w_q, d.w_s, BF16)
    assert_parity(yb, y_ref, t, RTOL, bf16_half_ulp(y_ref), what=f"small split bf16 M={M}")


# 3..16 rows with a workspace take the sliced kernel (one slice per 32
# blocks): scales staged through LDS (K/32 a multiple of 8), loaded per lane
# in aligned groups (36 blocks: a multiple of 4 only) and one by one (65
# blocks), last slices of 4 and of 1 block, ragged 128-row weight groups,
# and both ends of its activation-row range.
@pytest.mark.parametrize("M,N,K", [(3, 300, 1152), (7, 129, 2080), (16, 257, 4096),
                                   (5, 1, 2048 + 32), (4, 640, 17408 + 128)])
def test_sliced_few_row_parity(M, N, K):
    need = q4.q4_matmul_workspace_bytes(M, N, K)
    slices = -(-(K // 32) // 32)
    assert need == slices * M * N * 4
    d = synthetic.dense_case(6950 + M + N, M, N, K)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    y = matmul_ex(d.x, d.w_q, d.w_s, F32)
    assert_parity(y, y_ref, t, RTOL, what=f"sliced M={M} N={N} K={K}")
    yb = matmul_ex(d.x, d.w_q, d.w_s, BF16)
    assert_parity(yb, y_ref, t, RTOL, bf16_half_ulp(y_ref), what=f"sliced bf16 M={M}")


@pytest.mark.parametrize("M", [4, 16])
@pytest.mark.parametrize("kind", ["normal", "huge", "tiny", "zero_rows", "wide", "subnormal",
                                  "rows_apart"])
def test_sliced_few_row_activation_ranges(M, kind):
    """The sliced kernel takes fp16 operands when a slice's nonzero
    activations span at most 2^29 (scaled by one power of two: by about
    2^-100 for "huge", 2^100 for "tiny", not at all for "normal" and
    "zero_rows") and exact bf16 ones otherwise ("wide": a value 2^63 times
    the rest; "subnormal"; "rows_apart": one row 2^40 below the others).
    Either way the bar is exact-weight parity, and zero rows give zero."""
    N, K = 300, 4096
    d = synthetic.dense_case(6960 + M, M, N, K)
    x = d.x.copy()
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    if kind == "huge":
        x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** 100))
    elif kind == "tiny":
        x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** -100))
    elif kind == "zero_rows":
        x[1::2] = 0
    elif kind == "wide":
        x[:, 7] = 0x5F00            # ~9.2e18 next to O(1) values
    elif kind == "subnormal":
        x[:, 100] = 0x0003
    elif kind == "rows_apart":
        x[M - 1] = synthetic.f32_to_bf16_bits(xf[M - 1] * np.float32(2.0 ** -40))
    assert q4.q4_matmul_workspace_bytes(M, N, K) == 4 * M * N * 4
    y_ref, t = oracle.matmul(x, d.w_q, d.w_s)
    y = matmul_ex(x, d.w_q, d.w_s, F32)
    assert_parity(y, y_ref, t, RTOL, what=f"sliced {kind} M={M}")
    for m in range(M):
        if not x[m].any():
            assert np.all(y[m] == 0)


def test_sliced_few_row_two_spikes():
    """Unit scales and two nonzero activations per row: the sliced kernel's
    result is the oracle's double result rounded to fp32 within one fp32 ulp
    (one MFMA sum and at most one fp32 addition per slice and in the
    combine), on both operand paths: spreads up to 2^29 take fp16 operands,
    2^30 and more the bf16 ones."""
    M, N, K = 4, 130, 4096
    d = synthetic.dense_case(6970, M, N, K)
    w_s = np.full_like(d.w_s, 0x3C00)                       # 1.0
    rng = np.random.default_rng(13)
    for a in (60, 15, 0, -14, -60):
        for spread in (0, 28, 29, 30, 45):
            x = np.stack([_two_spikes(K, k0, k1, a, spread, rng)
                          for k0, k1 in ((96, 100), (100, 101), (100, 2100), (17, K - 20))])
            y = matmul_ex(x, d.w_q, w_s, F32)
            y_ref, _ = oracle.matmul(x, d.w_q, w_s)
            want = y_ref.astype(np.float32).astype(np.float64)
            ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
            assert np.all(np.abs(y - want) <= ulp), f"a={a} spread={spread}"


def test_small_split_deterministic_and_workspace_reuse():
    M, N, K = 4, 300, 17408
    d = synthetic.dense_case(6950, M, N, K)
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    need = q4.q4_matmul_workspace_bytes(M, N, K)
    work = torch.full((need,), 0x7F, dtype=torch.uint8, device=x.device)   # junk contents
    y1 = q4.q4_matmul_ex(x, wq, ws, workspace=work)
    y2 = q4.q4_matmul_ex(x, wq, ws, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    e = synthetic.dense_case(6951, 5, 64, 2048)
    y3 = host(q4.q4_matmul_ex(dev(e.x), dev(e.w_q), dev(e.w_s), workspace=work))
    y_ref, t = oracle.matmul(e.x, e.w_q, e.w_s)
    assert_parity(y3, y_ref, t, RTOL, what="small split, reused workspace")
    with pytest.raises(q4.Q4Error):
        q4.q4_matmul_ex(x, wq, ws, workspace=work[: need - 16])


# ---------------------------------------------------- prefill (MFMA)


# Tiled path: more than 128 rows, or 33..128 rows with at least 256 tiles
# (N >= 32641); ragged tiles in M, N and K steps of 64.
@pytest.mark.parametrize("M,N,K", [(33, 34816, 64), (100, 32641 + 30, 96), (128, 34816, 32),
                                   (129, 257, 1024), (256, 384, 2048 + 32), (300, 77, 160),
                                   (129, 1, 32)])
def test_mfma_parity(M, N, K):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_MFMA
    d = synthetic.dense_case(3000 + M + N, M, N, K)
    _check_dense(d, F32, what=f"mfma M={M} N={N} K={K}")


# More than 128 rows with K a multiple of 64 take tiles of 256 x 128: one
# tile partly filled, a tile edge at 256 rows and one past it, ragged weight
# tiles, one K step and an odd number of them.
@pytest.mark.parametrize("M,N,K", [(129, 128, 64), (256, 129, 128), (257, 300, 64 * 5),
                                   (511, 1000, 1024), (513, 64, 64 * 3), (700, 257, 2048)])
def test_mfma_wide_tile_parity(M, N, K):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_MFMA
    d = synthetic.dense_case(3500 + M + N, M, N, K)
    _check_dense(d, F32, what=f"mfma wide M={M} N={N} K={K}")
    _check_dense(d, BF16, what=f"mfma wide bf16 M={M} N={N} K={K}")


# With a workspace, a grid of wide tiles that fills whole rounds of the chip
# (256 tiles) and a last round at most half full cuts the last round's tiles
# along K: 258 tiles (2 of them in the tail, 4 slices of 4 steps), 300 tiles
# (44 in the tail, 5 slices of 4 steps, a ragged last M tile and N tile).
@pytest.mark.parametrize("M,N,K,tail,slices", [(257, 128 * 128 + 1, 1024, 2, 4),
                                               (300, 150 * 128 - 5, 64 * 20, 44, 5)])
def test_mfma_wide_tail_parity(M, N, K, tail, slices):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_workspace_bytes(M, N, K) == tail * slices * 256 * 128 * 4
    d = synthetic.dense_case(3600 + M, M, N, K)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    y = matmul_ex(d.x, d.w_q, d.w_s, F32)
    assert_parity(y, y_ref, t, RTOL, what=f"wide tail M={M} N={N} K={K}")
    yb = matmul_ex(d.x, d.w_q, d.w_s, BF16)
    assert_parity(yb, y_ref, t, RTOL, bf16_half_ulp(y_ref), what=f"wide tail bf16 M={M}")


@pytest.mark.parametrize("M,N,K", [(160, 200, 512), (512, 256, 5120)])
def test_mfma_bf16_output(M, N, K):
    d = synthetic.dense_case(4000 + M, M, N, K)
    _check_dense(d, BF16, what=f"mfma bf16 M={M}")


# K slices on the tiled path: q4_matmul_ex with a workspace cuts grids of
# fewer than 512 tiles along K (2 to 64 slices of at least 8 K steps, the
# last one ragged), then adds the fp32 slice sums in order.  M * N = 33153
# and 23100 take the combine kernel's scalar and 16-byte forms.
@pytest.mark.parametrize("M,N,K", [(129, 257, 1024), (256, 384, 2048 + 64 * 3),
                                   (300, 77, 64 * 37), (512, 640, 5120), (200, 128, 64 * 520)])
def test_mfma_split_parity(M, N, K):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_workspace_bytes(M, N, K) >= 2 * M * N * 4
    d = synthetic.dense_case(4100 + M + N, M, N, K)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    y = matmul_ex(d.x, d.w_q, d.w_s, F32)
    assert_parity(y, y_ref, t, RTOL, what=f"mfma split M={M} N={N} K={K}")
    yb = matmul_ex(d.x, d.w_q, d.w_s, BF16)
    assert_parity(yb, y_ref, t, RTOL, bf16_half_ulp(y_ref), what=f"mfma split bf16 M={M}")
    y0 = matmul_ex(d.x, d.w_q, d.w_s, F32, workspace=None)
    assert_parity(y0, y_ref, t, RTOL, what=f"mfma unsplit M={M} N={N} K={K}")


# With a workspace, 33..128 rows on weight matrices of at least 2^24 entries
# leave the few-row slabs for the tiled kernel cut along K; without one the
# same shapes stay on the slabs.  Both use exact weights.
@pytest.mark.parametrize("M,N,K", [(33, 4096, 4096 + 64 * 3), (100, 5120, 5120), (128, 2048, 8192)])
def test_slab_shapes_with_a_workspace(M, N, K):
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_SMALL
    assert q4.q4_matmul_path_ex(M, N, K, True) == q4.Q4_PATH_MFMA
    d = synthetic.dense_case(4300 + M, M, N, K)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    y = matmul_ex(d.x, d.w_q, d.w_s, F32)
    assert_parity(y, y_ref, t, RTOL, what=f"slab shape tiled M={M} N={N} K={K}")
    yb = matmul_ex(d.x, d.w_q, d.w_s, BF16)
    assert_parity(yb, y_ref, t, RTOL, bf16_half_ulp(y_ref), what=f"slab shape tiled bf16 M={M}")
    y0 = matmul_ex(d.x, d.w_q, d.w_s, F32, workspace=None)
    assert_parity(y0, y_ref, t, RTOL, what=f"slab shape slabs M={M} N={N} K={K}")


def test_prefill_down_split_sampled_and_deterministic():
    """The prefill FFN's down projection (512 x 5120 x 17408: 80 tiles of 256 x 128) with
    a workspace, against sampled outputs of the oracle; junk workspace
    contents do not matter and two calls agree bit for bit."""
    M, N, K = 512, 5120, 17408
    d = synthetic.dense_case(4200, M, N, K)
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    need = q4.q4_matmul_workspace_bytes(M, N, K)
    assert need == 3 * M * N * 4
    work = torch.full((need,), 0x7F, dtype=torch.uint8, device=x.device)
    y1 = q4.q4_matmul_ex(x, wq, ws, out_dtype=BF16, workspace=work)
    y2 = q4.q4_matmul_ex(x, wq, ws, out_dtype=BF16, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y = host(y1)
    ms, ns = stratified_outputs(M, N)
    y_ref, t = oracle.matmul_sampled(d.x, d.w_q, d.w_s, ms, ns)
    assert_parity(y[ms, ns], y_ref, t, RTOL, bf16_half_ulp(y_ref), what="prefill down split")


# ------------------------------------------------- exact special cases


def test_identity_activations_give_dequantised_weights():
    """x = I (K x K): y[m][n] = w[n][m], the exact fp32 weights, on the tiled
    matrix-core path (M = 256; in bf16 output, their nearest-even rounding),
    the few-row matrix-core path and the matrix-vector path (row slices)."""
    K, N = 256, 192
    d = synthetic.dense_case(5000, 1, N, K)
    eye = np.zeros((K, K), dtype=np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    assert q4.q4_matmul_path(K, N, K) == q4.Q4_PATH_MFMA
    wf = oracle.dequant_f32(d.w_q, d.w_s).astype(np.float64)
    y = matmul(eye, d.w_q, d.w_s)                      # M = 256: tiled
    assert np.array_equal(y, wf.T)
    yb = matmul(eye, d.w_q, d.w_s, BF16)
    wb = oracle.dequant_bf16_bits(d.w_q, d.w_s)
    assert np.array_equal(yb, (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64).T)
    for m0 in range(0, K, 8):                           # M = 8 slices: few-row path
        ys = matmul(eye[m0:m0 + 8], d.w_q, d.w_s)
        assert np.array_equal(ys, wf[:, m0:m0 + 8].T)
    for m0 in (0, 30, 254):                             # M = 2: matrix-vector
        ys = matmul(eye[m0:m0 + 2], d.w_q, d.w_s)
        assert np.array_equal(ys, wf[:, m0:m0 + 2].T)
    for m0 in (0, 31, 32, 255):                         # M = 1, across block edges
        ys = matmul(eye[m0:m0 + 1], d.w_q, d.w_s)
        assert np.array_equal(ys[0], wf[:, m0])


@pytest.mark.parametrize("M", [1, 4, 64])
def test_zero_codes_give_exact_zero(M):
    d = synthetic.dense_case(5100 + M, M, 130, 512)
    w_q = np.full_like(d.w_q, 0x88)
    y = matmul(d.x, w_q, d.w_s)
    assert np.all(y == 0)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_sparse_codes_exact_per_weight(M):
    """Nearly every code 8 (weight 0): the GEMV path's exact weights keep the
    tolerance even though sum |x*w| is tiny next to sum |x|."""
    d = synthetic.dense_case(5200 + M, M, 64, 1024)
    rng = np.random.default_rng(7)
    w_q = np.full_like(d.w_q, 0x88)
    hit = rng.random(w_q.shape) < 0.01
    w_q[hit] = d.w_q[hit]
    y = matmul(d.x, w_q, d.w_s)
    y_ref, t = oracle.matmul(d.x, w_q, d.w_s)
    assert_parity(y, y_ref, t, RTOL, what="sparse codes")


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("kind", ["wide", "subnormal", "huge", "tiny"])
def test_gemv_activation_ranges(M, kind):
    """Activation rows of extreme range: a value 2^63 times the rest, a bf16
    subnormal, and every value scaled by 2^100 or 2^-100."""
    N, K = 200, 5120
    d = synthetic.dense_case(5300 + M, M, N, K)
    x = d.x.copy()
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    if kind == "wide":
        x[:, 7] = 0x5F00            # ~9.2e18 next to O(1) values
    elif kind == "subnormal":
        x[:, 100] = 0x0003          # bf16 subnormal
    elif kind == "huge":
        x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** 100))
    else:
        x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** -100))
    y = matmul(x, d.w_q, d.w_s)
    y_ref, t = oracle.matmul(x, d.w_q, d.w_s)
    assert_parity(y, y_ref, t, RTOL, what=f"range {kind} M={M}")


def _two_spikes(K, k0, k1, a, spread, rng):
    """A bf16 row that is zero but for x[k0] = +-2^a (1 + f) and
    x[k1] = +-2^(a - spread) (1 + g), f and g random 7-bit fractions."""
    x = np.zeros(K, np.float32)
    for k, e in ((k0, a), (k1, a - spread)):
        frac = 1.0 + rng.integers(0, 128) / 128.0
        x[k] = np.float32(rng.choice([-1.0, 1.0]) * frac * 2.0 ** e)
    return synthetic.f32_to_bf16_bits(x)


# (k0, k1): both spikes in one dword (k and k + 4; k and k + 1), in stages 0
# and 1, and the second one in the leftover stage
def _spikes(K):
    return [(96, 100), (100, 101), (100, 2100), (17, K - 20)]


@pytest.mark.parametrize("K", [5120, 2048 + 32 * 40])
def test_gemv_two_spikes_exactly_rounded(K):
    """With unit scales and two nonzero activations per row, the decode
    kernel forms y[n] = (c0 - 8) x0 + (c1 - 8) x1 with a single rounding
    (every product is exact and every other term is an exact zero), so y
    must be the oracle's double result rounded to fp32, bit for bit, for
    spikes up to 2^45 apart and at both ends of the exponent range."""
    N = 130
    d = synthetic.dense_case(5350, 1, N, K)
    w_s = np.full_like(d.w_s, 0x3C00)                       # 1.0
    rng = np.random.default_rng(11)
    for k0, k1 in _spikes(K):
        for a in (100, 40, 15, 3, 0, -14, -40, -70):
            for spread in (0, 1, 15, 28, 29, 30, 31, 45):
                x = _two_spikes(K, k0, k1, a, spread, rng)[None, :]
                y = matmul(x, d.w_q, w_s)[0]
                y_ref, _ = oracle.matmul(x, d.w_q, w_s)
                want = y_ref[0].astype(np.float32).astype(np.float64)
                assert np.array_equal(y, want), f"K={K} k=({k0},{k1}) a={a} spread={spread}"


def test_gemv_two_rows_of_different_ranges():
    """M = 2: a random row next to a row of two values 2^40 apart, next to an
    all-zero row, and two zero rows; a zero row gives exactly zero."""
    N, K = 200, 5120
    d = synthetic.dense_case(5360, 2, N, K)
    x = d.x.copy()
    odd = _two_spikes(K, 10, 4000, 5, 40, np.random.default_rng(12))
    zero = np.zeros(K, np.uint16)
    for rows in (np.stack([x[0], odd]), np.stack([odd, x[1]]), np.stack([x[0], zero]),
                 np.stack([zero, zero])):
        y = matmul(rows, d.w_q, d.w_s)
        y_ref, t = oracle.matmul(rows, d.w_q, d.w_s)
        assert_parity(y, y_ref, t, RTOL, what="two rows")
        for m in range(2):
            if not rows[m].any():
                assert np.all(y[m] == 0)


@pytest.mark.parametrize("M", [1, 16])
def test_closed_form_constant(M):
    K, N = 512, 70
    x = np.full((M, K), 0x3FC0, dtype=np.uint16)          # 1.5
    w_q = np.full((N, K // 2), 0xDD, dtype=np.uint8)      # code 13 -> +5
    w_s = np.full((N, K // 32), 0x2C00, dtype=np.uint16)  # 2^-4
    y = matmul(x, w_q, w_s)
    assert np.all(y == K * 1.5 * 5 * 2.0 ** -4)


@pytest.mark.parametrize("M,K", [(129, 512), (256, 5120), (300, 2048 + 32)])
@pytest.mark.parametrize("code,factor", [(0x99, 1), (0xFF, 7), (0x00, -8)])
def test_tiled_closed_form_scale_outside_bf16(M, K, code, factor):
    """Tiled path, x = 1, every code the same, scale fp16 0x3C03 = 1.0029296875
    (11 significant bits, not a bf16 value): y = K * (c - 8) * 1.0029296875
    exactly (every partial sum is a small multiple of the scale)."""
    N = 257
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_MFMA
    x = np.full((M, K), 0x3F80, dtype=np.uint16)
    w_q = np.full((N, K // 2), code, dtype=np.uint8)
    w_s = np.full((N, K // 32), 0x3C03, dtype=np.uint16)
    y = matmul(x, w_q, w_s)
    assert np.all(y == K * factor * 1.0029296875)
    y_ref, t = oracle.matmul(x, w_q, w_s)
    assert_parity(y, y_ref, t, RTOL, what="tiled closed form")


@pytest.mark.parametrize("kind", ["wide", "subnormal", "huge", "tiny", "sparse"])
def test_tiled_activation_ranges_and_sparse_codes(kind):
    """The tiled path on inputs where rounded weights or scaled activations
    would break the bar: an activation 2^63 times the rest whose weight is
    zero, bf16 subnormal activations, both ends of bf16's range, and nearly
    all codes 8 (sum |x w| tiny next to sum |x|)."""
    M, N, K = 160, 200, 2048
    d = synthetic.dense_case(5400, M, N, K)
    x, w_q = d.x.copy(), d.w_q.copy()
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    if kind == "wide":
        x[:, 7] = 0x5F00            # ~9.2e18
        w_q[:, 3] = (w_q[:, 3] & 0x0F) | 0x80   # its weight (k = 7, high nibble) is 0
    elif kind == "subnormal":
        x[:, 100] = 0x0003
        x[::3, 5] = 0x8001
    elif kind == "huge":
        x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** 100))
    elif kind == "tiny":
        x = synthetic.f32_to_bf16_bits(xf * np.float32(2.0 ** -100))
    else:
        rng = np.random.default_rng(8)
        hit = rng.random(w_q.shape) < 0.01
        w_q = np.where(hit, d.w_q, 0x88).astype(np.uint8)
    assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_MFMA
    y = matmul(x, w_q, d.w_s)
    y_ref, t = oracle.matmul(x, w_q, d.w_s)
    assert_parity(y, y_ref, t, RTOL, what=f"tiled {kind}")


# ------------------------------------------------------ full-size configs


def _full_dense(name, out_dtype):
    c = synthetic.CONFIGS[name]
    d = synthetic.dense_case(c["seed"], c["M"], c["N"], c["K"])
    y = matmul(d.x, d.w_q, d.w_s, out_dtype)
    return d, y


def test_decode_gate_up_full_size():
    d, y = _full_dense("decode_gate_up", F32)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    assert_parity(y, y_ref, t, RTOL, what="decode_gate_up")


def test_batched_down_full_size():
    d, y = _full_dense("batched_down", F32)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    assert_parity(y, y_ref, t, RTOL, what="batched_down")
    y = matmul_ex(d.x, d.w_q, d.w_s, F32)           # K slices in the workspace
    assert_parity(y, y_ref, t, RTOL, what="batched_down through q4_matmul_ex")


def test_prefill_full_size_stratified():
    """The prefill workload (512 x 34816 x 5120, bf16 output) against the
    exact-weight oracle on one output of every column, spread so that every
    row and every 128 x 128 output tile is hit."""
    d, y = _full_dense("prefill", BF16)
    M, N = y.shape
    ms, ns = stratified_outputs(M, N)
    assert len(set(ms.tolist())) == M and len(set(ns.tolist())) == N
    assert len(set(zip((ms // 128).tolist(), (ns // 128).tolist()))) == (M // 128) * (N // 128)
    y_ref, t = oracle.matmul_sampled(d.x, d.w_q, d.w_s, ms, ns)
    assert_parity(y[ms, ns], y_ref, t, RTOL, bf16_half_ulp(y_ref), what="prefill")
    assert np.isfinite(y).all()
    # as the benchmark calls it: q4_matmul_ex with its workspace, where the
    # 32 tiles of the last round (columns 32768 and up) are cut into 8 K
    # slices each; a junk workspace does not matter and two calls agree
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    need = q4.q4_matmul_workspace_bytes(M, N, d.x.shape[1])
    assert need == 32 * 8 * 256 * 128 * 4
    work = torch.full((need,), 0x7F, dtype=torch.uint8, device=x.device)
    y1 = q4.q4_matmul_ex(x, wq, ws, out_dtype=BF16, workspace=work)
    y2 = q4.q4_matmul_ex(x, wq, ws, out_dtype=BF16, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ye = host(y1)
    assert_parity(ye[ms, ns], y_ref, t, RTOL, bf16_half_ulp(y_ref), what="prefill with workspace")
    assert np.isfinite(ye).all()
    # the whole tiles are the same computation either way
    assert np.array_equal(ye[:, :32768].view(np.uint16), y[:, :32768].view(np.uint16))


# ------------------------------------------------------------------ MoE


def test_moe_config_full():
    c = synthetic.CONFIGS["moe"]
    m = synthetic.moe_case(c["seed"], c["T"], c["topk"], c["E"], c["N"], c["K"])
    y = moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    assert_parity(y, y_ref, t, RTOL, what="moe")


# Up to 64 (token, slot) pairs with few pairs per expert over at most 256
# experts, the expert workgroups find their pairs from the ids themselves (no
# prep kernel); (40, 2, 64, ...) has 80 pairs and (4, 2, 300, ...) 300
# experts, and both take the prep kernel's buckets; (64, 2, 4, ...) and (80,
# 8, 16, ...) have many pairs per expert and take the grouped matrix-core
# product; K = 8192 + 32 (more than 4 stages) takes the chunked
# global-activation kernel.  K of 37 and 48 blocks: rows of one leftover
# stage spread over all lanes (without and with the prep).
@pytest.mark.parametrize("T,topk,E,N,K", [(1, 1, 1, 33, 64), (5, 3, 4, 100, 256),
                                          (64, 2, 4, 96, 512), (3, 4, 50, 70, 2048 + 32),
                                          (40, 2, 64, 96, 1024 + 32), (4, 2, 300, 40, 256),
                                          (5, 2, 9, 70, 37 * 32), (40, 2, 64, 50, 48 * 32),
                                          (80, 8, 16, 40, 256), (4, 2, 6, 20, 8192 + 32)])
def test_moe_parity_shapes(T, topk, E, N, K):
    m = synthetic.moe_case(6000 + T + E, T, topk, E, N, K)
    y = moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    assert_parity(y, y_ref, t, RTOL, what=f"moe T={T} topk={topk} E={E}")


def test_moe_top1_unit_gate_equals_dense():
    T, E, N, K = 6, 5, 96, 1024
    m = synthetic.moe_case(6100, T, 1, E, N, K)
    gates = np.ones((T, 1), dtype=np.float32)
    y = moe(m.x, m.w_q, m.w_s, m.ids, gates)
    for tok in range(T):
        e = int(m.ids[tok, 0])
        yd = matmul(m.x[tok:tok + 1], m.w_q[e], m.w_s[e])
        assert np.array_equal(y[tok], yd[0])


def test_moe_repeated_and_invalid_ids():
    T, topk, E, N, K = 4, 4, 6, 64, 256
    m = synthetic.moe_case(6200, T, topk, E, N, K)
    ids = m.ids.copy()
    ids[0, 1] = ids[0, 0]      # repeated id: summed
    ids[1, 2] = E              # out of range: ignored
    ids[2, 3] = -5
    y = moe(m.x, m.w_q, m.w_s, ids, m.gates)
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, ids, m.gates)
    assert_parity(y, y_ref, t, RTOL, what="moe repeated/invalid ids")


def test_moe_prep_free_one_expert_takes_every_pair():
    # 64 pairs over 200 experts, all but two on expert 7 (one id invalid):
    # the prep-free path runs one expert's 62 pairs in a row
    T, topk, E, N, K = 8, 8, 200, 72, 1024 + 32
    m = synthetic.moe_case(6300, T, topk, E, N, K)
    ids = np.full((T, topk), 7, dtype=np.int32)
    ids[3, 5] = 199
    ids[6, 0] = -1
    y = moe(m.x, m.w_q, m.w_s, ids, m.gates)
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, ids, m.gates)
    assert_parity(y, y_ref, t, RTOL, what="moe, one expert takes every pair")


def test_moe_deterministic_and_workspace_reuse():
    c = synthetic.CONFIGS["moe"]
    m = synthetic.moe_case(c["seed"], c["T"], c["topk"], 32, 256, 1024)
    x, wq, ws, ids, g = dev(m.x), dev(m.w_q), dev(m.w_s), dev(m.ids), dev(m.gates)
    need = q4.q4_moe_workspace_bytes(c["T"], c["topk"], 32, 256)
    wsp = torch.full((need,), 0x5A, dtype=torch.uint8, device=x.device)   # garbage contents
    outs = [q4.q4_moe_matmul(x, wq, ws, ids, g, workspace=wsp).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


# ---------------------------------------------- run-to-run and guard bands


def test_run_to_run_bit_identical():
    for M in (1, 4, 200):
        d = synthetic.dense_case(7000 + M, M, 1000, 2048)
        x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
        a = q4.q4_matmul(x, wq, ws)
        b = q4.q4_matmul(x, wq, ws)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), M


@pytest.mark.parametrize("M,out_dtype", [(1, F32), (3, BF16), (40, F32), (40, BF16)])
def test_output_guard_bands_untouched(M, out_dtype):
    N, K = 333, 640
    d = synthetic.dense_case(7100 + M, M, N, K)
    pad = 64
    buf = torch.full((M * N + 2 * pad,), 7.0, dtype=out_dtype, device="cuda:0")
    y = buf[pad:pad + M * N].view(M, N)
    q4.q4_matmul(dev(d.x), dev(d.w_q), dev(d.w_s), out=y)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + M * N:] == 7.0)
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    extra = bf16_half_ulp(y_ref) if out_dtype == BF16 else 0.0
    assert_parity(host(y), y_ref, t, RTOL, extra, what="guard")


def test_errors_leave_output_untouched():
    import ctypes
    d = synthetic.dense_case(7200, 2, 64, 256)
    y = torch.full((2, 64), 3.0, device="cuda:0")
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    P = ctypes.c_void_p
    # x two bytes past an aligned address: rejected before any launch
    st = q4.lib.q4_matmul(P(x.data_ptr() + 2), P(wq.data_ptr()), P(ws.data_ptr()),
                          P(y.data_ptr()), q4.Q4_F32, 2, 64, 256, None)
    assert st == q4.Q4_ERR_ALIGN
    st = q4.lib.q4_matmul(P(x.data_ptr()), P(wq.data_ptr()), P(ws.data_ptr()),
                          P(y.data_ptr()), q4.Q4_F32, 2, 64, 250, None)
    assert st == q4.Q4_ERR_SHAPE
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)


def test_non_default_stream():
    d = synthetic.dense_case(7300, 4, 500, 1024)
    s = torch.cuda.Stream()
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = q4.q4_matmul(x, wq, ws, stream=s)
    s.synchronize()
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    assert_parity(host(y), y_ref, t, RTOL, what="stream")


@pytest.mark.parametrize("M,N,K", [(2, 300, 17408), (4, 300, 17408), (300, 200, 64 * 40)])
def test_split_calls_on_a_non_default_stream(M, N, K):
    """The cut calls (matrix-vector slices, few-row and tiled K slices) put their product
    and their combine kernel on the caller's stream; the workspace is
    allocated on that stream too."""
    d = synthetic.dense_case(7400 + M, M, N, K)
    need = q4.q4_matmul_workspace_bytes(M, N, K)
    assert need > 0
    s = torch.cuda.Stream()
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        work = torch.full((need,), 0x7F, dtype=torch.uint8, device=x.device)
        y = q4.q4_matmul_ex(x, wq, ws, workspace=work, stream=s)
    s.synchronize()
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    assert_parity(host(y), y_ref, t, RTOL, what=f"split on a stream M={M}")


def test_auto_workspace_on_a_stream_that_is_not_current():
    """A call given stream=s while another stream is current: the binding's
    temporary workspace belongs to s, so allocations made on the current
    stream right after the call (which reuse freed blocks) cannot take it
    while the call's kernels still run."""
    M, N, K = 300, 200, 64 * 40
    d = synthetic.dense_case(7500, M, N, K)
    m = synthetic.moe_case(7501, 8, 4, 16, 512, 1024)
    x, wq, ws = dev(d.x), dev(d.w_q), dev(d.w_s)
    mx, mwq, mws, mids, mg = dev(m.x), dev(m.w_q), dev(m.w_s), dev(m.ids), dev(m.gates)
    assert q4.q4_matmul_workspace_bytes(M, N, K) > 0
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    assert torch.cuda.current_stream() != s
    y = q4.q4_matmul_ex(x, wq, ws, stream=s)
    ym = q4.q4_moe_matmul(mx, mwq, mws, mids, mg, stream=s)
    junk = [torch.full((1 << 20,), 1e30, device=DEV) for _ in range(8)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    y_ref, t = oracle.matmul(d.x, d.w_q, d.w_s)
    assert_parity(host(y), y_ref, t, RTOL, what="matmul_ex on a stream that is not current")
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    assert_parity(host(ym), y_ref, t, RTOL, what="moe on a stream that is not current")

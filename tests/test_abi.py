"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU.

None of these tests needs a GPU.  Calls with valid arguments and fake
device pointers are made only where no GPU is present (they must then stop
at the device check); on a machine with a GPU those cases are skipped so a
fake pointer is never launched on.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


def _lib():
    q4 = pytest.importorskip("quantized_q4_block_amd")
    return q4, q4.lib


def _header():
    return open(HEADER).read()


def _declared_symbols():
    return re.findall(r"^Q4_API\s+[^(]*?\b(q4_\w+)\s*\(", _header(), flags=re.M)


def _defines():
    return {k: int(v) for k, v in re.findall(r"^#define\s+(Q4_\w+)\s+(-?\d+)", _header(), flags=re.M)}


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def test_header_declares_the_abi():
    syms = _declared_symbols()
    assert set(syms) == {"q4_abi_version", "q4_status_str", "q4_matmul_path", "q4_matmul_path_ex",
                         "q4_matmul",
                         "q4_matmul_workspace_bytes", "q4_matmul_ex", "q4_dequantize",
                         "q4_rmsnorm_matmul_workspace_bytes", "q4_rmsnorm_matmul", "q4_quantize",
                         "q4_sb_matmul_workspace_bytes", "q4_sb_matmul",
                         "q4_moe_workspace_bytes", "q4_moe_matmul", "q4_moe_matmul_noalloc",
                         "q4_moe_ffn_workspace_bytes",
                         "q4_moe_ffn", "q4_moe_ffn_ex", "q4_mx_matmul",
                         "q4_mx_matmul_workspace_bytes",
                         "q4_mx_matmul_ex", "q4_stream_read_sink_words", "q4_stream_read"}


def test_every_declared_symbol_is_exported():
    q4, L = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", q4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for s in _declared_symbols():
        assert s in exported, s
        getattr(L, s)
    # nothing but the ABI leaks out of the library
    assert {s for s in exported if s.startswith("q4")} == set(_declared_symbols())


def test_constants_match_header():
    q4, L = _lib()
    d = _defines()
    for name in ("Q4_ABI_VERSION", "Q4_OK", "Q4_ERR_NULL", "Q4_ERR_SHAPE", "Q4_ERR_ALIGN",
                 "Q4_ERR_DTYPE", "Q4_ERR_WORKSPACE", "Q4_ERR_DEVICE", "Q4_ERR_LAUNCH",
                 "Q4_ERR_PENDING", "Q4_ERR_SCRATCH", "Q4_ERR_FLAGS", "Q4_MOE_WEIGHTED_DOWN",
                 "Q4_F32", "Q4_BF16", "Q4_PATH_GEMV", "Q4_PATH_MFMA", "Q4_PATH_SMALL"):
        assert getattr(q4, name) == d[name], name
    assert L.q4_abi_version() == d["Q4_ABI_VERSION"]


def test_status_strings():
    q4, L = _lib()
    seen = set()
    for code in range(0, 11):
        s = q4.q4_status_str(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 11
    assert q4.q4_status_str(99) == "unknown status"
    assert q4.q4_status_str(-1) == "unknown status"


def test_path_dispatch():
    q4, _ = _lib()
    for N, K in ((34816, 5120), (5120, 17408), (7, 32)):
        for M in range(0, 3):
            assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_GEMV
        for M in (3, 4, 8, 9, 16, 17, 32):
            assert q4.q4_matmul_path(M, N, K) == q4.Q4_PATH_SMALL
    # past 32 rows: tiles of 128 x 128 decide (fewer than 256 -> small path,
    # up to 128 rows)
    assert q4.q4_matmul_path(33, 34816, 5120) == q4.Q4_PATH_MFMA      # 272 tiles
    assert q4.q4_matmul_path(128, 32640, 5120) == q4.Q4_PATH_SMALL    # 255 tiles
    assert q4.q4_matmul_path(128, 32641, 5120) == q4.Q4_PATH_MFMA     # 256 tiles
    assert q4.q4_matmul_path(64, 5120, 17408) == q4.Q4_PATH_SMALL
    assert q4.q4_matmul_path(129, 5120, 17408) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_path(512, 34816, 5120) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_path(1 << 20, 64, 64) == q4.Q4_PATH_MFMA
    # with a workspace: 33..128 rows on large weights leave the slabs for the
    # tiled kernel cut along K; small matrices, K % 64 != 0 and <= 32 rows stay
    assert q4.q4_matmul_path_ex(64, 5120, 17408, False) == q4.Q4_PATH_SMALL
    assert q4.q4_matmul_path_ex(64, 5120, 17408, True) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_path_ex(33, 5120, 5120, True) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_path_ex(128, 1024, 4096, True) == q4.Q4_PATH_SMALL    # 2^22 weights
    assert q4.q4_matmul_path_ex(64, 5120, 17408 + 32, True) == q4.Q4_PATH_SMALL
    assert q4.q4_matmul_path_ex(32, 5120, 17408, True) == q4.Q4_PATH_SMALL
    assert q4.q4_matmul_path_ex(1, 5120, 17408, True) == q4.Q4_PATH_GEMV
    assert q4.q4_matmul_path_ex(512, 34816, 5120, True) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_path_ex(-1, 64, 64, True) == -1
    # sizes far past any device: answers without overflowing a product
    assert q4.q4_matmul_path(1 << 40, 1 << 40, 64) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_path_ex(100, 1 << 40, 1 << 40, True) == q4.Q4_PATH_MFMA
    assert q4.q4_matmul_workspace_bytes(1 << 40, 1 << 40, 64) == 0
    assert q4.q4_matmul_workspace_bytes(100, 1 << 40, 1 << 30) == 0
    for bad in ((-1, 8, 32), (4, -1, 32), (4, 8, 0), (4, 8, 48)):
        assert q4.q4_matmul_path(*bad) == -1


A = 1 << 20          # a 16-byte aligned fake address
MIS = A + 8          # misaligned


def _mm(L, x=A, wq=A, ws=A, y=A, dt=0, M=1, N=32, K=64):
    P = ctypes.c_void_p
    return L.q4_matmul(P(x), P(wq), P(ws), P(y), dt, M, N, K, None)


def test_matmul_argument_errors():
    q4, L = _lib()
    assert _mm(L, dt=2) == q4.Q4_ERR_DTYPE
    assert _mm(L, dt=-1) == q4.Q4_ERR_DTYPE
    assert _mm(L, K=0) == q4.Q4_ERR_SHAPE
    assert _mm(L, K=48) == q4.Q4_ERR_SHAPE
    assert _mm(L, K=-32) == q4.Q4_ERR_SHAPE
    assert _mm(L, N=-1) == q4.Q4_ERR_SHAPE
    assert _mm(L, M=-1) == q4.Q4_ERR_SHAPE
    assert _mm(L, M=1 << 40, N=1 << 40) == q4.Q4_ERR_SHAPE
    assert _mm(L, N=1 << 40, K=1 << 40) == q4.Q4_ERR_SHAPE
    # dtype is checked before shape
    assert _mm(L, dt=7, K=3) == q4.Q4_ERR_DTYPE
    # zero-size calls are no-ops, even with NULL pointers
    assert _mm(L, x=0, wq=0, ws=0, y=0, M=0) == q4.Q4_OK
    assert _mm(L, x=0, wq=0, ws=0, y=0, N=0) == q4.Q4_OK
    # NULL, then alignment
    for kw in ("x", "wq", "ws", "y"):
        assert _mm(L, **{kw: 0}) == q4.Q4_ERR_NULL, kw
        assert _mm(L, **{kw: MIS}) == q4.Q4_ERR_ALIGN, kw
    # shape errors win over NULL
    assert _mm(L, x=0, K=33) == q4.Q4_ERR_SHAPE


def test_matmul_workspace_bytes():
    q4, _ = _lib()
    # rows that fit one workgroup's LDS, the matrix-core paths and bad
    # shapes need none
    assert q4.q4_matmul_workspace_bytes(1, 34816, 5120) == 0
    # wide tiles (256 x 128, 256 a round): 544 tiles leave 32 for a third
    # round, cut into 8 K slices of 10 steps (256 x 128 fp32 blocks); whole
    # rounds, or a last round more than half full, take no workspace
    assert q4.q4_matmul_workspace_bytes(512, 34816, 5120) == 32 * 8 * 256 * 128 * 4
    assert q4.q4_matmul_workspace_bytes(512, 36864, 5120) == 64 * 4 * 256 * 128 * 4
    assert q4.q4_matmul_workspace_bytes(512, 32768, 5120) == 0
    assert q4.q4_matmul_workspace_bytes(512, 28672, 4096) == 0      # 448 tiles
    assert q4.q4_matmul_workspace_bytes(512, 34816, 5120 + 32) == 0  # K % 64 != 0
    # tiled path, more than 128 rows and K a multiple of 64 (tiles of 256
    # rows, one workgroup per CU): grids of 171 tiles or more are never cut
    # along K; fewer tiles take up to 256 / tiles slices of at least 8 K
    # steps, none empty
    assert q4.q4_matmul_workspace_bytes(512, 5120, 17408) == 3 * 512 * 5120 * 4   # 80 tiles
    assert q4.q4_matmul_workspace_bytes(1024, 5120, 17408) == 0                   # 160 tiles
    assert q4.q4_matmul_workspace_bytes(2048, 5120, 17408) == 64 * 4 * 256 * 128 * 4  # 320: tail
    # up to 128 rows (tiles of 128): 512 tiles or more are never cut; fewer
    # take up to 768 / tiles slices
    assert q4.q4_matmul_workspace_bytes(64, 5120, 17408) == 19 * 64 * 5120 * 4    # 40 tiles
    # slabs of 32 rows (64 workgroups of 32 weight rows): 4 K slices of 8 groups
    assert q4.q4_matmul_workspace_bytes(64, 1024, 4096) == 4 * 64 * 1024 * 4
    assert q4.q4_matmul_workspace_bytes(129, 130, 64) == 0                 # one K step
    assert q4.q4_matmul_workspace_bytes(129, 130, 64 * 16) == 2 * 129 * 130 * 4
    assert q4.q4_matmul_workspace_bytes(200, 128, 64 * 520) == 58 * 200 * 128 * 4
    assert q4.q4_matmul_workspace_bytes(300, 77, 96) == 0                  # K % 64 != 0
    # 3..16 rows with a workspace: one K slice per 32 blocks when that makes
    # 2 .. 64 slices (544 blocks: 17 slices; 160 blocks: 5; 128 blocks: 4)
    for M in (3, 4, 5, 16):
        assert q4.q4_matmul_workspace_bytes(M, 5120, 17408) == 17 * M * 5120 * 4
    assert q4.q4_matmul_workspace_bytes(4, 100, 5120) == 5 * 4 * 100 * 4
    assert q4.q4_matmul_workspace_bytes(4, 32768, 4096) == 4 * 4 * 32768 * 4
    assert q4.q4_matmul_workspace_bytes(4, 5120, 1024) == 0                  # one slice
    # longer rows, and 17..32 rows: grids of fewer than 1024 workgroups (32
    # weight rows by 16 or 32 activation rows) are cut along K, aiming at 1024
    # workgroups, into slices of a multiple of 8 four-block groups: 160
    # workgroups and 136 groups at 5120 x 17408 make 6 slices of 24 groups
    assert q4.q4_matmul_workspace_bytes(32, 5120, 17408) == 6 * 32 * 5120 * 4
    assert q4.q4_matmul_workspace_bytes(4, 5120, 512) == 0                   # 4 groups
    # 2080 blocks would make 65 slices of 32: the few-row kernel's plan (520
    # four-block groups, 160 workgroups: 7 slices of 80 groups)
    assert q4.q4_matmul_workspace_bytes(4, 5120, 66560) == 7 * 4 * 5120 * 4
    assert q4.q4_matmul_workspace_bytes(2, 5120, 48) == 0
    assert q4.q4_matmul_workspace_bytes(-1, 5120, 17408) == 0
    # long rows on the matrix-vector path: one fp32 partial sum per slice,
    # output and row; 544 blocks make 5 two-stage slices of 108-109 blocks
    for M, slices in ((1, 5), (2, 5)):
        assert q4.q4_matmul_workspace_bytes(M, 5120, 17408) == slices * M * 5120 * 4
    assert q4.q4_matmul_workspace_bytes(2, 100, 8192) == 0
    # 257 blocks (K = 8224): 3 slices of 86 blocks
    assert q4.q4_matmul_workspace_bytes(1, 7, 8224) == 3 * 1 * 7 * 4
    # 8065 blocks: two-stage slices would leave a last slice of 64, so
    # one-stage slices (127 of them)
    assert q4.q4_matmul_workspace_bytes(2, 5, 258080) == 127 * 2 * 5 * 4


def _mmx(L, ws_ptr, ws_bytes, x=A, M=2, N=32, K=17408):
    P = ctypes.c_void_p
    return L.q4_matmul_ex(P(x), P(A), P(A), P(A), 0, M, N, K, P(ws_ptr), ws_bytes, None)


def test_matmul_ex_workspace_errors():
    q4, L = _lib()
    need = q4.q4_matmul_workspace_bytes(2, 32, 17408)
    assert need > 0
    assert _mmx(L, A, need - 1) == q4.Q4_ERR_WORKSPACE
    assert _mmx(L, MIS, need) == q4.Q4_ERR_WORKSPACE
    # tensor NULL / alignment checks come first
    assert _mmx(L, A, 0, x=0) == q4.Q4_ERR_NULL
    assert _mmx(L, A, 0, x=MIS) == q4.Q4_ERR_ALIGN
    # zero-size is a no-op whatever the workspace
    assert _mmx(L, 0, 0, M=0) == q4.Q4_OK


@pytest.mark.skipif(_gpu_present(), reason="would launch on fake pointers")
def test_matmul_without_gpu_is_device_error():
    q4, L = _lib()
    assert _mm(L) == q4.Q4_ERR_DEVICE
    assert _mm(L, M=64, dt=1) == q4.Q4_ERR_DEVICE
    need = q4.q4_matmul_workspace_bytes(2, 32, 17408)
    assert _mmx(L, A, need) == q4.Q4_ERR_DEVICE
    assert _mmx(L, 0, 0) == q4.Q4_ERR_DEVICE


def _mx(L, x=A, wq=A, we=A, y=A, dt=0, M=1, N=64, K=256):
    P = ctypes.c_void_p
    L.q4_mx_matmul.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_int64, P]
    L.q4_mx_matmul.restype = ctypes.c_int32
    return L.q4_mx_matmul(P(x), P(wq), P(we), P(y), dt, M, N, K, P(0))


def test_mx_matmul_argument_errors():
    q4, L = _lib()
    assert _mx(L, dt=2) == q4.Q4_ERR_DTYPE
    assert _mx(L, K=0) == q4.Q4_ERR_SHAPE
    assert _mx(L, K=48) == q4.Q4_ERR_SHAPE
    assert _mx(L, N=-1) == q4.Q4_ERR_SHAPE
    assert _mx(L, M=-1) == q4.Q4_ERR_SHAPE
    assert _mx(L, M=65535 * 32 + 1) == q4.Q4_ERR_SHAPE   # past the slab limit
    assert _mx(L, dt=7, M=-1) == q4.Q4_ERR_DTYPE      # dtype before shape
    assert _mx(L, x=0, wq=0, we=0, y=0, M=0) == q4.Q4_OK
    assert _mx(L, x=0, wq=0, we=0, y=0, N=0) == q4.Q4_OK
    for kw in ("x", "wq", "we", "y"):
        assert _mx(L, **{kw: 0}) == q4.Q4_ERR_NULL, kw
        assert _mx(L, **{kw: MIS}) == q4.Q4_ERR_ALIGN, kw
    if not _gpu_present():
        assert _mx(L) == q4.Q4_ERR_DEVICE
        assert _mx(L, M=64, dt=1) == q4.Q4_ERR_DEVICE


def test_mx_matmul_ex_workspace():
    """Workspace sizes of the 4-bit float product: the tiled path's K slices
    only (grids of fewer than 512 tiles, K a multiple of 64); its checks as
    q4_matmul_ex's."""
    q4, L = _lib()
    assert q4.q4_mx_matmul_workspace_bytes(512, 5120, 17408) == 4 * 512 * 5120 * 4
    assert q4.q4_mx_matmul_workspace_bytes(200, 300, 2112) == 4 * 200 * 300 * 4
    assert q4.q4_mx_matmul_workspace_bytes(512, 34816, 5120) == 0      # 1088 tiles
    assert q4.q4_mx_matmul_workspace_bytes(200, 300, 2080) == 0        # K % 64 != 0
    assert q4.q4_mx_matmul_workspace_bytes(16, 5120, 17408) == 0       # few-row path
    assert q4.q4_mx_matmul_workspace_bytes(1, 5120, 17408) == 0        # matrix-vector
    assert q4.q4_mx_matmul_workspace_bytes(-1, 64, 256) == 0
    assert q4.q4_mx_matmul_workspace_bytes(200, 300, 48) == 0
    P = ctypes.c_void_p
    L.q4_mx_matmul_ex.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, P, ctypes.c_size_t, P]
    L.q4_mx_matmul_ex.restype = ctypes.c_int32

    def mxx(ws_ptr, ws_bytes, x=A, M=512, N=5120, K=17408, dt=0):
        return L.q4_mx_matmul_ex(P(x), P(A), P(A), P(A), dt, M, N, K, P(ws_ptr), ws_bytes, None)

    need = q4.q4_mx_matmul_workspace_bytes(512, 5120, 17408)
    assert mxx(A, need - 1) == q4.Q4_ERR_WORKSPACE
    assert mxx(MIS, need) == q4.Q4_ERR_WORKSPACE
    assert mxx(A, 0, x=0) == q4.Q4_ERR_NULL
    assert mxx(A, 0, x=MIS) == q4.Q4_ERR_ALIGN
    assert mxx(A, 0, dt=5) == q4.Q4_ERR_DTYPE
    assert mxx(A, 0, K=40) == q4.Q4_ERR_SHAPE
    assert mxx(0, 0, M=0) == q4.Q4_OK
    if not _gpu_present():
        assert mxx(A, need) == q4.Q4_ERR_DEVICE
        assert mxx(0, 0) == q4.Q4_ERR_DEVICE


def test_dequantize_argument_errors():
    q4, L = _lib()
    P = ctypes.c_void_p

    def dq(wq=A, ws=A, out=A, dt=0, N=4, K=64):
        return L.q4_dequantize(P(wq), P(ws), P(out), dt, N, K, None)

    assert dq(dt=3) == q4.Q4_ERR_DTYPE
    assert dq(K=31) == q4.Q4_ERR_SHAPE
    assert dq(N=-2) == q4.Q4_ERR_SHAPE
    assert dq(wq=0, ws=0, out=0, N=0) == q4.Q4_OK
    assert dq(wq=0) == q4.Q4_ERR_NULL
    assert dq(out=0) == q4.Q4_ERR_NULL
    assert dq(ws=MIS) == q4.Q4_ERR_ALIGN
    if not _gpu_present():
        assert dq() == q4.Q4_ERR_DEVICE


def test_moe_workspace_bytes():
    q4, _ = _lib()
    assert q4.q4_moe_workspace_bytes(-1, 8, 128, 1536) == 0
    assert q4.q4_moe_workspace_bytes(8, -1, 128, 1536) == 0
    assert q4.q4_moe_workspace_bytes(1 << 40, 1 << 20, 4, 4) == 0
    b = q4.q4_moe_workspace_bytes(8, 8, 128, 1536)
    # at least the per-(token, slot) fp32 partial rows
    assert b >= 8 * 8 * 1536 * 4
    assert b % 256 == 0
    assert q4.q4_moe_workspace_bytes(16, 8, 128, 1536) > b
    assert q4.q4_moe_workspace_bytes(8, 8, 256, 1536) > b


def test_moe_argument_errors():
    q4, L = _lib()
    P = ctypes.c_void_p
    T, topk, E, N, K = 8, 8, 128, 1536, 4096
    need = q4.q4_moe_workspace_bytes(T, topk, E, N)

    def moe(x=A, wq=A, ws=A, ids=A, g=A, y=A, T=T, topk=topk, E=E, N=N, K=K, w=A, wb=need):
        return L.q4_moe_matmul(P(x), P(wq), P(ws), P(ids), P(g), P(y), T, topk, E, N, K, P(w),
                               wb, None)

    assert moe(K=100) == q4.Q4_ERR_SHAPE
    assert moe(T=-1) == q4.Q4_ERR_SHAPE
    assert moe(E=-1) == q4.Q4_ERR_SHAPE
    assert moe(topk=-1) == q4.Q4_ERR_SHAPE
    assert moe(T=70000, topk=1, E=70000) == q4.Q4_ERR_SHAPE
    assert moe(x=0, wq=0, ws=0, ids=0, g=0, y=0, w=0, T=0) == q4.Q4_OK
    for kw in ("x", "wq", "ws", "ids", "g", "y"):
        assert moe(**{kw: 0}) == q4.Q4_ERR_NULL, kw
        assert moe(**{kw: MIS}) == q4.Q4_ERR_ALIGN, kw
    assert moe(w=0) == q4.Q4_ERR_WORKSPACE
    assert moe(w=MIS) == q4.Q4_ERR_WORKSPACE
    assert moe(wb=need - 1) == q4.Q4_ERR_WORKSPACE
    if not _gpu_present():
        assert moe() == q4.Q4_ERR_DEVICE


def test_moe_ffn_workspace_bytes():
    q4, _ = _lib()
    assert q4.q4_moe_ffn_workspace_bytes(-1, 8, 128, 4096, 1536) == 0
    assert q4.q4_moe_ffn_workspace_bytes(8, 8, 128, -1, 1536) == 0
    assert q4.q4_moe_ffn_workspace_bytes(1 << 40, 1 << 20, 4, 32, 32) == 0
    b = q4.q4_moe_ffn_workspace_bytes(8, 8, 128, 4096, 1536)
    # the down partial rows [P][H] and the SwiGLU outputs [P][F], fp32
    assert b >= 64 * (4096 + 1536) * 4
    assert b % 256 == 0
    assert b > q4.q4_moe_workspace_bytes(8, 8, 128, 4096)


def test_moe_ffn_argument_errors():
    q4, L = _lib()
    P = ctypes.c_void_p
    T, topk, E, H, F = 8, 8, 128, 4096, 1536
    need = q4.q4_moe_ffn_workspace_bytes(T, topk, E, H, F)

    def ffn(x=A, w13q=A, w13s=A, w2q=A, w2s=A, ids=A, g=A, y=A, T=T, topk=topk, E=E, H=H, F=F,
            w=A, wb=need):
        return L.q4_moe_ffn(P(x), P(w13q), P(w13s), P(w2q), P(w2s), P(ids), P(g), P(y), T, topk,
                            E, H, F, P(w), wb, None)

    for bad in (dict(H=100), dict(F=48), dict(H=0), dict(F=0), dict(H=8192 + 32),
                dict(F=8192 + 32), dict(T=-1), dict(E=-1), dict(topk=-1),
                dict(T=70000, topk=1, E=70000)):
        assert ffn(**bad) == q4.Q4_ERR_SHAPE, bad
    assert ffn(x=0, w13q=0, w13s=0, w2q=0, w2s=0, ids=0, g=0, y=0, w=0, T=0) == q4.Q4_OK
    for kw in ("x", "w13q", "w13s", "w2q", "w2s", "ids", "g", "y"):
        assert ffn(**{kw: 0}) == q4.Q4_ERR_NULL, kw
        assert ffn(**{kw: MIS}) == q4.Q4_ERR_ALIGN, kw
    assert ffn(w=0) == q4.Q4_ERR_WORKSPACE
    assert ffn(w=MIS) == q4.Q4_ERR_WORKSPACE
    assert ffn(wb=need - 1) == q4.Q4_ERR_WORKSPACE
    if not _gpu_present():
        assert ffn() == q4.Q4_ERR_DEVICE

    def ffn_ex(flags, **kw):
        a = dict(x=A, w13q=A, w13s=A, w2q=A, w2s=A, ids=A, g=A, y=A, T=T, topk=topk, E=E, H=H,
                 F=F, w=A, wb=need)
        a.update(kw)
        return L.q4_moe_ffn_ex(P(a["x"]), P(a["w13q"]), P(a["w13s"]), P(a["w2q"]), P(a["w2s"]),
                               P(a["ids"]), P(a["g"]), P(a["y"]), a["T"], a["topk"], a["E"],
                               a["H"], a["F"], flags, P(a["w"]), a["wb"], None)

    # unknown flag bits first, then the same checks as q4_moe_ffn
    for flags in (2, 4, 0x80000000, 0xFFFFFFFF):
        assert ffn_ex(flags) == q4.Q4_ERR_FLAGS, flags
        assert ffn_ex(flags, H=100) == q4.Q4_ERR_FLAGS, flags
    for flags in (0, q4.Q4_MOE_WEIGHTED_DOWN):
        assert ffn_ex(flags, H=100) == q4.Q4_ERR_SHAPE
        assert ffn_ex(flags, x=0) == q4.Q4_ERR_NULL
        assert ffn_ex(flags, y=MIS) == q4.Q4_ERR_ALIGN
        assert ffn_ex(flags, wb=need - 1) == q4.Q4_ERR_WORKSPACE
        assert ffn_ex(flags, T=0, x=0, y=0, w=0) == q4.Q4_OK
        if not _gpu_present():
            assert ffn_ex(flags) == q4.Q4_ERR_DEVICE


def test_binding_rejects_host_tensors():
    q4, _ = _lib()
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 64), dtype=torch.bfloat16)
    wq = torch.zeros((4, 32), dtype=torch.uint8)
    ws = torch.zeros((4, 2), dtype=torch.float16)
    with pytest.raises(ValueError):
        q4.q4_matmul(x, wq, ws)
    with pytest.raises(ValueError):
        q4.q4_dequantize(wq, ws)


def test_library_has_no_host_fallback():
    """The package is only the binding: no compute in Python, no oracle."""
    pkg = os.path.join(ROOT, "quantized_q4_block_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert "import oracle" not in src and "from oracle" not in src, name

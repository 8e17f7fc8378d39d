"""CPU oracle for the 4-bit block-quantised matmul -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library path (``quantized_q4_block_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``q4_oracle.c`` (plain C, double accumulation in
ascending k, one output at a time); this module builds it with gcc, loads it
with ctypes and converts numpy arrays.  See the C file's header for the
definition computed and the passages it follows.

Pinning (tests/test_oracle.py): exhaustive dequantisation of all 16 codes x
all 65,536 fp16 scale patterns against numpy's fp16 decoding and torch's
float32->bf16 rounding; a hand-written nibble-order fixture; closed forms on
constant and alternating inputs; exact rational brute force on 8x64 tiles;
agreement with a float64 library matmul of the dequantised weights; MoE
reductions to the dense case.  The routed FFN (tests/test_oracle_ffn.py):
closed forms with a saturated and a shut SwiGLU gate, an exact bound when the
up product cancels, exact zeros, the composition of pinned dense products
with numpy, and scalar brute force on a tiny case; planted mistakes in it are
caught (tests/test_oracle_mutants.py).  The 4-bit float block variant
(tests/test_oracle_mx.py): the E8M0 scales against torch's float8_e8m0fnu
decoding, the e2m1 element set by the properties that identify it, closed
forms, exact rational brute force and a float64 library matmul.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of the oracle (the mutation
# test compiles deliberately broken copies to show the pins catch them).
_LIB_PATH = os.environ.get("Q4_ORACLE_LIB", _DEFAULT_LIB)
_lib = None

BLOCK = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over output rows)."""
    if force or not os.path.exists(_DEFAULT_LIB):
        compile_to(_SRC, _DEFAULT_LIB)
    return _DEFAULT_LIB


def compile_to(src: str, out: str) -> None:
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_PATH == _DEFAULT_LIB and not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_fp16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_round_bits.argtypes = [ctypes.c_double]
    lib.oracle_bf16_round_bits.restype = ctypes.c_uint16
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_dequant_f32.argtypes = [P, P, I64, I64, P]
    lib.oracle_dequant_bf16.argtypes = [P, P, I64, I64, P]
    lib.oracle_matmul.argtypes = [P, P, P, I64, I64, I64, ctypes.c_int, P, P]
    lib.oracle_matmul_sampled.argtypes = [P, P, P, I64, I64, I64, ctypes.c_int,
                                          P, P, I64, P, P]
    lib.oracle_moe.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, P, P]
    lib.oracle_moe_ffn.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P]
    lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_rmsnorm.argtypes = [P, P, ctypes.c_double, I64, I64, P]
    lib.oracle_bf16_half_ulp.argtypes = [ctypes.c_double]
    lib.oracle_bf16_half_ulp.restype = ctypes.c_double
    lib.oracle_rmsnorm_matmul.argtypes = [P, P, ctypes.c_double, P, P, I64, I64, I64, P, P, P]
    lib.oracle_rmsnorm_matmul_sampled.argtypes = [P, P, ctypes.c_double, P, P, I64, I64, I64,
                                                  P, P, I64, P, P, P]
    lib.oracle_quantize.argtypes = [P, I64, I64, P, P]
    lib.oracle_sb_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.oracle_sb_matmul.argtypes = [P, P, P, P, I64, I64, I64, P, P]
    lib.oracle_mx_dequant.argtypes = [P, P, I64, I64, P]
    lib.oracle_mx_matmul.argtypes = [P, P, P, I64, I64, I64, P, P]
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def fp16_value(bits: int) -> float:
    return float(_load().oracle_fp16_value(int(bits)))


def bf16_value(bits: int) -> float:
    return float(_load().oracle_bf16_value(int(bits)))


def bf16_round_bits(v: float) -> int:
    return int(_load().oracle_bf16_round_bits(float(v)))


def _check_w(w_q, w_s):
    N, kh = w_q.shape[-2:]
    K = 2 * kh
    if K % BLOCK or w_s.shape[-1] != K // BLOCK or w_s.shape[-2] != N:
        raise ValueError("inconsistent w_q / w_s shapes")
    return N, K


def dequant_f32(w_q: np.ndarray, w_s: np.ndarray) -> np.ndarray:
    """float32 [N][K] dequantised weights (exact)."""
    N, K = _check_w(w_q, w_s)
    wq, ws = _c(w_q, np.uint8), _c(w_s, np.uint16)
    out = np.empty((N, K), dtype=np.float32)
    _load().oracle_dequant_f32(_ptr(wq), _ptr(ws), N, K, _ptr(out))
    return out


def dequant_bf16_bits(w_q: np.ndarray, w_s: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [N][K]: dequantised weights rounded nearest-even."""
    N, K = _check_w(w_q, w_s)
    wq, ws = _c(w_q, np.uint8), _c(w_s, np.uint16)
    out = np.empty((N, K), dtype=np.uint16)
    _load().oracle_dequant_bf16(_ptr(wq), _ptr(ws), N, K, _ptr(out))
    return out


def matmul(x: np.ndarray, w_q: np.ndarray, w_s: np.ndarray,
           bf16_weights: bool = False):
    """(y, t): double [M][N] result and sum_k |x*w| per output."""
    N, K = _check_w(w_q, w_s)
    x = _c(x, np.uint16)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x has the wrong K")
    wq, ws = _c(w_q, np.uint8), _c(w_s, np.uint16)
    y = np.empty((M, N), dtype=np.float64)
    t = np.empty((M, N), dtype=np.float64)
    _load().oracle_matmul(_ptr(x), _ptr(wq), _ptr(ws), M, N, K, int(bool(bf16_weights)),
                          _ptr(y), _ptr(t))
    return y, t


def matmul_sampled(x: np.ndarray, w_q: np.ndarray, w_s: np.ndarray,
                   ms: np.ndarray, ns: np.ndarray, bf16_weights: bool = False):
    """(y, t) for the outputs (ms[i], ns[i]) only; double [count]."""
    N, K = _check_w(w_q, w_s)
    x = _c(x, np.uint16)
    M = x.shape[0]
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D and equal length")
    if ms.size and (ms.min() < 0 or ms.max() >= M or ns.min() < 0 or ns.max() >= N):
        raise ValueError("sample index out of range")
    wq, ws = _c(w_q, np.uint8), _c(w_s, np.uint16)
    y = np.empty(ms.size, dtype=np.float64)
    t = np.empty(ms.size, dtype=np.float64)
    _load().oracle_matmul_sampled(_ptr(x), _ptr(wq), _ptr(ws), M, N, K,
                                  int(bool(bf16_weights)), _ptr(ms), _ptr(ns), ms.size,
                                  _ptr(y), _ptr(t))
    return y, t


def moe(x: np.ndarray, w_q: np.ndarray, w_s: np.ndarray, ids: np.ndarray,
        gates: np.ndarray):
    """(y, t): double [T][N] expert-routed weighted sum and its |.| scale."""
    E = w_q.shape[0]
    N, K = _check_w(w_q, w_s)
    x = _c(x, np.uint16)
    T = x.shape[0]
    ids = _c(ids, np.int32)
    gates = _c(gates, np.float32)
    topk = ids.shape[1]
    if ids.shape != (T, topk) or gates.shape != (T, topk):
        raise ValueError("ids / gates must be [T][topk]")
    wq, ws = _c(w_q, np.uint8), _c(w_s, np.uint16)
    y = np.empty((T, N), dtype=np.float64)
    t = np.empty((T, N), dtype=np.float64)
    _load().oracle_moe(_ptr(x), _ptr(wq), _ptr(ws), _ptr(ids), _ptr(gates),
                       T, topk, E, N, K, _ptr(y), _ptr(t))
    return y, t


def moe_ffn(x: np.ndarray, w13_q: np.ndarray, w13_s: np.ndarray, w2_q: np.ndarray,
            w2_s: np.ndarray, ids: np.ndarray, gates: np.ndarray):
    """(y, b): double [T][H] routed expert FFN -- gate/up (rows 2f / 2f+1 of
    w13), a = silu(gate) * up, down (w2), weighted sum over the slots -- and
    its tolerance scale b (see oracle_moe_ffn in q4_oracle.c)."""
    E, F2, Hh = w13_q.shape
    F = F2 // 2
    H = Hh * 2
    if F2 % 2 or w13_s.shape != (E, F2, H // 32) or w2_q.shape != (E, H, F // 2) \
            or w2_s.shape != (E, H, F // 32) or H % 32 or F % 32:
        raise ValueError("inconsistent FFN weight shapes")
    x = _c(x, np.uint16)
    T = x.shape[0]
    if x.shape != (T, H):
        raise ValueError("x must be [T][H]")
    ids = _c(ids, np.int32)
    gates = _c(gates, np.float32)
    topk = ids.shape[1]
    if ids.shape != (T, topk) or gates.shape != (T, topk):
        raise ValueError("ids / gates must be [T][topk]")
    a = [_c(w13_q, np.uint8), _c(w13_s, np.uint16), _c(w2_q, np.uint8), _c(w2_s, np.uint16)]
    y = np.empty((T, H), dtype=np.float64)
    b = np.empty((T, H), dtype=np.float64)
    _load().oracle_moe_ffn(_ptr(x), _ptr(a[0]), _ptr(a[1]), _ptr(a[2]), _ptr(a[3]),
                           _ptr(ids), _ptr(gates), T, topk, E, H, F, _ptr(y), _ptr(b))
    return y, b


# ---- 4-bit float blocks (e2m1 elements, E8M0 block scales) ----------------

def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code)))


def e8m0_value(bits: int) -> float:
    return float(_load().oracle_e8m0_value(int(bits)))


def _check_mx(w_q, w_e):
    N, kh = w_q.shape[-2:]
    K = 2 * kh
    if K % BLOCK or w_e.shape[-1] != K // BLOCK or w_e.shape[-2] != N:
        raise ValueError("inconsistent w_q / w_e shapes")
    return N, K


def mx_dequant(w_q: np.ndarray, w_e: np.ndarray) -> np.ndarray:
    """float64 [N][K]: e2m1(code) * 2^(E - 127), exact."""
    N, K = _check_mx(w_q, w_e)
    wq, we = _c(w_q, np.uint8), _c(w_e, np.uint8)
    out = np.empty((N, K), dtype=np.float64)
    _load().oracle_mx_dequant(_ptr(wq), _ptr(we), N, K, _ptr(out))
    return out


def mx_matmul(x: np.ndarray, w_q: np.ndarray, w_e: np.ndarray):
    """(y, t): double [M][N] product with 4-bit float block weights and
    sum_k |x*w| per output."""
    N, K = _check_mx(w_q, w_e)
    x = _c(x, np.uint16)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x has the wrong K")
    wq, we = _c(w_q, np.uint8), _c(w_e, np.uint8)
    y = np.empty((M, N), dtype=np.float64)
    t = np.empty((M, N), dtype=np.float64)
    _load().oracle_mx_matmul(_ptr(x), _ptr(wq), _ptr(we), M, N, K, _ptr(y), _ptr(t))
    return y, t


# ---- RMSNorm prologue ------------------------------------------------------

def bf16_half_ulp(v: float) -> float:
    """Half a bf16 unit in the last place of |v|."""
    return float(_load().oracle_bf16_half_ulp(float(v)))


def _check_norm(x, gamma):
    x = _c(x, np.uint16)
    gamma = _c(gamma, np.uint16)
    if x.ndim != 2 or gamma.shape != (x.shape[1],):
        raise ValueError("x must be [M][K] and gamma [K]")
    return x, gamma


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """double [M][K]: x[m,k] * gamma[k] / sqrt(mean_k x[m,k]^2 + eps)."""
    x, gamma = _check_norm(x, gamma)
    M, K = x.shape
    out = np.empty((M, K), dtype=np.float64)
    _load().oracle_rmsnorm(_ptr(x), _ptr(gamma), float(eps), M, K, _ptr(out))
    return out


def rmsnorm_matmul(x: np.ndarray, gamma: np.ndarray, eps: float, w_q: np.ndarray,
                   w_s: np.ndarray):
    """(y, t, u): double [M][N] product of the normalised activations with
    dequant(W), sum_k |x'*w|, and sum_k hulp(x'_k)*|w_k| (what rounding the
    normalised activations to bf16 can move y by)."""
    N, K = _check_w(w_q, w_s)
    x, gamma = _check_norm(x, gamma)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x has the wrong K")
    wq, ws = _c(w_q, np.uint8), _c(w_s, np.uint16)
    y, t, u = (np.empty((M, N), dtype=np.float64) for _ in range(3))
    _load().oracle_rmsnorm_matmul(_ptr(x), _ptr(gamma), float(eps), _ptr(wq), _ptr(ws), M, N, K,
                                  _ptr(y), _ptr(t), _ptr(u))
    return y, t, u


def rmsnorm_matmul_sampled(x: np.ndarray, gamma: np.ndarray, eps: float, w_q: np.ndarray,
                           w_s: np.ndarray, ms: np.ndarray, ns: np.ndarray):
    """(y, t, u) of rmsnorm_matmul for the outputs (ms[i], ns[i]) only."""
    N, K = _check_w(w_q, w_s)
    x, gamma = _check_norm(x, gamma)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x has the wrong K")
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D and equal length")
    if ms.size and (ms.min() < 0 or ms.max() >= M or ns.min() < 0 or ns.max() >= N):
        raise ValueError("sample index out of range")
    wq, ws = _c(w_q, np.uint8), _c(w_s, np.uint16)
    y, t, u = (np.empty(ms.size, dtype=np.float64) for _ in range(3))
    _load().oracle_rmsnorm_matmul_sampled(_ptr(x), _ptr(gamma), float(eps), _ptr(wq), _ptr(ws),
                                          M, N, K, _ptr(ms), _ptr(ns), ms.size, _ptr(y), _ptr(t),
                                          _ptr(u))
    return y, t, u


# ---- quantiser --------------------------------------------------------------

def quantize(w: np.ndarray):
    """(w_q, w_s): bf16 weights [N][K] (bit patterns) in this format -- per
    32-element block s = fp16(m / -8) with m the largest-magnitude element,
    codes clamp(rint(w / s) + 8, 0, 15) (fp32 quotient)."""
    w = _c(w, np.uint16)
    if w.ndim != 2 or w.shape[1] % BLOCK:
        raise ValueError("w must be [N][K] with K a multiple of 32")
    N, K = w.shape
    wq = np.zeros((N, K // 2), dtype=np.uint8)
    ws = np.zeros((N, K // BLOCK), dtype=np.uint16)
    _load().oracle_quantize(_ptr(w), N, K, _ptr(wq), _ptr(ws))
    return wq, ws


# ---- super-block (two-level) scales -----------------------------------------

def _check_sb(w_q, w_d, w_sc):
    N, kh = w_q.shape
    K = 2 * kh
    if K % 256 or w_d.shape != (N, K // 256) or w_sc.shape != (N, K // BLOCK):
        raise ValueError("inconsistent w_q / w_d / w_sc shapes (K a multiple of 256)")
    return N, K


def sb_dequant(w_q: np.ndarray, w_d: np.ndarray, w_sc: np.ndarray) -> np.ndarray:
    """float64 [N][K]: (code - 8) * d[k / 256] * sc[k / 32], exact."""
    N, K = _check_sb(w_q, w_d, w_sc)
    out = np.empty((N, K), dtype=np.float64)
    _load().oracle_sb_dequant(_ptr(_c(w_q, np.uint8)), _ptr(_c(w_d, np.uint16)),
                              _ptr(_c(w_sc, np.uint8)), N, K, _ptr(out))
    return out


def sb_matmul(x: np.ndarray, w_q: np.ndarray, w_d: np.ndarray, w_sc: np.ndarray):
    """(y, t): double [M][N] product with super-block-scaled weights and
    sum_k |x*w| per output."""
    N, K = _check_sb(w_q, w_d, w_sc)
    x = _c(x, np.uint16)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x has the wrong K")
    y = np.empty((M, N), dtype=np.float64)
    t = np.empty((M, N), dtype=np.float64)
    _load().oracle_sb_matmul(_ptr(x), _ptr(_c(w_q, np.uint8)), _ptr(_c(w_d, np.uint16)),
                             _ptr(_c(w_sc, np.uint8)), M, N, K, _ptr(y), _ptr(t))
    return y, t

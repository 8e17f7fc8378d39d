"""Python binding of libq4 -- weight-only 4-bit block-quantised matmul on
MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libq4.so`` (built in-tree from ``csrc/`` by ``_build.py``).
PyTorch supplies device memory and streams.  The functions carry the names
of the C ABI in ``include/q4.h``:

    q4_abi_version()                        -> int
    q4_status_str(status)                   -> str
    q4_matmul_path(M, N, K)                 -> Q4_PATH_GEMV | Q4_PATH_SMALL | Q4_PATH_MFMA
    q4_matmul_path_ex(M, N, K, with_workspace) -> the path q4_matmul_ex takes
    q4_matmul(x, w_q, w_s, out=None, out_dtype=torch.float32, stream=None) -> y
    q4_matmul_workspace_bytes(M, N, K)      -> int
    q4_matmul_ex(x, w_q, w_s, out=None, out_dtype=torch.float32, workspace="auto",
                 stream=None) -> y
    q4_dequantize(w_q, w_s, out=None, out_dtype=torch.float32, stream=None) -> w
    q4_quantize(w, w_q=None, w_s=None, stream=None) -> (w_q, w_s)
    q4_sb_matmul_workspace_bytes(M, N, K) -> int
    q4_sb_matmul(x, w_q, w_d, w_sc, out=None, out_dtype=torch.float32, workspace="auto",
                 stream=None) -> y
    q4_rmsnorm_matmul_workspace_bytes(M, N, K) -> int
    q4_rmsnorm_matmul(x, gamma, eps, w_q, w_s, out=None, out_dtype=torch.float32,
                      workspace="auto", stream=None) -> y
    q4_moe_workspace_bytes(T, topk, E, N)   -> int
    q4_moe_matmul(x, w_q, w_s, topk_ids, topk_w, out=None, workspace=None,
                  stream=None) -> y
    q4_moe_matmul_noalloc(x, w_q, w_s, topk_ids, topk_w, out=None, stream=None) -> y
    q4_moe_ffn_workspace_bytes(T, topk, E, H, F) -> int
    q4_moe_ffn(x, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_w, out=None,
               workspace=None, stream=None) -> y
    q4_mx_matmul(x, w_q, w_e, out=None, out_dtype=torch.float32, stream=None) -> y
    q4_mx_matmul_workspace_bytes(M, N, K)   -> int
    q4_mx_matmul_ex(x, w_q, w_e, out=None, out_dtype=torch.float32, workspace="auto",
                    stream=None) -> y

Tensor conventions (all CUDA/HIP device tensors, contiguous):
    x    torch.bfloat16 [M][K]       (or int16/uint16 holding bf16 bits)
    w_q  torch.uint8    [N][K/2]     (MoE: [E][N][K/2])
    w_s  torch.float16  [N][K/32]    (or int16/uint16 holding fp16 bits)
    w_e  torch.uint8    [N][K/32]    (4-bit float blocks: E8M0 scale bytes)
A non-zero status from the library raises ``Q4Error``.  If ``libq4.so`` is
missing the import fails: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4.so")

Q4_ABI_VERSION = 10
Q4_OK = 0
Q4_ERR_NULL = 1
Q4_ERR_SHAPE = 2
Q4_ERR_ALIGN = 3
Q4_ERR_DTYPE = 4
Q4_ERR_WORKSPACE = 5
Q4_ERR_DEVICE = 6
Q4_ERR_LAUNCH = 7
Q4_ERR_PENDING = 8
Q4_ERR_SCRATCH = 9
Q4_ERR_FLAGS = 10
Q4_MOE_WEIGHTED_DOWN = 1
Q4_MOE_NOALLOC_MAX_BYTES = 8 << 20
Q4_F32 = 0
Q4_BF16 = 1
Q4_PATH_GEMV = 0
Q4_PATH_MFMA = 1
Q4_PATH_SMALL = 2

__all__ = [
    "Q4Error", "lib", "q4_abi_version", "q4_status_str", "q4_matmul_path", "q4_matmul_path_ex",
    "q4_matmul",
    "q4_matmul_workspace_bytes", "q4_matmul_ex", "q4_dequantize", "q4_moe_workspace_bytes",
    "q4_rmsnorm_matmul_workspace_bytes", "q4_rmsnorm_matmul", "q4_quantize",
    "q4_sb_matmul_workspace_bytes", "q4_sb_matmul",
    "q4_moe_matmul", "q4_moe_matmul_noalloc", "q4_moe_ffn_workspace_bytes", "q4_moe_ffn", "q4_mx_matmul",
    "q4_mx_matmul_workspace_bytes", "q4_mx_matmul_ex", "q4_stream_read",
]


class Q4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {q4_status_str(status)} (status {status})")


def _open():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python quantized_q4_block_amd/_build.py`")
    # torch (when installed) first: it carries its own HIP runtime, and the
    # library must bind to that same runtime rather than load a second one
    # that does not see torch's devices and streams
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.q4_abi_version.argtypes = []
    L.q4_abi_version.restype = I32
    L.q4_status_str.argtypes = [I32]
    L.q4_status_str.restype = ctypes.c_char_p
    L.q4_matmul_path.argtypes = [I64, I64, I64]
    L.q4_matmul_path.restype = I32
    L.q4_matmul_path_ex.argtypes = [I64, I64, I64, I32]
    L.q4_matmul_path_ex.restype = I32
    L.q4_matmul.argtypes = [P, P, P, P, I32, I64, I64, I64, P]
    L.q4_matmul.restype = I32
    L.q4_matmul_workspace_bytes.argtypes = [I64, I64, I64]
    L.q4_matmul_workspace_bytes.restype = ctypes.c_size_t
    L.q4_matmul_ex.argtypes = [P, P, P, P, I32, I64, I64, I64, P, ctypes.c_size_t, P]
    L.q4_matmul_ex.restype = I32
    L.q4_rmsnorm_matmul_workspace_bytes.argtypes = [I64, I64, I64]
    L.q4_rmsnorm_matmul_workspace_bytes.restype = ctypes.c_size_t
    L.q4_rmsnorm_matmul.argtypes = [P, P, ctypes.c_float, P, P, P, I32, I64, I64, I64, P,
                                    ctypes.c_size_t, P]
    L.q4_rmsnorm_matmul.restype = I32
    L.q4_quantize.argtypes = [P, P, P, I64, I64, P]
    L.q4_sb_matmul_workspace_bytes.argtypes = [I64, I64, I64]
    L.q4_sb_matmul_workspace_bytes.restype = ctypes.c_size_t
    L.q4_sb_matmul.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P, ctypes.c_size_t, P]
    L.q4_sb_matmul.restype = I32
    L.q4_quantize.restype = I32
    L.q4_dequantize.argtypes = [P, P, P, I32, I64, I64, P]
    L.q4_dequantize.restype = I32
    L.q4_moe_workspace_bytes.argtypes = [I64, I64, I64, I64]
    L.q4_moe_workspace_bytes.restype = ctypes.c_size_t
    L.q4_moe_matmul.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, P, ctypes.c_size_t, P]
    L.q4_moe_matmul.restype = I32
    L.q4_moe_matmul_noalloc.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, P]
    L.q4_moe_matmul_noalloc.restype = I32
    L.q4_moe_ffn_workspace_bytes.argtypes = [I64, I64, I64, I64, I64]
    L.q4_moe_ffn_workspace_bytes.restype = ctypes.c_size_t
    L.q4_moe_ffn.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, ctypes.c_size_t,
                             P]
    L.q4_moe_ffn.restype = I32
    L.q4_moe_ffn_ex.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I64, I64,
                                ctypes.c_uint32, P, ctypes.c_size_t, P]
    L.q4_moe_ffn_ex.restype = I32
    L.q4_mx_matmul.argtypes = [P, P, P, P, I32, I64, I64, I64, P]
    L.q4_mx_matmul.restype = I32
    L.q4_mx_matmul_workspace_bytes.argtypes = [I64, I64, I64]
    L.q4_mx_matmul_workspace_bytes.restype = ctypes.c_size_t
    L.q4_mx_matmul_ex.argtypes = [P, P, P, P, I32, I64, I64, I64, P, ctypes.c_size_t, P]
    L.q4_mx_matmul_ex.restype = I32
    L.q4_stream_read_sink_words.argtypes = []
    L.q4_stream_read_sink_words.restype = I32
    L.q4_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    L.q4_stream_read.restype = I32
    if L.q4_abi_version() != Q4_ABI_VERSION:
        raise ImportError(f"libq4 ABI version {L.q4_abi_version()} != {Q4_ABI_VERSION}")
    return L


lib = _open()


def q4_abi_version() -> int:
    return int(lib.q4_abi_version())


def q4_status_str(status: int) -> str:
    return lib.q4_status_str(int(status)).decode()


def q4_matmul_path(M: int, N: int, K: int) -> int:
    return int(lib.q4_matmul_path(int(M), int(N), int(K)))


def q4_matmul_path_ex(M: int, N: int, K: int, with_workspace: bool) -> int:
    return int(lib.q4_matmul_path_ex(int(M), int(N), int(K), 1 if with_workspace else 0))


# ---------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _scratch(torch, nbytes, device, stream):
    """A temporary workspace for a call enqueued on `stream` (None: the current
    stream).  It is allocated with that stream current, so the caching
    allocator gives the block to another allocation only in that stream's
    order, after the call's kernels, even when the caller's current stream is
    another one."""
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_dev(t, name, dtypes, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out_code(dtype):
    torch = _torch()
    if dtype == torch.float32:
        return Q4_F32
    if dtype == torch.bfloat16:
        return Q4_BF16
    raise TypeError(f"unsupported output dtype {dtype}")


def _matmul_args(x, w_q, w_s, out, out_dtype):
    torch = _torch()
    _check_dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _check_dev(w_q, "w_q", (torch.uint8,), 2)
    _check_dev(w_s, "w_s", (torch.float16, torch.int16, torch.uint16), 2)
    M, K = x.shape
    N = w_q.shape[0]
    if w_q.shape[1] * 2 != K or tuple(w_s.shape) != (N, K // 32):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_q {tuple(w_q.shape)}, "
                         f"w_s {tuple(w_s.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=x.device)
    else:
        _check_dev(out, "out", (torch.float32, torch.bfloat16), 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    return M, N, K, out


def q4_matmul(x, w_q, w_s, out=None, out_dtype=None, stream=None):
    """y[M][N] = x[M][K] . dequant(W)[N][K]^T (fp32 or bf16 output)."""
    M, N, K, out = _matmul_args(x, w_q, w_s, out, out_dtype)
    st = lib.q4_matmul(_ptr(x), _ptr(w_q), _ptr(w_s), _ptr(out), _out_code(out.dtype),
                       M, N, K, _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_matmul")
    return out


def _mx_args(x, w_q, w_e, out, out_dtype):
    torch = _torch()
    _check_dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _check_dev(w_q, "w_q", (torch.uint8,), 2)
    _check_dev(w_e, "w_e", (torch.uint8,), 2)
    M, K = x.shape
    N = w_q.shape[0]
    if w_q.shape[1] * 2 != K or tuple(w_e.shape) != (N, K // 32):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_q {tuple(w_q.shape)}, "
                         f"w_e {tuple(w_e.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=x.device)
    else:
        _check_dev(out, "out", (torch.float32, torch.bfloat16), 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    return M, N, K, out


def q4_mx_matmul(x, w_q, w_e, out=None, out_dtype=None, stream=None):
    """y[M][N] = x[M][K] . W^T with 4-bit float block weights: w = e2m1(code)
    * 2^(E - 127), one E8M0 byte E per 32 k (fp32 or bf16 output)."""
    M, N, K, out = _mx_args(x, w_q, w_e, out, out_dtype)
    st = lib.q4_mx_matmul(_ptr(x), _ptr(w_q), _ptr(w_e), _ptr(out), _out_code(out.dtype),
                          M, N, K, _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_mx_matmul")
    return out


def q4_mx_matmul_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q4_mx_matmul_workspace_bytes(int(M), int(N), int(K)))


def q4_mx_matmul_ex(x, w_q, w_e, out=None, out_dtype=None, workspace="auto", stream=None):
    """q4_mx_matmul with a workspace: "auto" allocates what the call can use
    (a torch tensor), None passes none, a uint8 device tensor is passed as is."""
    torch = _torch()
    M, N, K, out = _mx_args(x, w_q, w_e, out, out_dtype)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device tensor')
        need = q4_mx_matmul_workspace_bytes(M, N, K)
        workspace = _scratch(torch, need, x.device, stream) if need else None
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.q4_mx_matmul_ex(_ptr(x), _ptr(w_q), _ptr(w_e), _ptr(out), _out_code(out.dtype),
                             M, N, K, _ptr(workspace), nbytes, _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_mx_matmul_ex")
    return out


def q4_matmul_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q4_matmul_workspace_bytes(int(M), int(N), int(K)))


def q4_matmul_ex(x, w_q, w_s, out=None, out_dtype=None, workspace="auto", stream=None):
    """q4_matmul with a workspace: "auto" allocates what the call can use (a
    torch tensor), None passes none, a uint8 device tensor is passed as is."""
    torch = _torch()
    M, N, K, out = _matmul_args(x, w_q, w_s, out, out_dtype)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device tensor')
        need = q4_matmul_workspace_bytes(M, N, K)
        workspace = _scratch(torch, need, x.device, stream) if need else None
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.q4_matmul_ex(_ptr(x), _ptr(w_q), _ptr(w_s), _ptr(out), _out_code(out.dtype),
                          M, N, K, _ptr(workspace), nbytes, _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_matmul_ex")
    return out


def q4_rmsnorm_matmul_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q4_rmsnorm_matmul_workspace_bytes(int(M), int(N), int(K)))


def q4_rmsnorm_matmul(x, gamma, eps, w_q, w_s, out=None, out_dtype=None, workspace="auto",
                      stream=None):
    """y = RMSNorm(x) . dequant(W)^T with RMSNorm(x)[m,k] = x[m,k] * gamma[k] /
    sqrt(mean_k x[m,k]^2 + eps).  workspace: "auto" allocates what the call
    can use (a torch tensor on the call's stream), None passes none, a uint8
    device tensor is passed as is."""
    torch = _torch()
    M, N, K, out = _matmul_args(x, w_q, w_s, out, out_dtype)
    _check_dev(gamma, "gamma", (torch.bfloat16, torch.int16, torch.uint16), 1)
    if gamma.shape[0] != K:
        raise ValueError("gamma must be [K]")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device tensor')
        need = q4_rmsnorm_matmul_workspace_bytes(M, N, K)
        workspace = _scratch(torch, need, x.device, stream) if need else None
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.q4_rmsnorm_matmul(_ptr(x), _ptr(gamma), float(eps), _ptr(w_q), _ptr(w_s), _ptr(out),
                               _out_code(out.dtype), M, N, K, _ptr(workspace), nbytes,
                               _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_rmsnorm_matmul")
    return out


def q4_quantize(w, w_q=None, w_s=None, stream=None):
    """bf16 weights [N][K] -> (codes uint8 [N][K/2], fp16 scales [N][K/32]):
    per 32-element block s = fp16(m / -8), m the largest-magnitude weight,
    codes clamp(rint(w / s) + 8, 0, 15)."""
    torch = _torch()
    _check_dev(w, "w", (torch.bfloat16, torch.int16, torch.uint16), 2)
    N, K = w.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if w_q is None:
        w_q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    else:
        _check_dev(w_q, "w_q", (torch.uint8,), 2)
        if tuple(w_q.shape) != (N, K // 2):
            raise ValueError("w_q has the wrong shape")
    if w_s is None:
        w_s = torch.empty((N, K // 32), dtype=torch.float16, device=w.device)
    else:
        _check_dev(w_s, "w_s", (torch.float16, torch.int16, torch.uint16), 2)
        if tuple(w_s.shape) != (N, K // 32):
            raise ValueError("w_s has the wrong shape")
    st = lib.q4_quantize(_ptr(w), _ptr(w_q), _ptr(w_s), N, K, _stream_handle(stream, w.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_quantize")
    return w_q, w_s


def q4_sb_matmul_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q4_sb_matmul_workspace_bytes(int(M), int(N), int(K)))


def q4_sb_matmul(x, w_q, w_d, w_sc, out=None, out_dtype=None, workspace="auto", stream=None):
    """y = x . W^T with super-block scales: w = (code - 8) * d[k/256] * sc[k/32];
    w_d fp16 [N][K/256], w_sc uint8 [N][K/32].  workspace: "auto" allocates
    one (a torch tensor on the call's stream), or a uint8 device tensor."""
    torch = _torch()
    _check_dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _check_dev(w_q, "w_q", (torch.uint8,), 2)
    _check_dev(w_d, "w_d", (torch.float16, torch.int16, torch.uint16), 2)
    _check_dev(w_sc, "w_sc", (torch.uint8,), 2)
    M, K = x.shape
    N = w_q.shape[0]
    if (w_q.shape[1] * 2 != K or K % 256 or tuple(w_d.shape) != (N, K // 256)
            or tuple(w_sc.shape) != (N, K // 32)):
        raise ValueError("shape mismatch (K a multiple of 256)")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=x.device)
    else:
        _check_dev(out, "out", (torch.float32, torch.bfloat16), 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto" or a device tensor')
        need = q4_sb_matmul_workspace_bytes(M, N, K)
        workspace = _scratch(torch, max(need, 1), x.device, stream)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.q4_sb_matmul(_ptr(x), _ptr(w_q), _ptr(w_d), _ptr(w_sc), _ptr(out), _out_code(out.dtype),
                          M, N, K, _ptr(workspace), nbytes, _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_sb_matmul")
    return out


def q4_dequantize(w_q, w_s, out=None, out_dtype=None, stream=None):
    """W[N][K] = (code - 8) * scale, fp32 (exact) or bf16 (nearest-even)."""
    torch = _torch()
    _check_dev(w_q, "w_q", (torch.uint8,), 2)
    _check_dev(w_s, "w_s", (torch.float16, torch.int16, torch.uint16), 2)
    N, KH = w_q.shape
    K = 2 * KH
    if tuple(w_s.shape) != (N, K // 32):
        raise ValueError("w_s has the wrong shape")
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype or torch.float32, device=w_q.device)
    else:
        _check_dev(out, "out", (torch.float32, torch.bfloat16), 2)
        if tuple(out.shape) != (N, K):
            raise ValueError("out has the wrong shape")
    st = lib.q4_dequantize(_ptr(w_q), _ptr(w_s), _ptr(out), _out_code(out.dtype), N, K,
                           _stream_handle(stream, w_q.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_dequantize")
    return out


def q4_moe_workspace_bytes(T: int, topk: int, E: int, N: int) -> int:
    return int(lib.q4_moe_workspace_bytes(int(T), int(topk), int(E), int(N)))


def _moe_args(x, w_q, w_s, topk_ids, topk_w, out):
    torch = _torch()
    _check_dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _check_dev(w_q, "w_q", (torch.uint8,), 3)
    _check_dev(w_s, "w_s", (torch.float16, torch.int16, torch.uint16), 3)
    _check_dev(topk_ids, "topk_ids", (torch.int32,), 2)
    _check_dev(topk_w, "topk_w", (torch.float32,), 2)
    T, K = x.shape
    E, N = w_q.shape[0], w_q.shape[1]
    topk = topk_ids.shape[1]
    if w_q.shape[2] * 2 != K or tuple(w_s.shape) != (E, N, K // 32):
        raise ValueError("weight shapes do not match x")
    if tuple(topk_ids.shape) != (T, topk) or tuple(topk_w.shape) != (T, topk):
        raise ValueError("topk_ids / topk_w must be [T][topk]")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=x.device)
    else:
        _check_dev(out, "out", (torch.float32,), 2)
        if tuple(out.shape) != (T, N):
            raise ValueError("out has the wrong shape")
    return T, topk, E, N, K, out


def q4_moe_matmul(x, w_q, w_s, topk_ids, topk_w, out=None, workspace=None, stream=None):
    """y[T][N] = sum_j topk_w[t][j] * x[t] . dequant(W[topk_ids[t][j]])^T (fp32).
    workspace None allocates one (a torch tensor on the stream the call runs on)."""
    torch = _torch()
    T, topk, E, N, K, out = _moe_args(x, w_q, w_s, topk_ids, topk_w, out)
    need = q4_moe_workspace_bytes(T, topk, E, N)
    if workspace is None:
        workspace = _scratch(torch, max(need, 1), x.device, stream)
    st = lib.q4_moe_matmul(_ptr(x), _ptr(w_q), _ptr(w_s), _ptr(topk_ids), _ptr(topk_w),
                           _ptr(out), T, topk, E, N, K, _ptr(workspace),
                           workspace.numel() * workspace.element_size(),
                           _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_moe_matmul")
    return out


def q4_moe_matmul_noalloc(x, w_q, w_s, topk_ids, topk_w, out=None, stream=None):
    """q4_moe_matmul with the library's built-in scratch as its workspace (no
    device allocation by the library; calls that overlap on one GPU race)."""
    T, topk, E, N, K, out = _moe_args(x, w_q, w_s, topk_ids, topk_w, out)
    st = lib.q4_moe_matmul_noalloc(_ptr(x), _ptr(w_q), _ptr(w_s), _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(out), T, topk, E, N, K, _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_moe_matmul_noalloc")
    return out


def q4_moe_ffn_workspace_bytes(T: int, topk: int, E: int, H: int, F: int) -> int:
    return int(lib.q4_moe_ffn_workspace_bytes(int(T), int(topk), int(E), int(H), int(F)))


def q4_moe_ffn(x, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_w, out=None, workspace=None,
               stream=None, weighted_down=False):
    """Routed expert FFN: y[T][H] = sum_j topk_w[t][j] *
    (silu(x W_gate^T) * (x W_up^T)) W_down^T of expert topk_ids[t][j]; gate and
    up rows interleaved in w13 (row 2f gate, 2f+1 up), down weights w2 (fp32 y).
    weighted_down: apply the route weights before the down product
    (Q4_MOE_WEIGHTED_DOWN)."""
    torch = _torch()
    _check_dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), 2)
    _check_dev(w13_q, "w13_q", (torch.uint8,), 3)
    _check_dev(w13_s, "w13_s", (torch.float16, torch.int16, torch.uint16), 3)
    _check_dev(w2_q, "w2_q", (torch.uint8,), 3)
    _check_dev(w2_s, "w2_s", (torch.float16, torch.int16, torch.uint16), 3)
    _check_dev(topk_ids, "topk_ids", (torch.int32,), 2)
    _check_dev(topk_w, "topk_w", (torch.float32,), 2)
    T, H = x.shape
    E, F2 = w13_q.shape[0], w13_q.shape[1]
    F = F2 // 2
    topk = topk_ids.shape[1]
    if (F2 % 2 or w13_q.shape[2] * 2 != H or tuple(w13_s.shape) != (E, F2, H // 32)
            or tuple(w2_q.shape) != (E, H, F // 2) or tuple(w2_s.shape) != (E, H, F // 32)):
        raise ValueError("weight shapes do not match x")
    if tuple(topk_ids.shape) != (T, topk) or tuple(topk_w.shape) != (T, topk):
        raise ValueError("topk_ids / topk_w must be [T][topk]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    else:
        _check_dev(out, "out", (torch.float32,), 2)
        if tuple(out.shape) != (T, H):
            raise ValueError("out has the wrong shape")
    need = q4_moe_ffn_workspace_bytes(T, topk, E, H, F)
    if workspace is None:
        workspace = _scratch(torch, max(need, 1), x.device, stream)
    flags = Q4_MOE_WEIGHTED_DOWN if weighted_down else 0
    st = lib.q4_moe_ffn_ex(_ptr(x), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s),
                           _ptr(topk_ids), _ptr(topk_w), _ptr(out), T, topk, E, H, F, flags,
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream_handle(stream, x.device))
    if st != Q4_OK:
        raise Q4Error(st, "q4_moe_ffn")
    return out


def q4_stream_read(src, sink=None, stream=None):
    """Read every byte of the device tensor src once (the benchmark's
    streaming ceiling; see include/q4.h).  Returns the uint32 sink tensor,
    whose XOR is the XOR of src's 32-bit words."""
    torch = _torch()
    if not isinstance(src, torch.Tensor) or src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = _scratch(torch, 4 * int(lib.q4_stream_read_sink_words()), src.device,
                        stream).view(torch.int32)
    st = lib.q4_stream_read(_ptr(src), nbytes, _ptr(sink), _stream_handle(stream, src.device))
    if st != 0:
        raise Q4Error(st, "q4_stream_read")
    return sink

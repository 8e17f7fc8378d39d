"""Helpers for the GPU parity tests: numpy <-> device tensors and calls
through the library's C ABI (via the thin binding)."""
from __future__ import annotations

import numpy as np
import torch

import quantized_q4_block_amd as q4

DEV = "cuda:0"


def dev(a: np.ndarray) -> torch.Tensor:
    """Device copy of a numpy array (16-bit patterns travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def bf16_bits_to_f64(t: torch.Tensor) -> np.ndarray:
    b = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def host(y: torch.Tensor) -> np.ndarray:
    if y.dtype == torch.bfloat16:
        return bf16_bits_to_f64(y)
    return y.cpu().numpy().astype(np.float64)


def matmul(x, w_q, w_s, out_dtype=torch.float32):
    y = q4.q4_matmul(dev(x), dev(w_q), dev(w_s), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(y)


def matmul_ex(x, w_q, w_s, out_dtype=torch.float32, workspace="auto"):
    y = q4.q4_matmul_ex(dev(x), dev(w_q), dev(w_s), out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return host(y)


def moe(x, w_q, w_s, ids, gates):
    y = q4.q4_moe_matmul(dev(x), dev(w_q), dev(w_s), dev(ids), dev(gates))
    torch.cuda.synchronize()
    return host(y)


def moe_ffn(c, ids=None, gates=None, workspace=None, weighted_down=False):
    y = q4.q4_moe_ffn(dev(c.x), dev(c.w13_q), dev(c.w13_s), dev(c.w2_q), dev(c.w2_s),
                      dev(c.ids if ids is None else ids), dev(c.gates if gates is None else gates),
                      workspace=workspace, weighted_down=weighted_down)
    torch.cuda.synchronize()
    return host(y)

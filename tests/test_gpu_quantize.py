"""Parity of q4_quantize (bf16 weights -> codes + fp16 scales) with the
oracle's quantiser, bit for bit, through the C ABI; and the quantised
weights through q4_matmul against the oracle."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import DEV, dev, host
from helpers import RTOL, assert_parity

pytestmark = pytest.mark.gpu

import quantized_q4_block_amd as q4  # noqa: E402


def bf16_bits(a):
    return synthetic.f32_to_bf16_bits(np.asarray(a, np.float32))


def _quant(w):
    wq, ws = q4.q4_quantize(dev(w))
    torch.cuda.synchronize()
    return wq.cpu().numpy(), ws.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("N,K,std", [(1, 32, 0.02), (77, 640, 0.02), (300, 4096, 1.0),
                                     (64, 2048, 3e-6), (1000, 5120, 0.02)])
def test_bit_exact(N, K, std):
    rng = np.random.default_rng(31000 + N)
    w = bf16_bits(rng.standard_normal((N, K)) * std)
    wq, ws = _quant(w)
    oq, os_ = oracle.quantize(w)
    assert np.array_equal(ws, os_)
    assert np.array_equal(wq, oq)


def test_special_blocks_bit_exact():
    K = 32 * 8
    rng = np.random.default_rng(32000)
    w = bf16_bits(rng.standard_normal((6, K)) * 0.01)
    w[0] = 0                                               # zeros: s = 0, codes 8
    w[1] = bf16_bits(np.full(K, 2.0 ** -130))              # s underflows to 0
    w[2] = bf16_bits(np.linspace(-1e6, 1e6, K))            # |s| clamped to 65504
    w[3, :32] = bf16_bits(np.full(32, 0.5))                # ties: the first max wins
    w[3, 5] = bf16_bits([-0.5])[0]
    w[4] = bf16_bits(rng.standard_normal(K) * 1e-6)        # fp16-subnormal scales
    w[5, 7] = 0x8001                                       # a bf16 subnormal weight
    wq, ws = _quant(w)
    oq, os_ = oracle.quantize(w)
    assert np.array_equal(ws, os_) and np.array_equal(wq, oq)


def test_full_gate_up_shape_and_matmul():
    """The decode gate+up weight shape (34816 x 5120), bit for bit; then those
    codes through q4_matmul against the oracle."""
    N, K = 34816, 5120
    rng = np.random.default_rng(33000)
    w = bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * 0.02)
    wq, ws = _quant(w)
    oq, os_ = oracle.quantize(w)
    assert np.array_equal(ws, os_) and np.array_equal(wq, oq)
    x = synthetic.dense_case(33001, 1, 1, K).x
    y = host(q4.q4_matmul(dev(x), dev(wq), dev(ws)))
    y_ref, t = oracle.matmul(x, oq, os_)
    assert_parity(y, y_ref, t, RTOL, what="quantised weights through q4_matmul")


def test_errors_leave_outputs_untouched():
    w = dev(np.zeros((4, 64), np.uint16))
    wq = torch.full((4, 32), 7, dtype=torch.uint8, device=DEV)
    ws = torch.full((4, 2), 7, dtype=torch.int16, device=DEV)
    P = ctypes.c_void_p
    assert q4.lib.q4_quantize(P(w.data_ptr()), P(wq.data_ptr()), P(ws.data_ptr()), 4, 48,
                              None) == q4.Q4_ERR_SHAPE
    assert q4.lib.q4_quantize(P(w.data_ptr() + 2), P(wq.data_ptr()), P(ws.data_ptr()), 4, 64,
                              None) == q4.Q4_ERR_ALIGN
    assert q4.lib.q4_quantize(P(0), P(wq.data_ptr()), P(ws.data_ptr()), 4, 64,
                              None) == q4.Q4_ERR_NULL
    torch.cuda.synchronize()
    assert torch.all(wq == 7) and torch.all(ws == 7)

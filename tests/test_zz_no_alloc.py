"""The no-allocation entry point q4_moe_matmul_noalloc, called through the C
ABI, against q4_moe_matmul with a caller-owned workspace (the same kernels:
results must agree bit for bit) and against the oracle (the parity bar), on
two calls in a row on one GPU, the second with a smaller input; plus the
size limit of the built-in scratch."""
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

P = ctypes.c_void_p


def _noalloc(m, fill=float("nan")):
    T, K = m.x.shape
    E, N = m.w_q.shape[0], m.w_q.shape[1]
    topk = m.ids.shape[1]
    x, wq, ws, ids, g = dev(m.x), dev(m.w_q), dev(m.w_s), dev(m.ids), dev(m.gates)
    y = torch.full((T, N), fill, dtype=torch.float32, device=DEV)
    st = q4.lib.q4_moe_matmul_noalloc(P(x.data_ptr()), P(wq.data_ptr()), P(ws.data_ptr()),
                                      P(ids.data_ptr()), P(g.data_ptr()), P(y.data_ptr()),
                                      T, topk, E, N, K, None)
    torch.cuda.synchronize()
    return st, host(y)


def _with_workspace(m):
    y = q4.q4_moe_matmul(dev(m.x), dev(m.w_q), dev(m.w_s), dev(m.ids), dev(m.gates))
    torch.cuda.synchronize()
    return host(y)


def test_noalloc_matches_the_workspace_call_twice():
    c = synthetic.CONFIGS["moe"]
    big = synthetic.moe_case(c["seed"], c["T"], c["topk"], c["E"], c["N"], c["K"])
    small = synthetic.moe_case(8100, 3, 2, 6, 100, 256)
    assert q4.q4_moe_workspace_bytes(3, 2, 6, 100) < q4.q4_moe_workspace_bytes(
        c["T"], c["topk"], c["E"], c["N"]) <= q4.Q4_MOE_NOALLOC_MAX_BYTES
    for what, m in (("moe workload", big), ("smaller second call", small)):
        st, y = _noalloc(m)
        assert st == q4.Q4_OK, q4.q4_status_str(st)
        y_ws = _with_workspace(m)
        assert np.array_equal(y.view(np.int64), y_ws.view(np.int64)), what
        y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
        assert_parity(y, y_ref, t, RTOL, what=what)


def test_noalloc_with_the_prep_buckets_then_without():
    # 80 pairs (more than the prep-free form takes): the prep kernel's tables
    # live in the built-in scratch; then a smaller call that skips the prep
    prep = synthetic.moe_case(8150, 40, 2, 64, 96, 1024)
    small = synthetic.moe_case(8160, 5, 2, 9, 70, 512)
    for what, m in (("prep buckets in the scratch", prep), ("smaller prep-free call", small)):
        st, y = _noalloc(m)
        assert st == q4.Q4_OK, q4.q4_status_str(st)
        y_ws = _with_workspace(m)
        assert np.array_equal(y.view(np.int64), y_ws.view(np.int64)), what
        y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
        assert_parity(y, y_ref, t, RTOL, what=what)


def test_noalloc_binding_and_repeated_ids():
    m = synthetic.moe_case(8200, 4, 4, 6, 64, 512)
    ids = m.ids.copy()
    ids[0, 1] = ids[0, 0]
    ids[1, 2] = 6            # out of range: contributes nothing
    y = q4.q4_moe_matmul_noalloc(dev(m.x), dev(m.w_q), dev(m.w_s), dev(ids), dev(m.gates))
    torch.cuda.synchronize()
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, ids, m.gates)
    assert_parity(host(y), y_ref, t, RTOL, what="noalloc binding")


def test_noalloc_rejects_more_than_its_scratch():
    # 64 pairs x N = 40000 fp32 partials: 10.24 MB, past the 8 MiB array
    T, topk, E, N, K = 16, 4, 8, 40000, 32
    assert q4.q4_moe_workspace_bytes(T, topk, E, N) > q4.Q4_MOE_NOALLOC_MAX_BYTES
    m = synthetic.moe_case(8300, T, topk, E, N, K)
    st, y = _noalloc(m, fill=3.0)
    assert st == q4.Q4_ERR_SCRATCH
    assert np.all(y == 3.0)

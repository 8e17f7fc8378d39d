"""GPU parity of the routed expert FFN (q4_moe_ffn, through the C ABI) with
the oracle.  Bar: |y - y_ref| <= 1e-3 * b per output, b the oracle's
first-order scale (each stage within 1e-3 of its own |.|-sum, carried
through the SwiGLU)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import moe_ffn
from helpers import RTOL

pytestmark = pytest.mark.gpu

import quantized_q4_block_amd as q4  # noqa: E402


def _check(y, y_ref, b, what):
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - y_ref)
    bad = err > RTOL * b
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs over the bar, worst "
                           f"{float(np.max(err / np.maximum(b, 1e-300))):.3e}")


# H and F of 1 to 4 stages (64 blocks each), whole and with leftovers of
# one block or more; experts shared by several tokens and single ones.  Few
# pairs per expert: the per-token product over the prep's buckets; (8, 8,
# 16, ...) and (9, 4, 5, ...): the grouped product.
@pytest.mark.parametrize("T,topk,E,H,F", [(1, 1, 1, 64, 32), (5, 3, 4, 96, 64),
                                          (8, 8, 16, 256, 160), (3, 2, 6, 1024 + 32, 2048 + 32),
                                          (4, 2, 3, 8192, 64), (2, 2, 3, 64, 8192),
                                          (40, 2, 64, 1024 + 32, 96),
                                          (6, 2, 8, 320, 37 * 32), (5, 3, 8, 224, 48 * 32),
                                          (9, 4, 5, 2048, 4096 + 96)])
def test_moe_ffn_parity_shapes(T, topk, E, H, F):
    c = synthetic.moe_ffn_case(8000 + T + H + F, T, topk, E, H, F)
    y = moe_ffn(c)
    y_ref, b = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.ids, c.gates)
    _check(y, y_ref, b, f"ffn T={T} topk={topk} E={E} H={H} F={F}")


def test_moe_ffn_config_full():
    cfg = synthetic.FFN_CONFIGS["moe_ffn"]
    c = synthetic.moe_ffn_case(cfg["seed"], cfg["T"], cfg["topk"], cfg["E"], cfg["H"], cfg["F"])
    y = moe_ffn(c)
    y_ref, b = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.ids, c.gates)
    _check(y, y_ref, b, "moe_ffn workload")


def test_moe_ffn_repeated_and_invalid_ids():
    c = synthetic.moe_ffn_case(8100, 3, 3, 4, 128, 64)
    ids = np.array([[1, 1, -1], [2, 9, 2], [0, 3, 1]], dtype=np.int32)
    y = moe_ffn(c, ids=ids)
    y_ref, b = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, ids, c.gates)
    _check(y, y_ref, b, "repeated / invalid ids")
    none = np.full_like(ids, -1)
    assert np.all(moe_ffn(c, ids=none) == 0)


def test_moe_ffn_deterministic_and_workspace_reuse():
    c = synthetic.moe_ffn_case(8200, 6, 4, 8, 512, 256)
    need = q4.q4_moe_ffn_workspace_bytes(6, 4, 8, 512, 256)
    work = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda:0")
    y1 = moe_ffn(c, workspace=work)
    y2 = moe_ffn(c, workspace=work)
    assert np.array_equal(y1, y2)
    d = synthetic.moe_ffn_case(8201, 2, 2, 3, 256, 128)
    y3 = moe_ffn(d, workspace=work)
    y_ref, b = oracle.moe_ffn(d.x, d.w13_q, d.w13_s, d.w2_q, d.w2_s, d.ids, d.gates)
    _check(y3, y_ref, b, "reused workspace")


# Route weights before the down product (Q4_MOE_WEIGHTED_DOWN): the same
# oracle result within the same bar, on the per-token path (few pairs per
# expert) and on the grouped path (many), with repeated and invalid ids.
@pytest.mark.parametrize("T,topk,E,H,F", [(5, 3, 4, 96, 64), (8, 8, 16, 256, 160),
                                          (40, 2, 64, 256, 160), (12, 2, 20, 96, 48 * 32),
                                          (40, 2, 3, 256, 160), (33, 8, 16, 1024 + 32, 512 + 96)])
def test_moe_ffn_weighted_down(T, topk, E, H, F):
    c = synthetic.moe_ffn_case(8300 + T + H + F, T, topk, E, H, F)
    ids = c.ids.copy()
    ids[0, -1] = E          # ignored
    if topk > 1:
        ids[1, 1] = ids[1, 0]   # summed
    y = moe_ffn(c, ids=ids, weighted_down=True)
    y_ref, b = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, ids, c.gates)
    _check(y, y_ref, b, f"weighted down T={T} topk={topk} E={E} H={H} F={F}")
    y2 = moe_ffn(c, ids=ids, weighted_down=True)
    assert np.array_equal(y, y2)

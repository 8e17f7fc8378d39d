"""GPU parity of the grouped routed-expert path (many pairs per expert:
q4_moe_matmul and q4_moe_ffn take matrix-core tiles over each expert's
bucket) with the oracle, through the C ABI.

The library takes the grouped path when the (token, slot) pairs are at least
4 per touched expert on average (P >= 4 min(P, E)); every shape here is
chosen on that side, and `grouped` re-checks it.  At the prefill-sized
workload (512 tokens, top-8 of 128 experts, experts of 1536 x 4096) the
oracle checks every token on a spread of output columns, and every column of
a set of tokens that together touch all experts."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_util import dev, moe, moe_ffn
from helpers import RTOL, assert_parity

pytestmark = pytest.mark.gpu

import quantized_q4_block_amd as q4  # noqa: E402


def grouped(T: int, topk: int, E: int) -> bool:
    P = T * topk
    return P > 0 and P >= 4 * min(P, E)


def _ffn_check(y, y_ref, b, what):
    assert np.all(np.isfinite(y)), what
    err = np.abs(y - y_ref)
    bad = err > RTOL * b
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs over the bar, worst "
                           f"{float(np.max(err / np.maximum(b, 1e-300))):.3e}")


# Slabs of 48 pairs, 128 weight rows per workgroup, 128-k steps: N below,
# at and past one column tile (ragged); K of one block, whole steps, and a
# last step of 1-3 blocks (K / 32 not a multiple of 4); experts with one slab,
# several, and a short last one.
@pytest.mark.parametrize("T,topk,E,N,K", [(16, 2, 2, 64, 32), (64, 4, 8, 96, 256),
                                          (40, 2, 2, 300, 416), (33, 8, 16, 520, 1024 + 32),
                                          (128, 8, 32, 256, 2048), (70, 3, 5, 257, 96 * 32 + 64)])
def test_grouped_parity_shapes(T, topk, E, N, K):
    assert grouped(T, topk, E)
    m = synthetic.moe_case(9000 + T + E + N, T, topk, E, N, K)
    y = moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    assert_parity(y, y_ref, t, RTOL, what=f"grouped T={T} topk={topk} E={E} N={N} K={K}")


def test_grouped_all_pairs_on_one_expert():
    # 100 pairs on expert 0 (slabs of 48, 48, 4), experts 1 and 2 idle
    T, E, N, K = 100, 3, 200, 512
    m = synthetic.moe_case(9100, T, 1, E, N, K)
    ids = np.zeros((T, 1), dtype=np.int32)
    y = moe(m.x, m.w_q, m.w_s, ids, m.gates)
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, ids, m.gates)
    assert_parity(y, y_ref, t, RTOL, what="all pairs on one expert")


def test_grouped_repeated_and_invalid_ids():
    T, topk, E, N, K = 48, 4, 6, 128, 256
    assert grouped(T, topk, E)
    m = synthetic.moe_case(9200, T, topk, E, N, K)
    ids = m.ids.copy()
    ids[0, 1] = ids[0, 0]      # repeated: summed
    ids[3, 2] = E              # out of range: ignored
    ids[5, 0] = -1
    ids[7, :] = -3             # a token with no valid slot: zero row
    y = moe(m.x, m.w_q, m.w_s, ids, m.gates)
    y_ref, t = oracle.moe(m.x, m.w_q, m.w_s, ids, m.gates)
    assert_parity(y, y_ref, t, RTOL, what="grouped repeated/invalid ids")
    assert np.all(y[7] == 0)


def test_grouped_deterministic_with_garbage_workspace():
    T, topk, E, N, K = 96, 8, 24, 384, 1024
    m = synthetic.moe_case(9300, T, topk, E, N, K)
    x, wq, ws, ids, g = dev(m.x), dev(m.w_q), dev(m.w_s), dev(m.ids), dev(m.gates)
    need = q4.q4_moe_workspace_bytes(T, topk, E, N)
    wsp = torch.full((need,), 0x5A, dtype=torch.uint8, device=x.device)
    outs = [q4.q4_moe_matmul(x, wq, ws, ids, g, workspace=wsp).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def _covering_tokens(ids: np.ndarray, E: int) -> np.ndarray:
    """Tokens, in increasing order, that together touch every expert any
    token touches (greedy: the first token that adds an untouched one)."""
    need = set(int(e) for e in np.unique(ids) if 0 <= e < E)
    out = []
    for t in range(ids.shape[0]):
        new = set(int(e) for e in ids[t]) & need
        if new:
            out.append(t)
            need -= new
        if not need:
            break
    return np.array(out, dtype=np.int64)


PREFILL_MOE = synthetic.MOE_PREFILL_CONFIGS["moe_prefill"]


def test_grouped_prefill_workload_sampled():
    c = PREFILL_MOE
    assert grouped(c["T"], c["topk"], c["E"])
    m = synthetic.moe_case(c["seed"], c["T"], c["topk"], c["E"], c["N"], c["K"])
    y = moe(m.x, m.w_q, m.w_s, m.ids, m.gates)
    assert y.shape == (c["T"], c["N"])
    # every token on 64 columns: 6 column tiles, every wavefront and 16-row
    # group position inside a tile
    i = np.arange(63)
    cols = np.unique(np.r_[i * 24 + (i * 5) % 24, c["N"] - 1])
    assert len(cols) == 64 and np.all(np.diff(cols // 256) >= 0)
    y_ref, t = oracle.moe(m.x, m.w_q[:, cols], m.w_s[:, cols], m.ids, m.gates)
    assert_parity(y[:, cols], y_ref, t, RTOL, what="prefill MoE, all tokens x 64 columns")
    # every column of tokens that together touch all experts
    toks = _covering_tokens(m.ids, c["E"])
    assert len(toks) <= 48
    y_ref, t = oracle.moe(m.x[toks], m.w_q, m.w_s, m.ids[toks], m.gates[toks])
    assert_parity(y[toks], y_ref, t, RTOL, what="prefill MoE, covering tokens x all columns")


# Routed FFN on the grouped path: gate/up with the SwiGLU into bf16 hi/lo,
# down over both, weighted sum.
@pytest.mark.parametrize("T,topk,E,H,F", [(16, 4, 4, 64, 32), (40, 2, 3, 256, 160),
                                          (33, 8, 16, 1024 + 32, 512 + 96),
                                          (64, 4, 8, 544, 2048)])
def test_grouped_ffn_parity_shapes(T, topk, E, H, F):
    assert grouped(T, topk, E)
    c = synthetic.moe_ffn_case(9400 + T + H + F, T, topk, E, H, F)
    y = moe_ffn(c)
    y_ref, b = oracle.moe_ffn(c.x, c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.ids, c.gates)
    _ffn_check(y, y_ref, b, f"grouped ffn T={T} topk={topk} E={E} H={H} F={F}")


def test_grouped_ffn_prefill_workload_sampled():
    cfg = synthetic.MOE_PREFILL_CONFIGS["moe_ffn_prefill"]
    T, topk, E, H, F = cfg["T"], cfg["topk"], cfg["E"], cfg["H"], cfg["F"]
    assert grouped(T, topk, E)
    c = synthetic.moe_ffn_case(cfg["seed"], T, topk, E, H, F)
    y = moe_ffn(c)
    toks = _covering_tokens(c.ids, E)
    y_ref, b = oracle.moe_ffn(c.x[toks], c.w13_q, c.w13_s, c.w2_q, c.w2_s, c.ids[toks],
                              c.gates[toks])
    _ffn_check(y[toks], y_ref, b, "prefill FFN, covering tokens x all columns")

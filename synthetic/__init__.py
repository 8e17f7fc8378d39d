"""Seeded synthetic inputs for the Q4 block matmul, shared by the oracle tests,
the GPU parity tests and the benchmark.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no nibble unpacking, no dequantisation, no dot products).
Every array is returned as raw bits in the storage layout the library's C ABI
takes:

* ``x``   -- bf16 activations, ``uint16[M][K]`` (bit patterns), drawn N(0, 1)
             in float32 and rounded to bf16 (round-to-nearest-even).
* ``w_q`` -- packed 4-bit codes, ``uint8[N][K/2]``.  Every byte is drawn
             uniformly from 0..255, which makes both nibbles of every byte
             independent and uniform over 0..15; which nibble maps to which
             k is the library's convention, not this module's concern.
* ``w_s`` -- one fp16 scale per 32-element block along K, ``uint16[N][K/32]``
             (bit patterns), |N(0, 1)| * 0.02 rounded to fp16.

Distributions follow the shapes and value laws of the workloads the specs'
T0 quantized-GEMM tier is sized for (spec "specialized model runtimes",
sections "Kernel and portability contract" and "Target package and
artifact": groupwise-int weight quantisation first); the MoE routing table
follows the expert-routed decode of the layer-package spec ("Policy
Resolution" MoE fixture paragraph): each token picks ``topk`` distinct
experts uniformly, with gates = softmax of N(0, 1) logits over the picked
experts.

Draw order inside one case: codes, scales, x, then (MoE) the router, token
by token.

RMSNorm prologue (``rms_case``): a dense case, then the norm's weights gamma,
bf16 ``uint16[K]`` drawn as 1 + 0.1 N(0, 1) (learned norm weights sit around
1); eps is 1e-6.

Super-block scales (``sb_case``): codes as above; one fp16 scale d per 256
elements of a row, |N(0, 1)| * 0.02 / 32 (so d * sc lands where the plain
format's block scales do); one multiplier byte sc per 32 elements, uniform
in 16..63 (the 6-bit range the K-quant profiles use for block scales).

4-bit float blocks (``mx_case``): the codes are drawn as above (e2m1
elements, the library's convention again); each block's E8M0 scale byte is
drawn uniformly from 118..122 (scales 2^-9 .. 2^-5, the range in which
blocks of weights of the magnitude above put their largest element near the
top of the e2m1 range, 6).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK = 32  # elements per quantisation block along K

__all__ = [
    "BLOCK", "DenseCase", "MoECase", "CONFIGS", "dense_case", "moe_case",
    "f32_to_bf16_bits", "config_case", "MXCase", "mx_case", "MX_CONFIGS",
    "RMSCase", "rms_case", "RMS_CONFIGS", "RMS_EPS", "SBCase", "sb_case", "SB_CONFIGS",
    "MOE_PREFILL_CONFIGS",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits.

    Used only to synthesise bf16 activations from float32 draws (finite
    values only).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


@dataclass
class DenseCase:
    x: np.ndarray    # uint16 [M][K]   bf16 bits
    w_q: np.ndarray  # uint8  [N][K/2] packed codes
    w_s: np.ndarray  # uint16 [N][K/32] fp16 bits

    @property
    def shape(self):
        M, K = self.x.shape
        return M, self.w_q.shape[0], K


@dataclass
class MoECase:
    x: np.ndarray      # uint16 [T][K]
    w_q: np.ndarray    # uint8  [E][N][K/2]
    w_s: np.ndarray    # uint16 [E][N][K/32]
    ids: np.ndarray    # int32  [T][topk]
    gates: np.ndarray  # float32 [T][topk]


@dataclass
class MoEFFNCase:
    x: np.ndarray      # uint16 [T][H]
    w13_q: np.ndarray  # uint8  [E][2F][H/2]  (row 2f gate, row 2f+1 up of unit f)
    w13_s: np.ndarray  # uint16 [E][2F][H/32]
    w2_q: np.ndarray   # uint8  [E][H][F/2]
    w2_s: np.ndarray   # uint16 [E][H][F/32]
    ids: np.ndarray    # int32  [T][topk]
    gates: np.ndarray  # float32 [T][topk]


def _weights(rng: np.random.Generator, lead: tuple, N: int, K: int, scale_std: float):
    w_q = rng.integers(0, 256, size=lead + (N, K // 2), dtype=np.uint8)
    s = np.abs(rng.standard_normal(lead + (N, K // BLOCK))) * scale_std
    w_s = s.astype(np.float16).view(np.uint16)
    return w_q, w_s


def dense_case(seed: int, M: int, N: int, K: int, scale_std: float = 0.02) -> DenseCase:
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    w_q, w_s = _weights(rng, (), N, K, scale_std)
    x = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    return DenseCase(x=x, w_q=w_q, w_s=w_s)


def moe_case(seed: int, T: int, topk: int, E: int, N: int, K: int,
             scale_std: float = 0.02) -> MoECase:
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    if topk > E:
        raise ValueError("topk distinct experts need topk <= E")
    rng = np.random.default_rng(seed)
    w_q, w_s = _weights(rng, (E,), N, K, scale_std)
    x = f32_to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    ids = np.empty((T, topk), dtype=np.int32)
    gates = np.empty((T, topk), dtype=np.float32)
    for t in range(T):
        ids[t] = rng.choice(E, size=topk, replace=False)
        logits = rng.standard_normal(topk)
        e = np.exp(logits - logits.max())
        gates[t] = (e / e.sum()).astype(np.float32)
    return MoECase(x=x, w_q=w_q, w_s=w_s, ids=ids, gates=gates)


def _route(rng: np.random.Generator, T: int, topk: int, E: int):
    ids = np.empty((T, topk), dtype=np.int32)
    gates = np.empty((T, topk), dtype=np.float32)
    for t in range(T):
        ids[t] = rng.choice(E, size=topk, replace=False)
        logits = rng.standard_normal(topk)
        e = np.exp(logits - logits.max())
        gates[t] = (e / e.sum()).astype(np.float32)
    return ids, gates


def moe_ffn_case(seed: int, T: int, topk: int, E: int, H: int, F: int,
                 scale_std: float = 0.02) -> MoEFFNCase:
    """Routed FFN inputs: gate/up weights [E][2F][H], down weights [E][H][F],
    bf16 tokens [T][H], router as in moe_case."""
    if H % BLOCK or F % BLOCK:
        raise ValueError("H and F must be multiples of 32")
    if topk > E:
        raise ValueError("topk distinct experts need topk <= E")
    rng = np.random.default_rng(seed)
    w13_q, w13_s = _weights(rng, (E,), 2 * F, H, scale_std)
    w2_q, w2_s = _weights(rng, (E,), H, F, scale_std)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    ids, gates = _route(rng, T, topk, E)
    return MoEFFNCase(x=x, w13_q=w13_q, w13_s=w13_s, w2_q=w2_q, w2_s=w2_s, ids=ids, gates=gates)


# The five workloads: shapes, seeds and output dtype.
CONFIGS = {
    "tiny_gemv":      dict(kind="dense", M=1, K=256, N=512, seed=0, out="f32"),
    "decode_gate_up": dict(kind="dense", M=1, K=5120, N=34816, seed=1, out="f32"),
    "batched_down":   dict(kind="dense", M=4, K=17408, N=5120, seed=2, out="f32"),
    "prefill":        dict(kind="dense", M=512, K=5120, N=34816, seed=3, out="bf16"),
    "moe":            dict(kind="moe", T=8, topk=8, E=128, K=4096, N=1536, seed=4, out="f32"),
}

# The routed FFN around the moe workload's expert shape: hidden H = 4096,
# expert width F = 1536 (gate/up [2F][H], down [H][F]).
FFN_CONFIGS = {
    "moe_ffn":        dict(kind="moe_ffn", T=8, topk=8, E=128, H=4096, F=1536, seed=5, out="f32"),
}

# The same expert shapes at prefill: 512 tokens, about 32 (token, slot)
# pairs per expert.
MOE_PREFILL_CONFIGS = {
    "moe_prefill":     dict(kind="moe", T=512, topk=8, E=128, K=4096, N=1536, seed=4, out="f32"),
    "moe_ffn_prefill": dict(kind="moe_ffn", T=512, topk=8, E=128, H=4096, F=1536, seed=5,
                            out="f32"),
}


def config_case(name: str):
    c = CONFIGS[name]
    if c["kind"] == "dense":
        return dense_case(c["seed"], c["M"], c["N"], c["K"])
    return moe_case(c["seed"], c["T"], c["topk"], c["E"], c["N"], c["K"])


@dataclass
class MXCase:
    x: np.ndarray    # uint16 [M][K]   bf16 bits
    w_q: np.ndarray  # uint8  [N][K/2] packed 4-bit elements
    w_e: np.ndarray  # uint8  [N][K/32] E8M0 scale bytes


def mx_case(seed: int, M: int, N: int, K: int, e_lo: int = 118, e_hi: int = 122) -> MXCase:
    """4-bit float block weights: uniform element bytes, E8M0 scale bytes
    uniform in e_lo..e_hi; bf16 x ~ N(0, 1)."""
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    w_q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    w_e = rng.integers(e_lo, e_hi + 1, size=(N, K // BLOCK), dtype=np.uint8)
    x = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    return MXCase(x=x, w_q=w_q, w_e=w_e)


# The decode gate+up and prefill shapes with 4-bit float block weights.
MX_CONFIGS = {
    "mx_decode_gate_up": dict(kind="mx", M=1, K=5120, N=34816, seed=6, out="f32"),
    "mx_prefill":        dict(kind="mx", M=512, K=5120, N=34816, seed=7, out="bf16"),
}


@dataclass
class RMSCase:
    x: np.ndarray      # uint16 [M][K]    bf16 bits (the un-normalised activations)
    gamma: np.ndarray  # uint16 [K]       bf16 bits
    w_q: np.ndarray    # uint8  [N][K/2]
    w_s: np.ndarray    # uint16 [N][K/32]
    eps: float


RMS_EPS = 1e-6


def rms_case(seed: int, M: int, N: int, K: int) -> RMSCase:
    """A dense case (codes, scales, x) followed by the norm weights."""
    d = dense_case(seed, M, N, K)
    rng = np.random.default_rng(seed + 1_000_003)
    gamma = f32_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(K, dtype=np.float32))
    return RMSCase(x=d.x, gamma=gamma, w_q=d.w_q, w_s=d.w_s, eps=RMS_EPS)


# The decode gate+up and prefill shapes behind an RMSNorm prologue.
RMS_CONFIGS = {
    "rms_decode_gate_up": dict(kind="rms", M=1, K=5120, N=34816, seed=8, out="f32"),
    "rms_prefill":        dict(kind="rms", M=512, K=5120, N=34816, seed=9, out="bf16"),
}


@dataclass
class SBCase:
    x: np.ndarray     # uint16 [M][K]     bf16 bits
    w_q: np.ndarray   # uint8  [N][K/2]   packed codes
    w_d: np.ndarray   # uint16 [N][K/256] fp16 bits (super-block scales)
    w_sc: np.ndarray  # uint8  [N][K/32]  block multipliers


def sb_case(seed: int, M: int, N: int, K: int) -> SBCase:
    if K % 256:
        raise ValueError("K must be a multiple of 256")
    rng = np.random.default_rng(seed)
    w_q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    w_d = (np.abs(rng.standard_normal((N, K // 256))) * (0.02 / 32)).astype(np.float16)
    w_sc = rng.integers(16, 64, size=(N, K // BLOCK), dtype=np.uint8)
    x = f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    return SBCase(x=x, w_q=w_q, w_d=w_d.view(np.uint16), w_sc=w_sc)


# The decode gate+up and prefill shapes with super-block scales.
SB_CONFIGS = {
    "sb_decode_gate_up": dict(kind="sb", M=1, K=5120, N=34816, seed=10, out="f32"),
    "sb_prefill":        dict(kind="sb", M=512, K=5120, N=34816, seed=11, out="bf16"),
}

"""Shared test helpers: golden-fixture parsing and the parity tolerance."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    """Parse a hand-worked fixture under tests/golden/."""
    rows, scales, wexp, xs, ys = [], [], [], [], []
    K = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tag, _, rest = line.partition(" ")
            if tag == "K":
                K = int(rest)
            elif tag == "row":
                b, s, w = (p.split() for p in rest.split("|"))
                rows.append([int(v, 16) for v in b])
                scales.append([int(v, 16) for v in s])
                wexp.append([float(v) for v in w])
            elif tag == "x":
                xs.append([int(v, 16) for v in rest.split()])
            elif tag == "y":
                m, n, v = rest.split()
                ys.append((int(m), int(n), float(v)))
    return dict(
        K=K,
        w_q=np.array(rows, dtype=np.uint8),
        w_s=np.array(scales, dtype=np.uint16),
        w=np.array(wexp, dtype=np.float64),
        x=np.array(xs, dtype=np.uint16),
        y=ys,
    )


# Parity bar for matmul outputs: |y - y_ref| <= RTOL * sum_k |x_k * w_k|.
RTOL = 1e-3


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place of |v| (rounding error of a bf16 store)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 0.0)


def within_tolerance(y, y_ref, t, rtol=RTOL, extra=0.0):
    """Boolean mask of outputs inside the parity bar (NaN never passes)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    return err <= rtol * t + extra


def assert_parity(y, y_ref, t, rtol=RTOL, extra=0.0, what=""):
    ok = within_tolerance(y, y_ref, t, rtol, extra)
    if not ok.all():
        y = np.asarray(y, dtype=np.float64)
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        ratio = np.abs(y - y_ref) / np.maximum(t, 1e-300)
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} outputs outside tolerance; first at {i}: "
            f"y={y[i]!r} ref={y_ref[i]!r} bound={t[i]!r}; worst |err|/bound={np.nanmax(ratio):.3e}")


def stratified_outputs(M: int, N: int):
    """One output (m, n) of every column n, with m = (7 n + n // 128) mod M.
    Within a 128-column tile m walks in steps of 7, so it passes through
    every 128-row tile; over the whole width it reaches every row (the tests
    that use it assert both coverages for their shapes)."""
    ns = np.arange(N, dtype=np.int64)
    ms = (7 * ns + ns // 128) % M
    return ms, ns

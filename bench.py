"""Benchmark: weight-only Q4 block matmul on one MI355X.

Headline workload: decode_gate_up -- the fused gate+up projection at decode,
M = 1, K = 5120, N = 34816 (int4 codes, 32-element blocks, fp16 scales,
bf16 activations, fp32 output).  A step is one q4_matmul_ex call (with the
workspace it asks for, none for this shape) over one
activation row, i.e. the whole decode hot path (activation staging, weight
and scale streaming, unpack + dequant, contraction, reduction, store).  The
weights rotate over byte-identical copies totalling more than 1 GB so that
neither the L2 caches nor the 256 MB Infinity Cache can serve them: every
step streams its 100.27 MB of codes and scales from HBM.

Printed: one JSON line with value = weight+scale GB/s (whole job), the
roofline of the dominant kernel (the decode GEMV) from HIP events over the
timed region, the CPU oracle's rate on the host (and on the batched decode,
prefill and MoE shapes), the shader clock under load, and the other
workloads (batched decode M = 4, prefill M = 512, 4-bit float block weights,
MoE and the routed expert FFN at 8 and 512 tokens, the RMSNorm prologue and
super-block scales at the decode and prefill shapes, the quantiser)
measured the same way as extra context.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "weight GB/s (% HBM peak) at decode M=1/4; TFLOP/s (% MFMA peak) at M=512"
ROTATE_BYTES = 1 << 30         # rotate weights over at least this much HBM


def weight_bytes(N, K):
    return N * K // 2 + N * (K // 32) * 2


# Sources the decode GEMV kernel is built from: a counter summary taken on
# other sources no longer describes the kernel.
GEMV_SOURCES = ("q4_api.hip", "q4_device.h", "q4_gemv.h", "q4_gemv.hip", "q4_launch.h")


def csrc_digest(names=GEMV_SOURCES):
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_q4_block_amd", "csrc")
    for name in sorted(names):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def all_sources_digest():
    d = os.path.join(ROOT, "quantized_q4_block_amd", "csrc")
    return csrc_digest(tuple(n for n in os.listdir(d) if n.endswith((".hip", ".h"))))


def under_profiler():
    """True inside a rocprofv3 run.  Its preloaded library reaches every
    child process too and, with counters, opens the GPU there before the
    child starts: children that are launchers (`env` in a script's #! line)
    would then replace a process that holds the GPU, so helpers that start
    other programs stay off."""
    return any(k.startswith("ROCPROF_") for k in os.environ)


def git_commit():
    """HEAD of the repository this script sits in, or None where the tree
    carries no git metadata (or under the profiler)."""
    import subprocess
    if under_profiler():
        return None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout.strip() or None if r.returncode == 0 else None


def library_build_info():
    """The commit the loaded library was built from and whether its sources
    differed from it (written by the build), or None."""
    try:
        with open(os.path.join(ROOT, "quantized_q4_block_amd", "build_info.json")) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def kernel_resources(mangled_prefix):
    """Register, LDS and occupancy figures the compiler reported for the
    kernel whose mangled name starts with mangled_prefix (written by the
    in-tree build next to the library), or None."""
    path = os.path.join(ROOT, "quantized_q4_block_amd", "kernel_resources.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    hits = [v for k, v in table.items() if k.startswith(mangled_prefix)]
    return hits[0] if len(hits) == 1 else None


def sample_sclk(torch, work, seconds=1.5):
    """The shader clock (MHz) rocm-smi reports while `work` keeps the GPU
    busy, or None if the tool is not there, prints no clock, or the run is
    under the profiler."""
    import re
    import subprocess
    import threading
    if under_profiler():
        return None
    box = {}

    def query():
        try:
            r = subprocess.run(["rocm-smi", "-d", "0", "--showclocks"], capture_output=True,
                               text=True, timeout=20)
            box["out"] = r.stdout
        except (OSError, subprocess.SubprocessError):
            box["out"] = ""
    stream = torch.cuda.current_stream()
    h = ctypes.c_void_p(stream.cuda_stream)
    th = threading.Thread(target=query)
    i, t0 = 0, time.perf_counter()
    for _ in range(200):            # busy before the query starts
        work.step(i, h)
        i += 1
    th.start()
    while th.is_alive() and time.perf_counter() - t0 < seconds + 20:
        for _ in range(100):
            work.step(i, h)
            i += 1
        torch.cuda.synchronize()
    th.join()
    for line in box.get("out", "").splitlines():
        if "sclk" in line.lower():
            m = re.search(r"\((\d+)\s*Mhz\)", line, flags=re.I)
            if m:
                return int(m.group(1))
    return None


def traffic_from_profile(kernel_tag, digest):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("csrc_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


class Dense:
    """Device copies of one dense workload, weights rotated over copies."""

    def __init__(self, torch, q4, name, copies=None):
        import synthetic
        c = synthetic.CONFIGS[name]
        self.name, self.M, self.N, self.K = name, c["M"], c["N"], c["K"]
        d = synthetic.dense_case(c["seed"], self.M, self.N, self.K)
        dev = "cuda:0"
        wb = weight_bytes(self.N, self.K)
        n = copies or max(2, -(-ROTATE_BYTES // wb) + 1)
        self.copies = n
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev)
        wq = torch.from_numpy(d.w_q).to(dev)
        ws = torch.from_numpy(d.w_s.view(np.int16)).to(dev)
        self.wq = [wq] + [wq.clone() for _ in range(n - 1)]
        self.ws = [ws] + [ws.clone() for _ in range(n - 1)]
        self.bf16 = c["out"] == "bf16"
        self.y = torch.empty((self.M, self.N), device=dev,
                             dtype=torch.bfloat16 if self.bf16 else torch.float32)
        # workspace for cutting long rows into slices, where the call can use one
        need = q4.q4_matmul_workspace_bytes(self.M, self.N, self.K)
        self.work = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        P = ctypes.c_void_p
        wptr = P(self.work.data_ptr()) if need else P(0)
        self.fn = q4.lib.q4_matmul_ex
        self.args = [(P(self.x.data_ptr()), P(self.wq[i].data_ptr()), P(self.ws[i].data_ptr()),
                      P(self.y.data_ptr()), q4.Q4_BF16 if self.bf16 else q4.Q4_F32,
                      self.M, self.N, self.K, wptr, need) for i in range(n)]
        self.wbytes = wb
        self.flops = 2 * self.M * self.N * self.K

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_matmul_ex failed with status {st}")


class StreamRead:
    """The streaming ceiling beside the decode kernel: q4_stream_read over the
    code bytes of the same rotating weight copies (16-byte non-temporal loads,
    the decode kernel's width and hint), one copy per step."""

    def __init__(self, torch, q4, dense):
        P = ctypes.c_void_p
        self.copies = dense.copies
        words = int(q4.lib.q4_stream_read_sink_words())
        self.sink = torch.empty(words, dtype=torch.int32, device="cuda:0")
        self.bytes = dense.wq[0].numel()
        self.fn = q4.lib.q4_stream_read
        self.args = [(P(w.data_ptr()), self.bytes, P(self.sink.data_ptr())) for w in dense.wq]

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_stream_read failed with status {st}")


class MxDense:
    """A dense shape with 4-bit float block weights (e2m1 elements, one E8M0
    byte per 32 k), weights rotated over copies."""

    def __init__(self, torch, q4, name="mx_decode_gate_up", copies=None):
        import synthetic
        c = synthetic.MX_CONFIGS[name]
        self.M, self.N, self.K = c["M"], c["N"], c["K"]
        d = synthetic.mx_case(c["seed"], self.M, self.N, self.K)
        dev = "cuda:0"
        wb = self.N * self.K // 2 + self.N * self.K // 32
        n = copies or max(2, -(-ROTATE_BYTES // wb) + 1)
        self.copies = n
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev)
        wq = torch.from_numpy(d.w_q).to(dev)
        we = torch.from_numpy(d.w_e).to(dev)
        self.wq = [wq] + [wq.clone() for _ in range(n - 1)]
        self.we = [we] + [we.clone() for _ in range(n - 1)]
        bf16 = c["out"] == "bf16"
        self.y = torch.empty((self.M, self.N), device=dev,
                             dtype=torch.bfloat16 if bf16 else torch.float32)
        P = ctypes.c_void_p
        self.fn = q4.lib.q4_mx_matmul
        self.args = [(P(self.x.data_ptr()), P(self.wq[i].data_ptr()), P(self.we[i].data_ptr()),
                      P(self.y.data_ptr()), q4.Q4_BF16 if bf16 else q4.Q4_F32,
                      self.M, self.N, self.K) for i in range(n)]
        self.wbytes = wb
        self.flops = 2.0 * self.M * self.N * self.K

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_mx_matmul failed with status {st}")


class MoE:
    def __init__(self, torch, q4, copies=None, config=None):
        import synthetic
        c = config or synthetic.CONFIGS["moe"]
        self.T, self.topk, self.E, self.N, self.K = c["T"], c["topk"], c["E"], c["N"], c["K"]
        m = synthetic.moe_case(c["seed"], self.T, self.topk, self.E, self.N, self.K)
        dev = "cuda:0"
        per_expert = weight_bytes(self.N, self.K)
        n = copies or max(2, -(-ROTATE_BYTES // (per_expert * self.E)) + 1)
        self.copies = n
        self.x = torch.from_numpy(m.x.view(np.int16)).to(dev)
        wq = torch.from_numpy(m.w_q).to(dev)
        ws = torch.from_numpy(m.w_s.view(np.int16)).to(dev)
        self.wq = [wq] + [wq.clone() for _ in range(n - 1)]
        self.ws = [ws] + [ws.clone() for _ in range(n - 1)]
        self.ids = torch.from_numpy(m.ids).to(dev)
        self.g = torch.from_numpy(m.gates).to(dev)
        self.y = torch.empty((self.T, self.N), device=dev, dtype=torch.float32)
        need = q4.q4_moe_workspace_bytes(self.T, self.topk, self.E, self.N)
        self.wsp = torch.empty(need, dtype=torch.uint8, device=dev)
        P = ctypes.c_void_p
        self.fn = q4.lib.q4_moe_matmul
        self.args = [(P(self.x.data_ptr()), P(self.wq[i].data_ptr()), P(self.ws[i].data_ptr()),
                      P(self.ids.data_ptr()), P(self.g.data_ptr()), P(self.y.data_ptr()),
                      self.T, self.topk, self.E, self.N, self.K, P(self.wsp.data_ptr()), need)
                     for i in range(n)]
        touched = len(np.unique(m.ids))
        self.touched = touched
        self.wbytes = touched * per_expert          # every touched expert read once
        self.flops = 2 * self.T * self.topk * self.N * self.K

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_moe_matmul failed with status {st}")


class MoeFfn:
    """The routed expert FFN around the moe workload's expert shape (hidden
    H = 4096, F = 1536 per expert, T = 8 tokens, top-8 of E = 128): gate/up
    product with the SwiGLU in its store, down product, weighted sum."""

    def __init__(self, torch, q4, copies=None, config=None):
        import synthetic
        c = config or synthetic.FFN_CONFIGS["moe_ffn"]
        self.T, self.topk, self.E, self.H, self.F = c["T"], c["topk"], c["E"], c["H"], c["F"]
        m = synthetic.moe_ffn_case(c["seed"], self.T, self.topk, self.E, self.H, self.F)
        dev = "cuda:0"
        per_expert = weight_bytes(2 * self.F, self.H) + weight_bytes(self.H, self.F)
        n = copies or max(2, -(-ROTATE_BYTES // (per_expert * self.E)) + 1)
        self.copies = n

        def put(a, i16=False):
            t = torch.from_numpy(a.view(np.int16) if i16 else a).to(dev)
            return [t] + [t.clone() for _ in range(n - 1)]
        self.x = torch.from_numpy(m.x.view(np.int16)).to(dev)
        self.w13q, self.w13s = put(m.w13_q), put(m.w13_s, True)
        self.w2q, self.w2s = put(m.w2_q), put(m.w2_s, True)
        self.ids = torch.from_numpy(m.ids).to(dev)
        self.g = torch.from_numpy(m.gates).to(dev)
        self.y = torch.empty((self.T, self.H), device=dev, dtype=torch.float32)
        need = q4.q4_moe_ffn_workspace_bytes(self.T, self.topk, self.E, self.H, self.F)
        self.wsp = torch.empty(need, dtype=torch.uint8, device=dev)
        P = ctypes.c_void_p
        self.fn = q4.lib.q4_moe_ffn
        self.args = [(P(self.x.data_ptr()), P(self.w13q[i].data_ptr()), P(self.w13s[i].data_ptr()),
                      P(self.w2q[i].data_ptr()), P(self.w2s[i].data_ptr()),
                      P(self.ids.data_ptr()), P(self.g.data_ptr()), P(self.y.data_ptr()),
                      self.T, self.topk, self.E, self.H, self.F, P(self.wsp.data_ptr()), need)
                     for i in range(n)]
        self.touched = len(np.unique(m.ids))
        self.wbytes = self.touched * per_expert     # every touched expert read once
        self.flops = 2 * self.T * self.topk * 3 * self.H * self.F

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_moe_ffn failed with status {st}")


class RmsDense:
    """q4_rmsnorm_matmul on a dense shape: RMSNorm(x) * gamma as the
    activations of the product (fused into the matrix-vector kernel at one
    row, a prologue kernel before the product otherwise)."""

    def __init__(self, torch, q4, name, copies=None):
        import synthetic
        c = synthetic.RMS_CONFIGS[name]
        self.M, self.N, self.K = c["M"], c["N"], c["K"]
        d = synthetic.rms_case(c["seed"], self.M, self.N, self.K)
        dev = "cuda:0"
        wb = weight_bytes(self.N, self.K)
        n = copies or max(2, -(-ROTATE_BYTES // wb) + 1)
        self.copies = n
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev)
        self.gamma = torch.from_numpy(d.gamma.view(np.int16)).to(dev)
        wq = torch.from_numpy(d.w_q).to(dev)
        ws = torch.from_numpy(d.w_s.view(np.int16)).to(dev)
        self.wq = [wq] + [wq.clone() for _ in range(n - 1)]
        self.ws = [ws] + [ws.clone() for _ in range(n - 1)]
        bf16 = c["out"] == "bf16"
        self.y = torch.empty((self.M, self.N), device=dev,
                             dtype=torch.bfloat16 if bf16 else torch.float32)
        need = q4.q4_rmsnorm_matmul_workspace_bytes(self.M, self.N, self.K)
        self.work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        P = ctypes.c_void_p
        self.fn = q4.lib.q4_rmsnorm_matmul
        self.args = [(P(self.x.data_ptr()), P(self.gamma.data_ptr()), ctypes.c_float(d.eps),
                      P(self.wq[i].data_ptr()), P(self.ws[i].data_ptr()), P(self.y.data_ptr()),
                      q4.Q4_BF16 if bf16 else q4.Q4_F32, self.M, self.N, self.K,
                      P(self.work.data_ptr()), need) for i in range(n)]
        self.wbytes = wb
        self.flops = 2 * self.M * self.N * self.K

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_rmsnorm_matmul failed with status {st}")


class SbDense:
    """q4_sb_matmul on a dense shape: codes with two-level (super-block)
    scales; the decode shape reads them as stored, the prefill shape expands
    them to fp32 block scales in the workspace first."""

    def __init__(self, torch, q4, name, copies=None):
        import synthetic
        c = synthetic.SB_CONFIGS[name]
        self.M, self.N, self.K = c["M"], c["N"], c["K"]
        d = synthetic.sb_case(c["seed"], self.M, self.N, self.K)
        dev = "cuda:0"
        wb = self.N * self.K // 2 + self.N * (self.K // 256) * 2 + self.N * (self.K // 32)
        n = copies or max(2, -(-ROTATE_BYTES // wb) + 1)
        self.copies = n
        self.x = torch.from_numpy(d.x.view(np.int16)).to(dev)

        def put(a, i16=False):
            t = torch.from_numpy(a.view(np.int16) if i16 else a).to(dev)
            return [t] + [t.clone() for _ in range(n - 1)]
        self.wq, self.wd, self.wsc = put(d.w_q), put(d.w_d.view(np.uint16), True), put(d.w_sc)
        bf16 = c["out"] == "bf16"
        self.y = torch.empty((self.M, self.N), device=dev,
                             dtype=torch.bfloat16 if bf16 else torch.float32)
        need = q4.q4_sb_matmul_workspace_bytes(self.M, self.N, self.K)
        self.work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        P = ctypes.c_void_p
        self.fn = q4.lib.q4_sb_matmul
        self.args = [(P(self.x.data_ptr()), P(self.wq[i].data_ptr()), P(self.wd[i].data_ptr()),
                      P(self.wsc[i].data_ptr()), P(self.y.data_ptr()),
                      q4.Q4_BF16 if bf16 else q4.Q4_F32, self.M, self.N, self.K,
                      P(self.work.data_ptr()), need) for i in range(n)]
        self.wbytes = wb
        self.flops = 2 * self.M * self.N * self.K

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_sb_matmul failed with status {st}")


class Quantize:
    """q4_quantize of the decode projection's weights: bf16 [N][K] in, codes
    and fp16 block scales out."""

    def __init__(self, torch, q4, N=34816, K=5120, copies=None):
        dev = "cuda:0"
        self.N, self.K = N, K
        g = torch.Generator(device="cpu").manual_seed(12)
        w = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16)
        rd = N * K * 2
        n = copies or max(2, -(-ROTATE_BYTES // rd) + 1)
        self.copies = n
        wdev = w.to(dev)
        self.w = [wdev] + [wdev.clone() for _ in range(n - 1)]
        self.wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        self.ws = torch.empty((N, K // 32), dtype=torch.float16, device=dev)
        P = ctypes.c_void_p
        self.fn = q4.lib.q4_quantize
        self.args = [(P(self.w[i].data_ptr()), P(self.wq.data_ptr()), P(self.ws.data_ptr()),
                      N, K) for i in range(n)]
        self.bytes = rd + N * K // 2 + N * (K // 32) * 2   # bf16 read, codes and scales written

    def step(self, i, stream):
        st = self.fn(*self.args[i % self.copies], stream)
        if st:
            raise RuntimeError(f"q4_quantize failed with status {st}")


def calibration_copy(torch, mib, reps=3):
    """A plain elementwise copy of known size (y = -x over `mib` MiB of fp32:
    `mib` MiB read, `mib` MiB written per launch), run so that a counter pass
    can scale the HBM byte counters against a kernel whose traffic is known."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def _counter_means(run_dir, counter):
    """Mean per-dispatch value of `counter` by kernel name, from the
    counter_collection.csv files a rocprofv3 --pmc run wrote under run_dir."""
    import csv
    sums, counts = {}, {}
    for dirpath, _, files in os.walk(run_dir):
        for fn in files:
            if not fn.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(dirpath, fn), newline="") as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    k = row["Kernel_Name"]
                    sums[k] = sums.get(k, 0.0) + float(row["Counter_Value"])
                    counts[k] = counts.get(k, 0) + 1
    return {k: (sums[k] / counts[k], counts[k]) for k in sums}


def summarize_pmc(fetch_dir, write_dir, copy_mib, kernel_tag, kernel_match, algorithmic, out):
    """HBM bytes per launch of the kernel whose name contains kernel_match:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the ratio of
    the calibration copy's known bytes to what the same counter read for it."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def pick(table, sub):
        hits = [(k, v) for k, v in table.items() if sub in k or sub in "q4::" + k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {sub!r}, found {[k for k, _ in hits]}")
        return hits[0]

    copy_bytes = copy_mib * (1 << 20)
    (ck, (cf, _)), (_, (cw, _)) = pick(fetch, "neg"), pick(write, "neg")
    (gk, (gf, nf)), (_, (gw, nw)) = pick(fetch, kernel_match), pick(write, kernel_match)
    f_read = copy_bytes / (cf * 1024.0)
    f_write = copy_bytes / (cw * 1024.0)
    traffic = gf * 1024.0 * f_read + gw * 1024.0 * f_write
    rec = {"kernel": gk, "dispatches": {"FETCH_SIZE": nf, "WRITE_SIZE": nw},
           "FETCH_SIZE_KiB": gf, "WRITE_SIZE_KiB": gw,
           "calibration": {"kernel": ck, "bytes_each_way": copy_bytes,
                           "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw,
                           "read_factor": f_read, "write_factor": f_write},
           "hbm_bytes_per_launch": round(traffic),
           "algorithmic_bytes_per_launch": algorithmic,
           "traffic_over_algorithmic": traffic / algorithmic,
           "csrc_digest": csrc_digest()}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


# The decode workload's kernel: the roofline object's kernel and the one the
# counter summary picks out of a --pmc run.
DECODE_KERNEL = "q4::gemv_lds_kernel<1, 2, 1, false, unsigned short>"


# After a few seconds without GPU work (input generation on the host) the
# chip needs several milliseconds of load before its clocks are back up: the
# MoE call measured 51 us in its first 200 launches and 44 us from then on.
CLOCK_WARM_MS = 60.0


def time_steps(torch, work, steps, warmup, warm_ms=0.0, blocks=0, spread=None):
    """Host-timed steps (synchronised on both sides) and HIP-event time over
    the same region on the launch stream.  `warmup` untimed steps first, and
    before them, if warm_ms > 0, untimed steps until the GPU has run this
    work for warm_ms.  With blocks > 1, events also split the timed steps
    into that many equal blocks, and `spread` (a list) receives each block's
    event time per step (ms)."""
    stream = torch.cuda.current_stream()
    h = ctypes.c_void_p(stream.cuda_stream)
    done, i = 0.0, 0
    while done < warm_ms:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for _ in range(20):
            work.step(i, h)
            i += 1
        w1.record(stream)
        torch.cuda.synchronize()
        done += w0.elapsed_time(w1)
    for j in range(warmup):
        work.step(i + j, h)
    warmup += i
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    per = steps // blocks if blocks > 1 else 0
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(blocks - 1)] if per else []
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        if per and i and i % per == 0 and i // per <= len(marks):
            marks[i // per - 1].record(stream)
        work.step(warmup + i, h)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if per and spread is not None:
        edges = [e0] + marks
        for b in range(len(edges)):
            end = edges[b + 1] if b + 1 < len(edges) else e1
            n = per if b + 1 < len(edges) else steps - per * len(marks)
            spread.append(edges[b].elapsed_time(end) / n)
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def cpu_baseline(min_seconds=12.0, max_reps=100000):
    """The CPU oracle on decode_gate_up, repeated until >= min_seconds."""
    import oracle
    import synthetic
    c = synthetic.CONFIGS["decode_gate_up"]
    d = synthetic.dense_case(c["seed"], c["M"], c["N"], c["K"])
    oracle.matmul(d.x[:, :], d.w_q[:64], d.w_s[:64])      # load + warm
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.matmul(d.x, d.w_q, d.w_s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    gbs = reps * weight_bytes(c["N"], c["K"]) / el / 1e9
    cores = oracle.max_threads()
    # the same oracle on one thread, over the first 2048 weight rows
    rows = 2048
    oracle.set_threads(1)
    try:
        reps1, t0 = 0, time.perf_counter()
        while True:
            oracle.matmul(d.x, d.w_q[:rows], d.w_s[:rows])
            reps1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= min_seconds / 4 or reps1 >= max_reps:
                break
    finally:
        oracle.set_threads(cores)
    gbs1 = reps1 * weight_bytes(rows, c["K"]) / el1 / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"full decode_gate_up (M=1, K=5120, N=34816) x {reps} reps, "
                      f"{el:.1f} s, double accumulation",
            "host_cpu": host_cpu_model(),
            "single_thread": {"value": round(gbs1, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"decode_gate_up rows 0..{rows - 1} x {reps1} reps, "
                                        f"{el1:.1f} s"}}


def cpu_baselines_other(runs=3):
    """The CPU oracle on the other headline shapes, each the median of `runs`
    timed calls, in the metric the GPU line reports for it: batched_down
    (whole call) and moe (whole call) as weight GB/s, prefill on a sample of
    256 weight rows (all 512 activation rows, all of K) as TFLOP/s."""
    import oracle
    import synthetic

    def med(f):
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), ts
    cores = oracle.max_threads()
    out = {}
    c = synthetic.CONFIGS["batched_down"]
    d = synthetic.dense_case(c["seed"], c["M"], c["N"], c["K"])
    t, ts = med(lambda: oracle.matmul(d.x, d.w_q, d.w_s))
    out["batched_down"] = {"value": round(weight_bytes(c["N"], c["K"]) / t / 1e9, 4),
                           "unit": "GB/s", "cores": cores, "kind": "oracle",
                           "sample": f"whole call M={c['M']} N={c['N']} K={c['K']}, median of "
                                     f"{runs} ({', '.join(f'{x:.2f}' for x in ts)} s)"}
    c = synthetic.CONFIGS["prefill"]
    rows = 256
    d = synthetic.dense_case(c["seed"], c["M"], rows, c["K"])
    t, ts = med(lambda: oracle.matmul(d.x, d.w_q, d.w_s))
    out["prefill"] = {"value": round(2.0 * c["M"] * rows * c["K"] / t / 1e12, 6),
                      "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                      "sample": f"M={c['M']}, {rows} of the {c['N']} weight rows, K={c['K']}, "
                                f"median of {runs} ({', '.join(f'{x:.2f}' for x in ts)} s)"}
    c = synthetic.CONFIGS["moe"]
    m = synthetic.moe_case(c["seed"], c["T"], c["topk"], c["E"], c["N"], c["K"])
    t, ts = med(lambda: oracle.moe(m.x, m.w_q, m.w_s, m.ids, m.gates))
    touched = len(np.unique(m.ids))
    out["moe"] = {"value": round(touched * weight_bytes(c["N"], c["K"]) / t / 1e9, 4),
                  "unit": "touched weight GB/s", "cores": cores, "kind": "oracle",
                  "sample": f"whole call T={c['T']} top-{c['topk']} of {c['E']}, "
                            f"N={c['N']} K={c['K']}, median of {runs} "
                            f"({', '.join(f'{x:.2f}' for x in ts)} s)"}
    return out


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def summarize_trace(run_dir):
    """Per-kernel dispatch count, mean, p10, median, p90, min and max duration
    (us) from the kernel_trace.csv files a rocprofv3 --kernel-trace run wrote
    under run_dir."""
    import csv
    durs = {}
    for dirpath, _, files in os.walk(run_dir):
        for fn in files:
            if not fn.endswith("kernel_trace.csv"):
                continue
            with open(os.path.join(dirpath, fn), newline="") as f:
                for row in csv.DictReader(f):
                    name = row["Kernel_Name"].replace("void ", "")
                    name = name.replace("(anonymous namespace)::", "").split("(")[0]
                    d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                    durs.setdefault(name, []).append(d)
    out = {}
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        a = np.asarray(v)
        out[name] = {"calls": int(a.size), "mean_us": round(float(a.mean()), 2),
                     "p10_us": round(float(np.percentile(a, 10)), 2),
                     "median_us": round(float(np.median(a)), 2),
                     "p90_us": round(float(np.percentile(a, 90)), 2),
                     "min_us": round(float(a.min()), 2), "max_us": round(float(a.max()), 2)}
    return out


def summarize_counters(run_dirs):
    """Per-kernel dispatch count and mean value per dispatch of every counter
    in the counter_collection.csv files that rocprofv3 --pmc runs wrote under
    run_dirs (one pass each; kernel names shortened as in summarize_trace)."""
    import csv
    out = {}
    for run_dir in run_dirs:
        vals = {}
        for dirpath, _, files in os.walk(run_dir):
            for fn in files:
                if not fn.endswith("counter_collection.csv"):
                    continue
                with open(os.path.join(dirpath, fn), newline="") as f:
                    for row in csv.DictReader(f):
                        name = row["Kernel_Name"].replace("void ", "")
                        name = name.replace("(anonymous namespace)::", "").split("(")[0]
                        per = vals.setdefault(name, {})
                        per.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
        for name, per in vals.items():
            rec = out.setdefault(name, {})
            rec.setdefault("dispatches", {})
            for c, v in sorted(per.items()):
                rec["dispatches"][c] = len(v)
                rec[c] = round(float(np.mean(v)), 1)
    return out


# MI355X: 256 compute units of 4 SIMDs in 8 XCDs; GRBM_GUI_ACTIVE counts in
# every XCD.
SIMDS, XCDS = 1024, 8


def counters_table(table, copy_mib=256):
    """Text table of the derived per-dispatch figures: waves, VALU and LDS
    instructions per wave, MFMA instructions, MFMA busy fraction, LDS bank
    conflict cycles, and HBM MB read and written (FETCH_SIZE / WRITE_SIZE
    scaled by what they read for the calibration copy of copy_mib MiB, if the
    runs hold it)."""
    neg = [v for k, v in table.items() if "neg_kernel" in k]
    f_read = f_write = None
    if neg and "FETCH_SIZE" in neg[0] and "WRITE_SIZE" in neg[0]:
        f_read = copy_mib * (1 << 20) / (neg[0]["FETCH_SIZE"] * 1024.0)
        f_write = copy_mib * (1 << 20) / (neg[0]["WRITE_SIZE"] * 1024.0)
    lines = []
    if f_read:
        lines.append(f"HBM bytes = FETCH_SIZE KiB x 1024 x {f_read:.4f} + WRITE_SIZE KiB x 1024 x "
                     f"{f_write:.4f} (factors from the {copy_mib} MiB copy calibration)")
    lines.append(f"{'kernel':46s} {'waves':>7s} {'VALU/wave':>9s} {'MFMA':>9s} {'MFMA busy':>9s} "
                 f"{'LDS/wave':>8s} {'bank cf':>8s} {'read MB':>8s} {'write MB':>8s}")
    for name, r in sorted(table.items(), key=lambda kv: kv[0]):
        if not name.startswith("q4::"):
            continue
        waves = r.get("SQ_WAVES", 0.0)
        per = (lambda c: r[c] / waves if waves and c in r else float("nan"))
        busy = float("nan")
        if r.get("GRBM_GUI_ACTIVE"):
            busy = r.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMDS * r["GRBM_GUI_ACTIVE"] / XCDS)
        rd = r["FETCH_SIZE"] * 1024 * f_read / 1e6 if f_read and "FETCH_SIZE" in r else float("nan")
        wr = r["WRITE_SIZE"] * 1024 * f_write / 1e6 if f_write and "WRITE_SIZE" in r else float("nan")
        lines.append(f"{name[:46]:46s} {waves:7.0f} {per('SQ_INSTS_VALU'):9.0f} "
                     f"{r.get('SQ_INSTS_MFMA', float('nan')):9.0f} {100 * busy:8.1f}% "
                     f"{per('SQ_INSTS_LDS'):8.1f} {r.get('SQ_LDS_BANK_CONFLICT', float('nan')):8.0f} "
                     f"{rd:8.1f} {wr:8.2f}")
    return "\n".join(lines)


def trace_table(table):
    lines = [f"{'Kernel (us)':52s} {'calls':>6s} {'mean':>8s} {'p10':>8s} {'median':>8s} "
             f"{'p90':>8s} {'min':>8s} {'max':>8s}"]
    for k, v in table.items():
        lines.append(f"{k[:52]:52s} {v['calls']:6d} {v['mean_us']:8.2f} {v['p10_us']:8.2f} "
                     f"{v['median_us']:8.2f} {v['p90_us']:8.2f} {v['min_us']:8.2f} {v['max_us']:8.2f}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    # untimed launches after the clock warm-up (CLOCK_WARM_MS); with 200 warmup
    # launches and no warm-up the decode read 20.5 us per launch, 19.4-19.8 after 3000
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain copy kernel of this many MiB (for counter scaling)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print per-kernel duration statistics (mean, p10, median, p90) of a "
                         "rocprofv3 --kernel-trace run of this script (no GPU needed)")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR", nargs="+",
                    help="print each kernel's mean counter values per dispatch from "
                         "rocprofv3 --pmc runs of this script, one pass each (no GPU needed)")
    ap.add_argument("--text", action="store_true",
                    help="with --summarize-trace or --summarize-counters: a text table "
                         "(derived figures for the counters) in place of JSON")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script with --calibrate-copy-mib 256 into the decode kernel's "
                         "HBM traffic record under profiles/ (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_trace:
        t = summarize_trace(args.summarize_trace)
        print(trace_table(t) if args.text else json.dumps(t, indent=1))
        return
    if args.summarize_counters:
        t = summarize_counters(args.summarize_counters)
        print(counters_table(t) if args.text else json.dumps(t, indent=1))
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], 256,
                      "gemv_decode_gate_up", DECODE_KERNEL + "(", weight_bytes(34816, 5120),
                      os.path.join(ROOT, "profiles", "gemv_decode_gate_up_pmc.json"))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the decode and prefill paths would shard the weight rows by output feature)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_q4_block_amd as q4
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    digest = csrc_digest()

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.calibrate_copy_mib:
        progress(f"calibration copy: {args.calibrate_copy_mib} MiB")
        calibration_copy(torch, args.calibrate_copy_mib)
    progress("decode_gate_up: generating inputs")
    head = Dense(torch, q4, "decode_gate_up")
    progress(f"decode_gate_up: timing {args.steps} steps over {head.copies} weight copies")
    blocks_ms = []
    ms_step, ev_ms = time_steps(torch, head, args.steps, args.warmup, CLOCK_WARM_MS,
                                blocks=10 if args.steps >= 100 else 0, spread=blocks_ms)
    copies = head.copies
    progress("decode_gate_up: sampling the shader clock under load")
    sclk = sample_sclk(torch, head)
    value = head.wbytes / (ms_step * 1e-3) / 1e9
    achieved = head.wbytes / (ev_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile("gemv_decode_gate_up", digest),
            # K = 5120 is 160 blocks a row: two full 64-lane stages and a
            # leftover stage of 32 blocks split between the half-waves
            "kernel": DECODE_KERNEL,
            "avg_launch_us": round(ev_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": head.wbytes}
    if blocks_ms:
        # the timed launches in 10 consecutive blocks: each block's mean
        us = sorted(b * 1e3 for b in blocks_ms)
        roof["launch_us_over_blocks"] = {"blocks": len(us), "min": round(us[0], 3),
                                         "median": round(float(np.median(us)), 3),
                                         "max": round(us[-1], 3)}
    progress("decode_gate_up: streaming ceiling (a read-only pass over the same copies)")
    probe = StreamRead(torch, q4, head)
    _, pr_ms = time_steps(torch, probe, max(50, args.steps // 4), max(10, args.warmup // 10),
                          CLOCK_WARM_MS)
    ceil = probe.bytes / (pr_ms * 1e-3) / 1e9
    roof["stream_read_ceiling"] = {"kernel": "q4::stream_read_kernel",
                                   "bytes_per_launch": probe.bytes,
                                   "avg_launch_us": round(pr_ms * 1e3, 3),
                                   "GB/s": round(ceil, 1),
                                   "frac_of_peak": round(ceil / HBM_PEAK_GBS, 4)}
    roof["frac_of_stream_ceiling"] = round(achieved / ceil, 4)
    del probe, head
    torch.cuda.empty_cache()

    others = {}
    if not args.headline_only:
        steps = max(50, args.steps // 10)
        for name in ("batched_down", "prefill"):
            progress(f"{name}: generating inputs")
            w = Dense(torch, q4, name)
            progress(f"{name}: timing")
            _, ev = time_steps(torch, w, steps, max(10, args.warmup // 10), CLOCK_WARM_MS)
            if name == "prefill":
                tf = w.flops / (ev * 1e-3) / 1e12
                others[name] = {"M": w.M, "N": w.N, "K": w.K, "avg_launch_us": round(ev * 1e3, 2),
                                "TFLOP/s": round(tf, 2), "frac_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
            else:
                gbs = w.wbytes / (ev * 1e-3) / 1e9
                others[name] = {"M": w.M, "N": w.N, "K": w.K, "avg_launch_us": round(ev * 1e3, 2),
                                "weight_GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
            del w
            torch.cuda.empty_cache()
        progress("mx_decode_gate_up: generating inputs")
        w = MxDense(torch, q4)
        progress("mx_decode_gate_up: timing")
        _, ev = time_steps(torch, w, args.steps // 2, max(10, args.warmup // 2), CLOCK_WARM_MS)
        gbs = w.wbytes / (ev * 1e-3) / 1e9
        others["mx_decode_gate_up"] = {"M": w.M, "N": w.N, "K": w.K,
                                       "format": "e2m1 elements, E8M0 scale per 32",
                                       "avg_launch_us": round(ev * 1e3, 2),
                                       "weight_GB/s": round(gbs, 1),
                                       "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del w
        torch.cuda.empty_cache()
        progress("mx_prefill: generating inputs")
        w = MxDense(torch, q4, "mx_prefill")
        progress("mx_prefill: timing")
        _, ev = time_steps(torch, w, steps, max(10, args.warmup // 10), CLOCK_WARM_MS)
        tf = w.flops / (ev * 1e-3) / 1e12
        others["mx_prefill"] = {"M": w.M, "N": w.N, "K": w.K,
                                "format": "e2m1 elements, E8M0 scale per 32",
                                "avg_launch_us": round(ev * 1e3, 2), "TFLOP/s": round(tf, 2),
                                "frac_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
        del w
        torch.cuda.empty_cache()
        progress("moe: generating inputs")
        w = MoE(torch, q4)
        progress("moe: timing")
        _, ev = time_steps(torch, w, steps, max(10, args.warmup // 10), CLOCK_WARM_MS)
        gbs = w.wbytes / (ev * 1e-3) / 1e9
        others["moe"] = {"T": w.T, "topk": w.topk, "E": w.E, "N": w.N, "K": w.K,
                         "touched_experts": w.touched, "avg_call_us": round(ev * 1e3, 2),
                         "touched_weight_GB/s": round(gbs, 1),
                         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del w
        torch.cuda.empty_cache()
        progress("moe_ffn: generating inputs")
        w = MoeFfn(torch, q4)
        progress("moe_ffn: timing")
        _, ev = time_steps(torch, w, steps, max(10, args.warmup // 10), CLOCK_WARM_MS)
        gbs = w.wbytes / (ev * 1e-3) / 1e9
        others["moe_ffn"] = {"T": w.T, "topk": w.topk, "E": w.E, "H": w.H, "F": w.F,
                             "touched_experts": w.touched, "avg_call_us": round(ev * 1e3, 2),
                             "touched_weight_GB/s": round(gbs, 1),
                             "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del w
        torch.cuda.empty_cache()
        import synthetic
        # the same expert shapes at 512 tokens: the grouped matrix-core path
        for name, cls in (("moe_prefill", MoE), ("moe_ffn_prefill", MoeFfn)):
            progress(f"{name}: generating inputs")
            w = cls(torch, q4, config=synthetic.MOE_PREFILL_CONFIGS[name])
            progress(f"{name}: timing")
            _, ev = time_steps(torch, w, max(20, steps // 4), 10, CLOCK_WARM_MS)
            gbs = w.wbytes / (ev * 1e-3) / 1e9
            tf = w.flops / (ev * 1e-3) / 1e12
            rec = {"T": w.T, "topk": w.topk, "E": w.E}
            rec.update({"N": w.N, "K": w.K} if cls is MoE else {"H": w.H, "F": w.F})
            rec.update({"touched_experts": w.touched, "avg_call_us": round(ev * 1e3, 2),
                        "touched_weight_GB/s": round(gbs, 1),
                        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                        "TFLOP/s": round(tf, 2), "frac_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4)})
            others[name] = rec
            del w
            torch.cuda.empty_cache()
        # RMSNorm prologue and super-block scales at the decode and prefill
        # shapes, and the quantiser on the decode projection's weights
        for name, cls in (("rms_decode_gate_up", RmsDense), ("rms_prefill", RmsDense),
                          ("sb_decode_gate_up", SbDense), ("sb_prefill", SbDense)):
            progress(f"{name}: generating inputs")
            w = cls(torch, q4, name)
            progress(f"{name}: timing")
            _, ev = time_steps(torch, w, steps, max(10, args.warmup // 10), CLOCK_WARM_MS)
            rec = {"M": w.M, "N": w.N, "K": w.K, "avg_launch_us": round(ev * 1e3, 2)}
            if w.M == 1:
                gbs = w.wbytes / (ev * 1e-3) / 1e9
                rec.update({"weight_GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
            else:
                tf = w.flops / (ev * 1e-3) / 1e12
                rec.update({"TFLOP/s": round(tf, 2), "frac_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4)})
            others[name] = rec
            del w
            torch.cuda.empty_cache()
        progress("quantize: generating inputs")
        w = Quantize(torch, q4)
        progress("quantize: timing")
        _, ev = time_steps(torch, w, max(20, steps // 4), 10, CLOCK_WARM_MS)
        gbs = w.bytes / (ev * 1e-3) / 1e9
        others["quantize"] = {"N": w.N, "K": w.K, "avg_launch_us": round(ev * 1e3, 2),
                              "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                              "bytes": "bf16 weights read, codes and fp16 scales written"}
        del w
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        progress("cpu baseline: timing the oracle")
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    if not args.no_cpu_baseline and not args.headline_only:
        progress("cpu baselines: batched_down, prefill sample, moe")
    cpu_others = (None if args.no_cpu_baseline or args.headline_only
                  else cpu_baselines_other())

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "clock_warm_ms": CLOCK_WARM_MS,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode_gate_up: y[1][34816] = x[1][5120] . dequant(W)^T, "
                               "int4 codes (value = code - 8), 32-element blocks, fp16 scales, "
                               "bf16 x, fp32 y, seed 1",
                   "M": 1, "K": 5120, "N": 34816, "parallelism": "single GPU",
                   "rotating_weight_copies": copies, "csrc_digest": digest},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baselines_other": cpu_others,
        "env": {"device": torch.cuda.get_device_properties(0).gcnArchName,
                "hip_runtime": torch.version.hip, "torch": torch.__version__,
                "sclk_mhz_under_load": sclk, "commit": git_commit(),
                "library_built_from": library_build_info(),
                "sources_digest": all_sources_digest(),
                "decode_kernel_resources": kernel_resources(
                    "_ZN2q415gemv_lds_kernelILi1ELi2ELi1ELb0EtEE")},
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Build libq4.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc."""
from __future__ import annotations

import json
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libq4.so")
SOURCES = ["q4_api.hip", "q4_dequant.hip", "q4_gemv.hip", "q4_gemm.hip", "q4_moe.hip",
           "q4_moe_mm.hip", "q4_mx.hip",
           "q4_norm.hip", "q4_probe.hip", "q4_quant.hip", "q4_sb.hip",
           "q4_small.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are kept out of the code objects on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
         "-Wall", "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# The tiled kernel applies each block's scale to the MFMA partial with VALU
# fmas; with the MFMA results in VGPRs (not AGPRs) those partials need no
# copy before the fmas read them.
EXTRA = {"q4_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "q4_moe_mm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


# Per-kernel register, LDS and occupancy figures of the build (the
# compiler's resource-usage remarks), for the benchmark record.
RESOURCES = os.path.join(PKG, "kernel_resources.json")
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs",
           "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
           "Occupancy [waves/SIMD]": "waves_per_simd", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds_bytes"}


def _resources(remarks: str) -> dict:
    out, cur = {}, None
    for line in remarks.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = out.setdefault(body.split(":", 1)[1].strip(), {})
        elif cur is not None and ":" in body:
            k, v = body.rsplit(":", 1)
            if k.strip() in _FIELDS:
                try:
                    cur[_FIELDS[k.strip()]] = int(v.strip())
                except ValueError:
                    pass
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-Rpass-analysis=kernel-resource-usage",
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, _resources(r.stderr)


# The commit the library is built from, and whether the kernel sources or
# the C ABI header differed from it at build time, for run records made
# where the tree carries no git metadata.
BUILD_INFO = os.path.join(PKG, "build_info.json")


def _build_info() -> dict:
    def git(*args):
        r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True,
                           timeout=20)
        return r.stdout.strip() if r.returncode == 0 else None
    try:
        head = git("rev-parse", "HEAD")
        status = git("status", "--porcelain", "--", "quantized_q4_block_amd/csrc", "include")
    except (OSError, subprocess.SubprocessError):
        head, status = None, None
    return {"commit": head or None,
            "sources_modified": None if head is None or status is None else status != ""}


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    res = {}
    for _, r in results:
        res.update(r)
    with open(RESOURCES, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
        f.write("\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(BUILD_INFO, "w") as f:
        json.dump(_build_info(), f, indent=1, sort_keys=True)
        f.write("\n")
    return LIB


if __name__ == "__main__":
    print(build())

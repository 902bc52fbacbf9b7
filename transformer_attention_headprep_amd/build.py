"""Build libattn.so and libpeak.so (HIP for gfx950) in-tree with hipcc.

    python -m transformer_attention_headprep_amd.build

Each source is compiled to an object under ``_build/`` in parallel, then linked into
``transformer_attention_headprep_amd/libattn.so`` (the attention path) and
``transformer_attention_headprep_amd/libpeak.so`` (calibration kernels for the
benchmark).  Device code is built for gfx950 only, with packed-f32 instructions turned
off.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libattn.so")
PEAK_OUT = os.path.join(PKG, "libpeak.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["attn_api.cpp", "prep.hip", "prefill_f32.hip", "prefill_bf16.hip", "decode.hip", "kvq.hip", "rows8.hip"]
PEAK_SOURCES = ["peak.hip"]
# Per-source flags.  The bf16 prefill kernel never sees NaN operands in valid use, so it
# drops NaN quieting: row maxima become single v_max3 instructions.
# The quantised-cache coding decides integer codes in f32 in the order it is written (the
# same order the checker uses), so that file forbids fusing a multiply into an add.
EXTRA = {"prefill_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"], "kvq.hip": ["-ffp-contract=off"],
         "rows8.hip": ["-ffp-contract=off"]}
ARCH = "gfx950"
# Kernels whose tile waits count their own loads into LDS (vmcnt) and so must not spill
# registers: scratch traffic would count too.  The build fails if one of them spills.
NO_SPILL = {"prefill_bf16.hip": ("prefill_bf16_kernel",), "decode.hip": ("decode_rows_kernel",)}
RESOURCE_REPORT = os.path.join(BUILD_DIR, "resource_usage.txt")


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libattn")
    return path


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    report = ["-Rpass-analysis=kernel-resource-usage"] if src in NO_SPILL else []
    cmd = [hipcc()] + _flags() + EXTRA.get(src, []) + report + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
    if report:
        _resources[src] = parse_resource_usage(r.stderr)
    return obj


_resources: dict = {}


def parse_resource_usage(text: str):
    """[(kernel, vgprs, vgpr_spill, sgpr_spill)] from the compiler's resource remarks."""
    rows, cur = [], None
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].strip()
        if body.startswith("Function Name:"):
            cur = [body.split(":", 1)[1].split(" [")[0].strip(), None, None, None]
            rows.append(cur)
        elif cur is not None:
            for key, i in (("VGPRs:", 1), ("VGPRs Spill:", 2), ("SGPRs Spill:", 3)):
                if body.startswith(key):
                    cur[i] = int(body.split(":", 1)[1].split()[0])
    return [tuple(r) for r in rows]


def _check_spills() -> None:
    lines, bad = [], []
    for src, rows in sorted(_resources.items()):
        for name, vgprs, vspill, sspill in rows:
            lines.append("%s %s vgprs=%s vgpr_spill=%s sgpr_spill=%s" % (src, name, vgprs, vspill, sspill))
            if any(k in name for k in NO_SPILL[src]) and vspill:
                bad.append("%s: %d VGPRs spilled" % (name, vspill))
    with open(RESOURCE_REPORT, "w") as f:
        f.write("\n".join(lines) + "\n")
    if bad:
        raise RuntimeError("kernels that must not spill registers do:\n" + "\n".join(bad))


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)


def build(jobs: int = 8) -> str:
    """Compile every source and link libattn.so and libpeak.so; returns libattn's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    _check_spills()
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PEAK_OUT)
    return OUT


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 8))

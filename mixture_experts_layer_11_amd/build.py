"""Build libmoe.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m mixture_experts_layer_11_amd.build        # or build() from Python

Every call recompiles.  Sources: csrc/*.hip and csrc/*.cpp; header: include/moe.h.
The build fails if any kernel needs scratch memory (register spills or private
arrays): the kernels are written to live in registers and LDS only.  The
per-kernel register, LDS and occupancy figures the compiler reports are kept
in _build/resources.txt.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++20",
    "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
    # packed fp32 VALU ops are kept out of the device code (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, objdir):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, RESOURCE_REMARKS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    usage = _resource_usage(lines)
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l and not l.lstrip().startswith(("|", "^"))
                    and not re.match(r"^\s*\d+ \|", l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err, usage


def _resource_usage(lines):
    """{kernel: {field: value}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for l in lines:
        m = re.search(r"remark: Function Name: (\S+)", l)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\S+) \[-Rpass-analysis", l)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = _sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, objdir), srcs))
    usage = {}
    for _, msg, u in results:
        usage.update(u)
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
    with open(os.path.join(objdir, "resources.txt"), "w") as f:
        for k in sorted(usage):
            f.write(k + " " + " ".join(f"{a}={b}" for a, b in usage[k].items()) + "\n")
    spill = {k: v.get("ScratchSize [bytes/lane]") for k, v in usage.items()
             if v.get("ScratchSize [bytes/lane]", "0") != "0"}
    if spill:
        raise RuntimeError(f"kernels that need scratch memory (bytes per lane): {spill}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def clean():
    shutil.rmtree(os.path.join(HERE, "_build"), ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libkcr.so, the gfx950 HIP library behind the C ABI in include/kcr.h.

Every source in csrc/ is compiled by hipcc for gfx950 only, in parallel, and
linked into kv_cache_rmsnorm_amd/libkcr.so. norm_inst.hip is compiled once
per storage type and norm variant (six objects). Packed-fp32 instruction
selection is switched off for the device code. The build fails if any
kernel uses scratch memory.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkcr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# (storage type, add variant) pairs of the row-norm engine
NORM_VARIANTS = [(t, add) for t in ("Bf16", "F16", "F32") for add in (0, 1)]


def _headers_mtime() -> float:
    hdrs = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(INCLUDE, "*.h"))
    return max(os.path.getmtime(h) for h in hdrs)


def _compile(job) -> str:
    src, defines, incremental = job
    tag = "".join(f"_{v}" for _, v in defines)
    obj = os.path.join(OUT_DIR, os.path.basename(src) + tag + ".o")
    if incremental and os.path.exists(obj) and \
            os.path.getmtime(obj) > max(os.path.getmtime(src), _headers_mtime()):
        return obj
    cmd = [HIPCC, *CXXFLAGS, *[f"-D{k}={v}" for k, v in defines], "-Rpass-analysis=kernel-resource-usage",
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    remarks = [l for l in r.stderr.splitlines() if "remark:" in l]
    bad = scratch_users(remarks)
    if bad:
        raise RuntimeError(f"{src}: kernels that use scratch memory (spills, or a private copy of the "
                           f"argument block): {', '.join(bad)}")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
    noise = [l for l in r.stderr.splitlines() if "warning:" in l and "packed-fp32-ops" not in l]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def scratch_users(remarks: list[str]) -> list[str]:
    """Kernels whose resource-usage remarks report scratch memory: every
    kernel here keeps its state in registers and LDS, so scratch means a
    register spill or an argument block the compiler copied to memory."""
    bad, name = [], None
    for line in remarks:
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0 and name:
            bad.append(name)
    return bad


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libkcr.so. Always
    rebuilds every object unless `incremental`, which keeps objects newer
    than their source and every header."""
    os.makedirs(OUT_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    inst = os.path.join(CSRC, "norm_inst.hip")
    work = [(s, (), incremental) for s in sources if s != inst]
    work += [(inst, (("KCR_NORM_T", t), ("KCR_NORM_ADD", add)), incremental) for t, add in NORM_VARIANTS]
    # the norm instantiations are the slowest; start them first
    work.sort(key=lambda j: j[0] != inst)
    jobs = min(len(work), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, work))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(sources)} sources ({len(work)} objects)")
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)

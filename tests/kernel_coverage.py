"""Which of the library's kernel variants the GPU parity suite runs.

Compares the kernels named in a rocprofv3 kernel trace of
``pytest tests -m gpu`` with every kernel instantiated in libkcr.so (the
host-side launch stubs that the HIP compiler emits for each __global__
instantiation, listed by ``nm``), and prints a markdown summary: per kernel
template, how many variants are compiled and how many ran, and any that did
not run.

    cd /tmp && rocprofv3 --kernel-trace --output-format csv -d $REPO/gpurun_out/prof_tests \\
        -o tests -- python3 -u -m pytest $REPO/tests -m gpu -q
    cd $REPO && python3 tests/kernel_coverage.py gpurun_out/prof_tests
"""
from __future__ import annotations

import collections
import csv
import glob
import gzip
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "..", "kv_cache_rmsnorm_amd", "libkcr.so")
STUB = "__device_stub__"


def canonical(name: str) -> str:
    """A kernel's template-id without return type, parameter list or spaces."""
    name = re.sub(r"^void ", "", name.strip())
    return name.split("(")[0].replace(" ", "").replace(STUB, "")


def compiled_kernels(nm_output: str) -> set[str]:
    out = set()
    for line in nm_output.splitlines():
        if STUB not in line:
            continue
        sym = re.sub(r"^[0-9a-fA-F]+ [A-Za-z] ", "", line.strip())
        out.add(canonical(sym))
    return out


def traced_kernels(trace_dir: str) -> set[str]:
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv*"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    names = set()
    for p in paths:
        opener = gzip.open if p.endswith(".gz") else open
        with opener(p, "rt") as f:
            for row in csv.DictReader(f):
                names.add(canonical(row["Kernel_Name"]))
    return names


def summary(compiled: set[str], ran: set[str]) -> str:
    fam_all, fam_ran = collections.Counter(), collections.Counter()
    missing = []
    for k in sorted(compiled):
        fam = k.split("<")[0]
        fam_all[fam] += 1
        if k in ran:
            fam_ran[fam] += 1
        else:
            missing.append(k)
    lines = ["| kernel template | variants compiled | variants run by the GPU tests |", "|---|---|---|"]
    for fam in sorted(fam_all):
        lines.append(f"| `{fam}` | {fam_all[fam]} | {fam_ran[fam]} |")
    total, done = sum(fam_all.values()), sum(fam_ran.values())
    lines.append(f"| all | {total} | {done} |")
    lines.append("")
    if missing:
        lines.append("Not run:")
        lines.append("")
        lines += [f"- `{k}`" for k in missing]
    else:
        lines.append("Every compiled kernel variant ran at least once.")
    return "\n".join(lines) + "\n"


def main(argv):
    if len(argv) != 2:
        raise SystemExit(__doc__)
    nm = subprocess.run(["nm", "-C", "--defined-only", LIB], capture_output=True, text=True, check=True)
    sys.stdout.write(summary(compiled_kernels(nm.stdout), traced_kernels(argv[1])))


if __name__ == "__main__":
    main(sys.argv)

"""Builds libssm_adjoint.so (gfx950) in-tree with hipcc.

Each source is compiled to an object in parallel, then the objects are
linked.  The compiler's per-kernel resource report is checked as part of the
build.  The fused reverse walk (k_bwd_main) places its end-of-sub-chunk
memory-counter wait by hand, counting exactly the walk's own stores issued
after the next sub-chunk's loads; compiler-generated scratch traffic there
(a register spill) would break the premise that nothing else is in flight
and would add waits the schedule does not expect, so any scratch in that
kernel fails the build.  Scratch in other kernels is reported.
"""
from __future__ import annotations

import glob
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssm_adjoint.so")
OBJ = os.path.join(HERE, "_build")

HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=gfx950",
    "-fPIC",
    # packed fp32 VALU forms stay disabled in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def kernel_resources(remarks: str) -> dict:
    """{kernel symbol: {field: value}} from the compiler's resource remarks."""
    out: dict = {}
    cur = None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z ]*?)(?: \[[^\]]*\])?: (\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


# Kernels that must not use scratch memory (symbol substrings).
NO_SCRATCH = ("k_bwd_main",)


def scratch_users(res: dict) -> list[tuple[str, int, int]]:
    """(kernel, scratch bytes per lane, spilled VGPRs) of every kernel with
    scratch memory.  SGPR spills go to VGPR lanes, not memory, and are not
    counted."""
    out = []
    for name, f in res.items():
        scratch = int(f.get("ScratchSize", "0"))
        if scratch:
            out.append((name, scratch, int(f.get("VGPRs Spill", "0"))))
    return out


def check_no_scratch(res: dict) -> list[str]:
    """Kernels of NO_SCRATCH whose report shows scratch memory, and a note if
    none of them was reported at all."""
    bad = [f"{n}: scratch {b} B/lane, {v} spilled VGPRs" for n, b, v in scratch_users(res)
           if any(k in n for k in NO_SCRATCH)]
    for k in NO_SCRATCH:
        if not any(k in n for n in res):
            bad.append(f"no resource report for {k}")
    return bad


def _compile(hipcc: str, src: str) -> tuple[str, str, dict]:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *REMARKS, "-c", "-o", obj, src]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} ({proc.returncode}):\n{proc.stderr[-8000:]}")
    return obj, " ".join(cmd), kernel_resources(proc.stderr)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    res: dict = {}
    for obj, cmd, r in results:
        if verbose:
            print(cmd, file=sys.stderr)
        res.update(r)
    if not res:
        raise RuntimeError("no kernel resource report from the compiler")
    bad = check_no_scratch(res)
    if bad:
        raise RuntimeError("scratch memory in a kernel whose memory waits are placed by hand:\n  "
                           + "\n  ".join(bad))
    if verbose:
        for n, b, v in scratch_users(res):
            print(f"note: {n} uses {b} B/lane of scratch ({v} spilled VGPRs)", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[r[0] for r in results]]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed ({proc.returncode}):\n{proc.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"{len(res)} kernels; no scratch in {', '.join(NO_SCRATCH)}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

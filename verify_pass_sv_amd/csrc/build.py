"""Build libspecverify.so in-tree with hipcc for gfx950.

Each .hip source is compiled to an object under verify_pass_sv_amd/_build/
and linked into verify_pass_sv_amd/libspecverify.so.  Always recompiles.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspecverify.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "qgemm_w4.hip", "qgemm_w4_packed.hip", "pass.hip", "pass_chain.hip",
           "qgemm_w8.hip", "qgemm_w4_i8.hip",
           "hadamard_i8.hip", "verify_accept.hip",
           "verify_sampled.hip", "verify_coupled.hip"]

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed FP32 VALU ops are not emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{HERE}",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


# Kernels that wait on exact counts of their own outstanding vector memory
# operations: a register spill would add scratch loads and stores to that
# count, so their build fails if any kernel of the file uses scratch.
NO_SCRATCH = {"pass.hip", "pass_chain.hip", "qgemm_w4_packed.hip", "qgemm_w4.hip"}
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def _check_no_scratch(src, text):
    kernel = None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) != 0:
            raise RuntimeError(f"{src}: kernel {kernel} uses {m.group(1)} bytes/lane of scratch "
                               "(register spills break its exact memory-operation count)")


def _run(cmd, verbose, src=None):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if src in NO_SCRATCH and p.returncode == 0:
        _check_no_scratch(src, p.stdout)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if ("packed-fp32-ops" not in l and "remark:" not in l) or "error" in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False, jobs=None):
    """Compile every HIP source for gfx950 and link libspecverify.so."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        extra = RESOURCE_REMARKS if src in NO_SCRATCH else []
        cmds.append(([hipcc, *CXXFLAGS, *extra, "-c", os.path.join(HERE, src), "-o", obj], src))
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c[0], verbose, c[1]), cmds))
    tmp = LIB + ".tmp"
    # -z defs: a symbol left undefined (such as a kernel launch stub the host
    # compile dropped) fails the link instead of the first load.
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", "-o", tmp, *objs],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

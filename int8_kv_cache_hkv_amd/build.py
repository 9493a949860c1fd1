"""Build libhkv.so (all HIP kernels + the C-ABI host code) for gfx950, in-tree.

Every source is compiled to an object of its own, in parallel, and the
objects are linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhkv.so")


# decode_inst.hip is compiled once per (head_dim, GQA group, cold-tile format) instance
DECODE_INST = "decode_inst.hip"
DECODE_INSTANCES = [(d, g, bits) for bits in (8, 4, 0) for d in (128, 64) for g in (1, 2, 4, 8)]


def sources() -> list:
    """Every translation unit of the library: the .hip kernel files and the host .cpp files."""
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def compile_units() -> list:
    """(source, extra defines, object name) of every object the library is linked from."""
    units = []
    for src in sources():
        if src == DECODE_INST:
            for d, g, bits in DECODE_INSTANCES:
                units.append((src, [f"-DHKV_D={d}", f"-DHKV_G={g}", f"-DHKV_BITS={bits}"],
                              f"decode_d{d}_g{g}_b{bits}.o"))
        else:
            units.append((src, [], src + ".o"))
    return units


HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",   # IEEE fp32 division for the quantiser
    "-fno-fast-math", "-ffp-contract=fast", "-fno-strict-aliasing",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libhkv")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (res.stderr or "").splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd[-3:])}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 0, out: str = LIB, host_flags: tuple = ()) -> str:
    """Compile every source into int8_kv_cache_hkv_amd/libhkv.so, or `out` (always recompiles).

    host_flags: extra options for the host side of every compile only (each is passed behind
    -Xarch_host, e.g. a sanitizer build of the host code; device code is unchanged)."""
    cc = hipcc()
    host = [x for f in host_flags for x in ("-Xarch_host", f)]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = jobs or min(16, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="hkv_build_") as tmpd:
        objs = []
        cmds = []
        for src, defs, name in compile_units():
            obj = os.path.join(tmpd, name)
            objs.append(obj)
            cmds.append([cc, *HIPCC_FLAGS, *host, *defs, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

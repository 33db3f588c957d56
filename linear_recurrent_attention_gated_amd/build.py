"""Builds libgdn.so (the C-ABI library of include/gdn.h) in-tree for gfx950.

Every translation unit is compiled with hipcc for gfx950 only; the prefill variants
are split into one object per (element type, chunk) so they compile in parallel.
Packed-fp32 instruction selection is disabled for device code.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
          "-Wno-unused-function", "-I" + CSRC, "-I" + os.path.join(ROOT, "include")]

HEADERS = ["gdn_device.h", "gdn_prefill.h", "gdn_decode.h", "gdn_sequential.h", "gdn_launch.h"]


def _units():
    units = []
    for bf in (1, 0):
        for c in (16, 32, 64):
            tag = f"prefill_{'bf16' if bf else 'f32'}_c{c}"
            units.append((tag, "gdn_prefill_inst.hip", [f"-DGDN_ELEM_BF16={bf}", f"-DGDN_CHUNK={c}"]))
    units.append(("decode", "gdn_decode.hip", []))
    units.append(("sequential", "gdn_sequential.hip", []))
    units.append(("api", "gdn_api.cpp", []))
    return units


def _compile(unit, verbose):
    tag, src, defs = unit
    obj = os.path.join(BUILD, tag + ".o")
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + defs + ["-x", "hip", "-c", os.path.join(CSRC, src),
                                                     "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {tag}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    units = _units()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(units)))) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), units))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

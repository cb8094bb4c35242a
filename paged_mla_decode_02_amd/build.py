"""Build libmla_decode.so in-tree with hipcc for gfx950.

Usage: python -m paged_mla_decode_02_amd.build   (or build() from Python).
Objects go to paged_mla_decode_02_amd/_build/, the library next to this file.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla_decode.so")
SOURCES = ["plan.cpp", "error.cpp", "api.cpp", "noalloc.hip", "decode.hip", "kernels.hip", "cache_write.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are turned off for all device code (the compiler would
# otherwise form v_pk_* fp32 instructions from ordinary float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr)
    # the host pass does not know the device target feature; that is harmless
    out = "\n".join(l for l in out.splitlines() if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    common = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
              "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [cc] + lang + common + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        objs.append(obj)
        procs.append(cmd)
    # the decode kernel's device assembly, for the QK-chain check below
    asm = os.path.join(OBJDIR, "decode.gfx950.s")
    procs.append([cc, "-x", "hip"] + common + DEVICE_FLAGS +
                 ["--cuda-device-only", "-S", os.path.join(CSRC, "decode.hip"), "-o", asm])
    # compile (a few in parallel)
    running = []
    for cmd in procs:
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(running) >= jobs:
            _wait(running.pop(0), verbose)
    for r in running:
        _wait(r, verbose)
    _check_decode_asm(asm)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


def _check_decode_asm(path):
    sys.path.insert(0, PKG)
    try:
        from asm_check import (check_m0, check_qk_chains, check_scratch_in_step_loops, check_valu_to_mfma,
                               check_waits_behind_tile_loads)
    finally:
        sys.path.pop(0)
    with open(path) as f:
        text = f.read()
    chains, bad = check_qk_chains(text)
    if chains == 0 or bad:
        raise RuntimeError(f"decode.hip: the generated code breaks the QK accumulator chains "
                           f"({chains} chains; offending lines of {path}):\n" + "\n".join(bad[:20]))
    hazards = check_valu_to_mfma(text)
    if hazards:
        raise RuntimeError(f"decode.hip: an assembly MFMA reads a VALU result without the required "
                           f"wait states (offending lines of {path}):\n" + "\n".join(hazards[:20]))
    m0 = check_m0(text)
    if m0:
        raise RuntimeError(f"decode.hip: M0 is used outside the direct-to-LDS load sequences, which set "
                           f"it without declaring it (offending lines of {path}):\n" + "\n".join(m0[:20]))
    spills = check_scratch_in_step_loops(text)
    if spills:
        raise RuntimeError(f"decode.hip: a spill access sits inside a per-tile step loop "
                           f"(offending lines of {path}):\n" + "\n".join(spills[:20]))
    waits = check_waits_behind_tile_loads(text)
    if waits:
        raise RuntimeError(f"decode.hip: the compiler waits for vector memory while tile loads are in flight "
                           f"(a spill reload or another load; offending lines of {path}):\n" + "\n".join(waits[:20]))


def _wait(item, verbose):
    cmd, p = item
    out, _ = p.communicate()
    out = "\n".join(l for l in out.splitlines() if "is not a recognized feature for this target" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

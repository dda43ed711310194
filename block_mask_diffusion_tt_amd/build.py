"""Build libtt.so (every HIP translation unit under csrc/) for gfx950 with
hipcc, in-tree: objects go to _build/, the library to this package directory.

Usage:  python -m block_mask_diffusion_tt_amd.build   (or build() from Python)
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtt.so")
SOURCES = ["attn.hip", "unmask.hip", "adaln.hip", "context.hip", "mamba.hip", "sublayer.hip",
           "validate.hip", "tt_api.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include")] + DEVICE_FLAGS


# The attention kernels never produce or consume NaN (masked scores are -inf,
# every softmax row has a finite score): dropping NaN canonicalization halves
# the cost of the running max.  The ILP-maximizing machine scheduler
# interleaves the matrix products with the softmax arithmetic better than the
# default occupancy-driven one for this one-workgroup-per-CU kernel
# (measured).  The iterative ILP scheduler measured about 0.8% faster still,
# but the compiler crashes on this file with it when debug info is on (the
# host-sanitizer build), so it is not used.
FILE_FLAGS = {"attn.hip": ["-fno-honor-nans", "-mllvm", "--amdgpu-sched-strategy=max-ilp"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# Files whose kernels write M0 themselves (inline asm right before each direct
# global->LDS copy).
M0_ASM = ["attn.hip", "sublayer.hip"]


def _check_m0(asm_path):
    """Fail the build if the compiler also uses M0 anywhere in a file whose
    kernels set it by hand, since nothing would then preserve it, or if any
    of its kernels spills to scratch: their copy waits count the copies in
    flight (s_waitcnt vmcnt(N)), and a spill reload is a memory operation the
    count does not know of."""
    text = open(asm_path).read()
    for m in re.finditer(r"^\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", text, re.M):
        if int(m.group(1)) != 0:
            raise RuntimeError(f"{asm_path}: a kernel uses {m.group(1)} bytes of scratch")
    if re.search(r"^\s*scratch_(load|store)", text, re.M):
        raise RuntimeError(f"{asm_path}: a kernel spills to scratch")
    lines = text.splitlines()
    for i, line in enumerate(lines):
        if re.search(r"\bm0\b", line.split(";")[0]):
            ok = (re.match(r"\s*s_mov_b32 m0, s\d+\s*$", line) and i + 2 < len(lines)
                  and lines[i + 1].strip() == "s_nop 0"
                  and lines[i + 2].strip().startswith("global_load_lds_dwordx4"))
            if not ok:
                raise RuntimeError(f"{asm_path}:{i + 1}: unexpected use of m0: {line.strip()}")


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD, src + ".o")
            objs.append(obj)
            cmd = [HIPCC] + CFLAGS + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    for src in M0_ASM:
        asm = os.path.join(BUILD, src.replace(".hip", ".s"))
        _run([HIPCC] + CFLAGS + FILE_FLAGS.get(src, []) +
             ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm])
        _check_m0(asm)
    tmp = LIB + ".tmp"
    out = _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

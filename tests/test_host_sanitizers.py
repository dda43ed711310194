"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer, without a GPU.  The library's sources are
compiled as the build compiles them, with the sanitizers added to the host
compilation only, linked into a shared library, and driven by
tests/sanitize/abi_checks.c, a plain C program that calls every entry point
with invalid arguments through the header's prototypes and checks the
returned status.  A memory error or undefined behaviour in the validation
code aborts the program."""
import concurrent.futures
import importlib.util
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_mask_diffusion_tt_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
# sanitizers for the host compilation only (each flag behind -Xarch_host)
HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang not installed")
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [str(tmp_path / (f + ".o")) for f in sources]

    # the build's own flags (loaded by path: importing the package would load libtt.so)
    spec = importlib.util.spec_from_file_location(
        "_tt_build", os.path.join(ROOT, "block_mask_diffusion_tt_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)

    def compile_one(src, obj):
        return _run([HIPCC] + build.CFLAGS + build.FILE_FLAGS.get(src, []) + ["-g"] + HOST_SAN
                    + ["-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        for (rc, out), src in zip(ex.map(compile_one, sources, objs), sources):
            assert rc == 0, f"{src}:\n{out[-3000:]}"
    lib = str(tmp_path / "libtt_san.so")
    rc, out = _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={build.ARCH}"] + HOST_SAN + objs
                   + ["-o", lib])
    assert rc == 0, out[-3000:]
    exe = str(tmp_path / "abi_checks")
    rc, out = _run([CLANG, "-g", "-O1", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", INCLUDE,
                    os.path.join(ROOT, "tests", "sanitize", "abi_checks.c"),
                    lib, f"-Wl,-rpath,{tmp_path}", "-lm", "-o", exe])
    assert rc == 0, out[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "abi checks ok" in out, out[-5000:]

"""The C ABI under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Builds the library with both sanitizers on its host code (the device code is
compiled as usual; no GPU is needed and nothing launches), links
tests/abi_fuzz/abi_fuzz.cpp against it with the same clang, and runs it: every
entry point gets a valid base shape with one defect at a time and must return
a non-OK status and a message, and the workspace-size queries must return 0
for bad arguments without overflowing for extreme ones.  Any sanitizer
report aborts the program, which fails the test.  The build takes about a
minute on eight cores.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_linear_delta_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["gdn_api.cpp", "gdn_decode.hip", "gdn_scan.hip", "gdn_chunked.hip", "gdn_segmented.hip", "gdn_moe.hip",
           "gdn_attention.hip", "gdn_noalloc.hip"]
# host-side sanitizers only: each -fsanitize= applies to the host compilation
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_abi_fuzz_under_sanitizers():
    work = tempfile.mkdtemp(prefix="gdn_asan_")
    try:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(work, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                   *SAN, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for cmd, p in procs:
            out, err = p.communicate()
            assert p.returncode == 0, f"{' '.join(cmd)}\n{err[-4000:]}"
        lib = os.path.join(work, "libgdn_san.so")
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, *objs, "-o", lib])
        exe = os.path.join(work, "abi_fuzz")
        # the driver stands in for a C caller that stores any int in the ABI's
        # enums, so it is built without the enum check (the library keeps it)
        _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize=enum",
              "-fno-sanitize-recover=all",
              "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_fuzz", "abi_fuzz.cpp"),
              lib, "-Wl,-rpath," + work, "-o", exe])
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        print(r.stdout[-3000:])
        assert r.returncode == 0, f"fuzz failed (exit {r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
        assert " 0 failures" in r.stdout
    finally:
        shutil.rmtree(work, ignore_errors=True)

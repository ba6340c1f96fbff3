"""CPU test: the library's host code (argument validation, size queries, launch set-up) built with
AddressSanitizer and UndefinedBehaviorSanitizer, and the C-ABI tests (tests/test_abi.py) run
against that build in a child process.  Only the host side is instrumented (-Xarch_host); the
device code is the ordinary gfx950 build.  Every call in those tests returns from host
validation, so no GPU is needed.  The build is cached by a hash of the sources and flags."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_51_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SRCS = ["selscan_fwd.hip", "selscan_bwd.hip", "selscan_conv.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN]


def _asan_runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _build(tmpdir):
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for name in sorted(os.listdir(CSRC)) + ["../../include/selscan.h"]:
        path = os.path.join(CSRC, name)
        if path.endswith((".hip", ".h")):
            h.update(open(path, "rb").read())
    out_dir = os.path.join(tmpdir, "selscan_host_asan_" + h.hexdigest()[:16])
    lib = os.path.join(out_dir, "libselscan_asan.so")
    if os.path.exists(lib):
        return lib
    os.makedirs(out_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = [subprocess.Popen([HIPCC, *FLAGS, *inc, "-c", "-o", os.path.join(out_dir, s + ".o"), os.path.join(CSRC, s)],
                              stdout=subprocess.PIPE, stderr=subprocess.STDOUT) for s in SRCS]
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out.decode()[-2000:]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", *SAN, "-o", lib + ".tmp",
                    *[os.path.join(out_dir, s + ".o") for s in SRCS]], check=True)
    os.replace(lib + ".tmp", lib)
    return lib


def test_abi_under_host_sanitizers(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc's clang")
    base = os.environ.get("TMPDIR", "/tmp")
    lib = _build(base if os.access(base, os.W_OK) else str(tmp_path_factory.mktemp("asan")))
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the host code is instrumented
    env = dict(os.environ, SELSCAN_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail

"""The host-side validation layer under AddressSanitizer.

Builds libcsa2 once more with the host code instrumented by AddressSanitizer
(the device code is compiled as usual; nothing is launched) and runs the
CPU ABI tests against that build in a child process with the sanitizer
runtime preloaded: every validation path of every entry point then runs with
out-of-bounds, use-after-free and similar host memory errors turned into a
failure."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "sparse_attention_decode_csa2_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_abi_validation_under_host_asan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    sys.path.insert(0, os.path.join(ROOT, "sparse_attention_decode_csa2_amd"))
    from build import SOURCES  # noqa: E402  (the library's own source list)
    lib = str(tmp_path / "libcsa2_asan.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           *[os.path.join(SRC, s) for s in SOURCES], "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the host code is instrumented: it calls into the sanitizer runtime
    syms = subprocess.check_output(["nm", "-D", "--undefined-only", lib], text=True)
    assert "__asan_report_load" in syms or "__asan_init" in syms
    runtime = subprocess.check_output([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, CSA2_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert r.returncode == 0 and "passed" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
    # and the child process loaded the instrumented build, not the in-tree one
    probe = subprocess.run([sys.executable, "-c", "from sparse_attention_decode_csa2_amd import csa2; csa2.load(); "
                            "print(csa2.LIB_PATH)"], capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, (probe.stdout, probe.stderr[-2000:])
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]

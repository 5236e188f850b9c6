"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are compiled with the sanitizers on the host side only
(device code is untouched), linked into tests/abi_sanitize_main.cpp, which
drives every entry point through its host validation (and the size queries
over a sweep of shapes and sizes), and run on the CPU: no kernel is launched.
A memory error or undefined behaviour aborts the driver; a wrong status makes
it exit non-zero."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_compressed_paged_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
# the host compiler behind hipcc, whose sanitizer runtimes match its objects
CLANGXX = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
ROCM_LIB = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
# host-side sanitizers only: each -fsanitize= directly after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


@pytest.mark.slow
def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC) or not os.path.exists(CLANGXX):
        pytest.skip("hipcc or its clang++ not found")
    from rank_compressed_paged_amd import build as b
    objs = []

    def comp(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fPIC", f"-I{INCLUDE}", "-O1", "-g",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", *HOST_SAN, "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(comp, b.SOURCES))
    drv = str(tmp_path / "drv.o")
    r = subprocess.run([CLANGXX, "-std=c++17", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", f"-I{INCLUDE}", "-c",
                        os.path.join(ROOT, "tests", "abi_sanitize_main.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_sanitize")
    r = subprocess.run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, "-o", exe,
                        f"-L{ROCM_LIB}", f"-Wl,-rpath,{ROCM_LIB}", "-lamdhip64"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all statuses as expected" in r.stdout

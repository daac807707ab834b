"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (no device): the
fp64 oracle on small synthetic inputs (tests/sanitize/oracle_driver.c), and
the C-ABI validation layer (moe_api.cpp, with its kernel launchers stubbed
out by tests/sanitize/launch_stubs.cpp) called with refused and accepted
arguments (tests/sanitize/api_driver.cpp).  Any out-of-bounds access, use
after free, leak (oracle) or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]


def _run(exe, leaks):
    env = dict(os.environ, ASAN_OPTIONS=f"detect_leaks={1 if leaks else 0}:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_host_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.run(["gcc", "-std=c99", "-fopenmp", *SAN_FLAGS, os.path.join(ROOT, "oracle", "moe_oracle.c"),
                    os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"], check=True)
    r = _run(exe, leaks=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not available")
def test_validation_layer_under_host_sanitizers(tmp_path):
    flags = ["-x", "c++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-Wno-c++20-extensions", *SAN_FLAGS]
    objs = []
    for src in (os.path.join(ROOT, "bit_dequant_expert_route_amd", "csrc", "moe_api.cpp"),
                os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "api_driver.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([CLANG, *flags, "-c", src, "-o", o], check=True)
        objs.append(o)
    exe = str(tmp_path / "api_asan")
    subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    # (leak checking off: the HIP runtime keeps allocations for the process)
    r = _run(exe, leaks=False)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "api ok" in r.stdout

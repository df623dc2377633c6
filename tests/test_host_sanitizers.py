"""Host-side sanitizer run of the C entry points' argument validation (CPU only).

abi.cpp, which holds every entry point's checks, is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (recovery off: the first report ends the run) and linked with
tests/host/abi_fuzz.cpp against the built library's internal launchers. The driver calls
every entry point with NULL pointers and hostile sizes, runs every size query on extreme
arguments, and checks peagle_cod_counts' writes against exactly sized heap arrays.

A call that passed validation would reach the launchers with NULL device pointers, so the
test runs only where no GPU is visible: there the HIP runtime refuses any launch, and the
driver counts such a call as a failure.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "token_drafting_amd")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_abi_validation_under_address_and_ub_sanitizers(tmp_path):
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is visible: the driver's NULL pointers must never reach a launch")
    gxx = shutil.which("g++")
    lib = os.path.join(PKG, "libpeagle.so")
    if gxx is None:
        pytest.skip("g++ not found")
    if not os.path.exists(lib):
        pytest.skip("libpeagle.so is not built")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    obj = str(tmp_path / "abi_san.o")
    exe = str(tmp_path / "abi_fuzz")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__",
                    f"-I{rocm}/include", f"-I{ROOT}/include", f"-I{PKG}/csrc", "-c",
                    os.path.join(PKG, "csrc", "abi.cpp"), "-o", obj],
                   check=True, capture_output=True, text=True, timeout=300)
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", *SAN, f"-I{ROOT}/include",
                    os.path.join(ROOT, "tests", "host", "abi_fuzz.cpp"), obj, f"-L{PKG}", "-lpeagle",
                    f"-Wl,-rpath,{PKG}", f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib",
                    "-o", exe],
                   check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "2000"], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "refused-wrongly 0 counts ok" in out, out[-4000:]

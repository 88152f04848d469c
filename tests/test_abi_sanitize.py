"""The C ABI layer (vda_api.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host, linked with the kernel objects, and driven through every argument check, overflow guard and
NULL-handle path (tests/native/abi_sanitize.c).  Host code only: the device code is not
instrumented, and no kernel runs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "frame_wise_delta_vda_amd", "csrc")
BUILD = os.path.join(ROOT, "frame_wise_delta_vda_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
KERNEL_OBJECTS = ["stats.hip.o", "scan.hip.o", "readout.hip.o", "bwd.hip.o", "noalloc.hip.o"]


def test_abi_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (python -m frame_wise_delta_vda_amd.build)")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include"),
           "-D__HIP_PLATFORM_AMD__"]
    api_o = str(tmp_path / "vda_api.o")
    drv_o = str(tmp_path / "abi_sanitize.o")
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run([cxx, "-std=c++17", "-O1", *san, *inc, "-c", os.path.join(CSRC, "vda_api.cpp"), "-o", api_o],
                   check=True)
    subprocess.run([shutil.which("gcc") or "gcc", "-std=c11", "-O1", *san, *inc, "-c",
                    os.path.join(ROOT, "tests", "native", "abi_sanitize.c"), "-o", drv_o], check=True)
    subprocess.run([cxx, *san, drv_o, api_o, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lm", "-o", exe], check=True)
    supp = tmp_path / "lsan.supp"
    # allocations the HIP runtime keeps for the life of the process are not this library's
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:librocprofiler\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               LSAN_OPTIONS=f"suppressions={supp}", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failure(s)" in r.stdout

"""CPU test: the host-side plan construction and argument checks of libcgtp
(cgtp_api.hip) built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
pass, linked with the library's other objects, and a driver program
(tests/sanitize/plan_driver.cpp) that creates plans for every workload's irreps and
exercises the parse errors, NULL arguments and refusals.  Nothing touches a device:
plans are host-only and every device entry point is called only with arguments it
refuses before any launch.  The device code is built without sanitizers (GPU
sanitizers are not used here)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "clebsch_gordan_tensor_node_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _objects():
    names = ["kernels_graph.o", "kernels_bwd.o"] + [f"kernels_conv_c{c}.o" for c in range(9)]
    return [os.path.join(BUILD, n) for n in names]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_plan_and_argument_checks_under_asan_ubsan(tmp_path):
    objs = _objects()
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (python -m clebsch_gordan_tensor_node_amd.build)")
    api = str(tmp_path / "cgtp_api_san.o")
    drv = str(tmp_path / "plan_driver.o")
    exe = str(tmp_path / "plan_driver")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    # host pass instrumented, device pass untouched: each sanitizer flag behind -Xarch_host
    cmd = [HIPCC, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address,undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer",
           "-c", os.path.join(CSRC, "cgtp_api.hip"), "-o", api]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([CLANG, "-std=c++17", "-O1", "-g", *san, "-c",
                        os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([CLANG, *san, drv, api, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]

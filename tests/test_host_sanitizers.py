"""The host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_driver.cpp calls every entry point with invalid, zero-size and
(without a GPU) valid arguments.  It is linked with libmha's host code
(mha_api.cpp, sdpa_route.cpp) compiled with the sanitizers on the host side
only, and with the kernel objects of the library build as they are.  A
sanitizer finding aborts the driver; a wrong status makes it exit 1.

CPU only: the driver never launches a kernel, and its no-device checks run
only where no GPU driver is present.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_head_scaled_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
# the library's kernel objects: every .hip source of the build
from transformer_head_scaled_amd.build import SOURCES  # noqa: E402
KERNEL_OBJS = [os.path.splitext(s)[0] + ".o" for s in SOURCES if s.endswith(".hip")]
HIPCC = "/opt/rocm/bin/hipcc"


def _have_inputs():
    return os.path.exists(HIPCC) and all(os.path.exists(os.path.join(BUILD, o)) for o in KERNEL_OBJS)


@pytest.mark.skipif(not _have_inputs(), reason="hipcc or the library's kernel objects are missing")
def test_abi_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    san = []
    for s in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", s]
    cmd = ([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"] + san +
           [os.path.join(CSRC, "mha_api.cpp"), os.path.join(CSRC, "sdpa_route.cpp"),
            os.path.join(ROOT, "tests", "abi_driver.cpp"), "-x", "none"] +
           [os.path.join(BUILD, o) for o in KERNEL_OBJS] + ["-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{' '.join(cmd)}\n{r.stderr[-3000:]}"
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    args = [exe] + ([] if os.path.exists("/dev/kfd") else ["--no-device"])
    run = subprocess.run(args, capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, f"driver failed ({run.returncode}):\n{run.stdout}\n{run.stderr[-4000:]}"
    assert "all checks passed" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr

"""The C boundary's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; no GPU, no HIP runtime).

``csrc/abi.cpp`` is compiled host-only with both sanitizers and linked with host
stand-ins for the kernel launchers (``tests/abi_sanitize/stubs.cpp``) and a driver
(``tests/abi_sanitize/driver.cpp``) that makes every kind of invalid call -- each must
return its documented status before any launcher runs ("Reverse-mode automatic
differentiation" (OneModel docs), section 2: errors are detected before any work) --
and valid calls whose workspace is a host buffer of exactly the size
``ssm_workspace_bytes`` reports, which the stand-ins fill region by region: a workspace
region past the buffer is a sanitizer error, overlapping regions fail the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "backward_mamba_ssd_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "abi_sanitize")
CXX = shutil.which("amdclang++") or "/opt/rocm/bin/amdclang++"

# sanitizers apply to host code only (the objects hold no device code)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-fno-sanitize-recover=all"]
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-I{ROOT}/include",
          f"-I{CSRC}", f"-I{HERE}"]


@pytest.mark.skipif(not os.path.exists(CXX), reason="amdclang++ is not installed")
def test_boundary_validation_under_sanitizers(tmp_path):
    objs = []
    for src, lang in ((os.path.join(CSRC, "abi.cpp"), ["-x", "hip", "--offload-host-only"]),
                      (os.path.join(HERE, "stubs.cpp"), ["-x", "hip", "--offload-host-only"]),
                      (os.path.join(HERE, "driver.cpp"), ["-x", "c++"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        p = subprocess.run([CXX, *lang, *COMMON, *SAN, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    p = subprocess.run([CXX, "-fsanitize=address", "-fsanitize=undefined", *objs, "-o", exe],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(p.stdout)
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-4000:]
    assert p.stdout.startswith("OK: 0 failures")

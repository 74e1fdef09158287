"""The binary16-normal-range shortcut of the SR16 rounding equals the general rule
(CPU only).  ``tests/sr16_check/fast_path.cpp`` compiles the library's own rounding
header for the host and compares the two forms: exhaustively in the 13 discarded
bits and the 13 entropy bits that decide, at the first and last significand of every
binary16 binade of both signs (every carry, including the one into infinity), and
on 50 million random values and entropy words over the whole range.  The rule is the
one of "Nemotron 3 Ultra: replaying a rounded state", section "Stochastic rounding
and the mean state" (up exactly when the entropy residue is below the discarded
remainder); the general form is the one pinned against the oracle."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CXX = shutil.which("amdclang++") or "/opt/rocm/bin/amdclang++"


@pytest.mark.skipif(not os.path.exists(CXX), reason="amdclang++ is not installed")
def test_normal_range_shortcut_equals_the_general_rule(tmp_path):
    exe = str(tmp_path / "sr16_fast_path")
    src = os.path.join(ROOT, "tests", "sr16_check", "fast_path.cpp")
    p = subprocess.run([CXX, "-x", "hip", "--offload-host-only", "-std=c++17", "-O2",
                        f"-I{ROOT}/backward_mamba_ssd_amd/csrc", f"-I{ROOT}/include", src,
                        "-o", exe], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-4000:]
    p = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(p.stdout)
    assert p.returncode == 0, p.stdout[-2000:]
    assert p.stdout.startswith("OK")

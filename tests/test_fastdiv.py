"""The split kernel divides by launch constants (split size, KV heads, items
per plan entry, bins) with FastDiv, a multiply and a shift whose constants the
host builds (pa_common.h). This builds tests/fastdiv_check.cpp against that
header, for the host, and runs it: every divisor up to 4096 against all
numerators below 2^16 and at the multiples of the divisor and the top of the
range, divisors at and around every power of two, and 2e7 random pairs, each
compared with plain integer division."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_fastdiv_matches_integer_division(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.run([HIPCC, "-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-O2",
                    "-std=c++17", f"-I{ROOT}/include", f"-I{ROOT}/paged_kv_cache_52_amd/csrc",
                    os.path.join(ROOT, "tests", "fastdiv_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:]

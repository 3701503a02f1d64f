"""Host build and run of tests/plan_check.hip: the partition arithmetic the
decode and combine kernels use to split the cache blocks (exact integer
results over every size the C ABI admits)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "mla_latent_kv_decode_amd", "csrc")


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_partition_arithmetic_is_exact(tmp_path):
    exe = str(tmp_path / "plan_check")
    subprocess.run(["hipcc", "-O2", "-std=c++17", "--offload-arch=gfx950", "-I", CSRC,
                    os.path.join(HERE, "plan_check.hip"), "-o", exe], check=True,
                   capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 wrong" in r.stdout

"""Host-side checks of the benchmark's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU; asking for more exits with status 2 and says
    why, before anything touches a device."""
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_source_hash_covers_the_decode_sources():
    """The traffic figure is tied to the decode kernel's source and the two
    headers it includes: changing any of them changes the hash."""
    import bench
    h = bench.source_hash("decode_mfma.hip", "mla_common.h", "mla_internal.h")
    assert len(h) == 16
    assert h != bench.source_hash("decode_mfma.hip", "mla_common.h")
    assert h != bench.source_hash("decode_generic.hip", "mla_common.h", "mla_internal.h")

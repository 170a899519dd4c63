"""Host logic of the measurement script (no GPU): the cache-copy rotation
that keeps every timed step reading from HBM, and the refusal of more than
one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

MiB = 1 << 20


def test_rotation_covers_twice_the_last_level_cache():
    # batch-4 index keys (exactly 256 MiB per copy): two copies already fill 2x the cache
    assert bench.rotation(256 * MiB, 2) == 2
    # the HCA cache at batch 4 (8,192 rows x 1 KiB x 4 sequences) needs 16
    assert bench.rotation(4 * 8192 * 1024, 2) == 16
    # fp8 keys + scales at batch 4 (132 B per entry)
    assert bench.rotation(4 * 262144 * 132, 2) == 4
    # never fewer than asked, never more than the cap
    assert bench.rotation(10 * 1024 * MiB, 3) == 3
    assert bench.rotation(1, 2) == 256
    # (the cap of 256 copies leaves per-copy sizes below 2 MiB short of the rule; no workload is that small)
    for b in (2 * MiB, 7 * MiB + 3, 33 * MiB, 129 * MiB, 300 * MiB):
        c = bench.rotation(b, 1)
        assert c * b >= 2 * bench.LLC_BYTES and (c - 1) * b < 2 * bench.LLC_BYTES


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)

"""bench.py's host-side contract (CPU only): more than one GPU is refused
with a message before anything touches a device, and the helpers that size
the cache-defeating buffer rotation and check the counted-traffic hashes
behave as documented."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_buffer_copies_cover_twice_the_last_level_cache():
    import bench
    for nbytes in (12_713_984, 50_356_224, 101_711_872, 251_674_624):
        c = bench.copies_for(nbytes)
        assert c * nbytes >= bench.ROTATE_BYTES > 2 * 256e6
        assert (c - 1) * nbytes < bench.ROTATE_BYTES
    assert bench.copies_for(20_000) == bench.MAX_COPIES      # tiny calls are capped
    assert bench.copies_for(10 << 30) == 1


def test_rotating_cycles_through_the_copies():
    import bench
    seen = []
    f = bench.rotating([lambda i=i: seen.append(i) for i in range(3)])
    for _ in range(7):
        f()
    assert seen == [0, 1, 2, 0, 1, 2, 0]


def test_counted_traffic_is_tied_to_the_source_it_was_taken_on():
    import bench
    for name, t in bench.KERNEL_TRAFFIC.items():
        assert len(t["sha1"]) == 40 and t["bytes"] > 0, name
        assert bench.kernel_traffic(name) in (None, t["bytes"]), name

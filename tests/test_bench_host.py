"""bench.py's host-side logic (CPU only): the algorithmic byte count, the counter-summary lookup that fills
roofline.traffic, and the single-GPU guard."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gemm_bytes_decode_sweep():
    """N*K codes + 4*(N/128)*(K/128) scale bytes + 2*M*K activation bytes + 2*M*N output bytes, at the decode
    sweep's shapes (K = 4096, N = 14336)."""
    want = {1: 58_771_456, 2: 58_808_320, 4: 58_882_048, 8: 59_029_504, 16: 59_324_416}
    for M, b in want.items():
        assert bench.gemm_bytes(M, 4096, 14336) == b


def test_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_source_hash() == h
    assert bench.kernel_source_hash("gemm_tiled.hip") != h


def test_traffic_lookup(tmp_path):
    """The summary's figure is used only when its source hash is the current one."""
    good = tmp_path / "good.md"
    good.write_text(f"source_hash: `{bench.kernel_source_hash()}`\n\nhbm_bytes_per_launch: 123456\n")
    assert bench.traffic_from_profiles(str(good)) == 123456.0
    stale = tmp_path / "stale.md"
    stale.write_text("source_hash: `0000000000000000`\nhbm_bytes_per_launch: 123456\n")
    assert bench.traffic_from_profiles(str(stale)) is None
    assert bench.traffic_from_profiles(str(tmp_path / "missing.md")) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr
    assert r.stdout == ""


def test_step_copies_never_repeat_within_the_cache_window():
    """Each launch of the decode step reads a weight copy that none of the previous n_copies - 1 launches read
    (the steps replay in order c = 0, 1, ..., C - 1, then again), so no launch finds its weights in the
    Infinity Cache."""
    for n_copies in (2, 9, 10, 16):
        n_per_step = 5
        seq = [bench.step_copy(c, j, n_per_step, n_copies) for _ in range(3) for c in range(n_copies)
               for j in range(n_per_step)]
        for i in range(len(seq)):
            window = seq[max(0, i - n_copies + 1):i]
            assert seq[i] not in window, (n_copies, i)

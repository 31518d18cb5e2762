"""bench.py's host-side logic (CPU only): the algorithmic byte count, the counter-summary lookup that fills
roofline.traffic, the single-GPU guard, the trial helpers and the MoE baseline's arguments."""
import os
import subprocess
import sys

import numpy as np

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


def test_median_of_trials_and_cpu_seconds():
    vals = iter([3.0, 1.0, 2.0, 5.0, 4.0])
    m, t = bench.median_of_trials(lambda: next(vals), n=5)
    assert m == 3.0 and t == [3.0, 1.0, 2.0, 5.0, 4.0]
    calls = []
    s, n = bench.cpu_seconds(lambda: calls.append(1), budget_s=10.0, max_runs=3)
    assert n == 3 and len(calls) == 3 and s >= 0.0


def test_moe_cpu_baseline_computes_the_workload(ora):
    """The MoE CPU baseline's compact-expert arguments (only the touched experts quantised, ids
    renumbered) give the oracle's output on the full expert set bit for bit."""
    import inputs
    T, H, E, I, k = 3, 256, 6, 128, 2
    x, logits, w13, w2 = inputs.moe_inputs(5, T, H, E, I)
    host = dict(x=x, logits=logits, k=k, H=H, I=I, E=E, w13=w13, w2=w2)
    compact = ora.moe_decode(*bench.moe_oracle_args(ora, host))
    ids, w = ora.moe_route(logits, k)
    q13, s13 = ora.quant_weight(w13.reshape(-1, H))
    q2, s2 = ora.quant_weight(w2.reshape(-1, I))
    full = ora.moe_decode(x, ids, w, q13.reshape(E, 2 * I, H), s13.reshape(E, 2 * I // 128, H // 128),
                          q2.reshape(E, H, I), s2.reshape(E, H // 128, I // 128))
    assert np.array_equal(compact, full)

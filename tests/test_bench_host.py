"""Host-side logic of bench.py (no GPU): bucket splitting and the --gpus
contract."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("seed", range(5))
def test_bucket_runs_cover_every_chunk_once(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 2049, int(rng.integers(1, 400)))
    for bp in (1, 100, 2048, 5000, 10**6):
        runs = bench.bucket_runs(lens, bp)
        covered = np.concatenate([np.arange(f, f + c) for f, c in runs])
        assert np.array_equal(covered, np.arange(len(lens)))
        sizes = [int(lens[f:f + c].sum()) for f, c in runs]
        assert all(sz >= bp for sz in sizes[:-1])
        # whole chunks, no bucket one chunk longer than needed
        for (f, c), sz in zip(runs[:-1], sizes[:-1]):
            assert int(lens[f:f + c - 1].sum()) < bp


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _write_counter_csv(path, counter, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w") as f:
        f.write(",".join(f'"{c}"' for c in cols) + "\n")
        for i, (name, grid, value) in enumerate(rows):
            f.write(f'{i},{i},{grid},"{name}","{counter}",{value}\n')


def test_ingest_counters_calibrates_against_the_copy(tmp_path, monkeypatch):
    """Counter KiB are scaled by the copy kernel's known bytes; only the step
    kernel's largest-grid dispatches count (the warm-start prefix launches
    have a smaller grid); the record lands under the source hash."""
    from synth import workloads as W
    w = W.get("gpt2")
    lo, hi = w.shard_range(0)
    n = hi - lo
    probe = 1 << 30
    step = "void zs::shard_step_kernel<(zero_dtype)0, 8, false, -1>(zs::StepArgs)"
    copy = "zs::probe_copy_kernel(unsigned int __vector(4) const*)"
    # the copy reads probe bytes as probe/2048 units, writes probe/1024 units
    fetch_kb = (2 * n * 8 + 12 * n) / 2048.0
    write_kb = 14 * n / 1024.0
    _write_counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                       [(step, 4096, 1.0), (step, 999424, fetch_kb), (step, 999424, fetch_kb * 1.01),
                        (copy, 65536, probe / 2048.0), (copy, 65536, probe / 2048.0)])
    _write_counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                       [(step, 4096, 1.0), (step, 999424, write_kb), (step, 999424, write_kb),
                        (copy, 65536, probe / 1024.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    rec = bench.ingest_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), w, 0, "fp32", probe)
    r = rec[f"shard_step_kernel<bf16,8>/{w.name}"]
    assert r["calibration"]["fetch_factor_bytes_per_kb"] == 2048.0
    assert r["calibration"]["write_factor_bytes_per_kb"] == 1024.0
    assert r["algorithmic_read_bytes"] == 28 * n and r["algorithmic_write_bytes"] == 14 * n
    assert r["fetch_over_algorithmic"] == pytest.approx(1.005)
    assert r["write_over_algorithmic"] == pytest.approx(1.0)
    assert r["dispatches"] == [2, 2] and r["grid"] == 999424
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: r["source_hash"])
    assert bench.load_traffic(f"shard_step_kernel<bf16,8>/{w.name}")["bytes_per_launch"] == r["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "another source")
    assert bench.load_traffic(f"shard_step_kernel<bf16,8>/{w.name}") is None


def test_trace_summary_groups_by_kernel_and_grid(tmp_path):
    cols = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp",
            "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Scratch_Size"]
    rows = [("k_a", 64, 64, 0, 1000), ("k_a", 64, 64, 5000, 8000), ("k_a", 128, 64, 0, 500),
            ("k_b", 256, 256, 0, 100)]
    with open(tmp_path / "t.csv", "w") as f:
        f.write(",".join(cols) + "\n")
        for name, g, wg, s, e in rows:
            f.write(f"{name},{g},{wg},{s},{e},8,0,16,0\n")
    lines = bench.trace_summary(str(tmp_path / "t.csv")).splitlines()
    assert lines[2].startswith("| k_a | 64 | 64 | 2 | 2.0 | 2.0 | 1.0 | 3.0 |")
    assert lines[3].startswith("| k_a | 128 | 64 | 1 | 0.5 |")
    assert lines[4].startswith("| k_b | 256 | 256 | 1 | 0.1 |")


@pytest.mark.parametrize("n_ranks,gdt", [(8, "bf16"), (16, "bf16"), (32, "f32")])
def test_bench_byte_model_matches_the_ledger(n_ranks, gdt):
    """The algorithmic bytes bench.py prices each state layout at are the
    oracle ledger's per-element step bytes (2N + 26, 2N + 18, 2N + 16 with
    bf16 partials; 2N + 38 for the three phases run separately)."""
    from oracle import ledger
    gb = 2 if gdt == "bf16" else 4
    want = {"fp32": ledger.shard_step_bytes_per_param(n_ranks, gb, 4),
            "bf16-moments": ledger.shard_step_bytes_per_param(n_ranks, gb, 2),
            "bf16-kahan": ledger.kahan_step_bytes_per_param(n_ranks, gb),
            "unfused": ledger.unfused_step_bytes_per_param(n_ranks, gb)}
    assert set(want) == set(bench.STATES)
    for state, (_, rd, wr, _) in bench.STATES.items():
        assert n_ranks * gb + rd + wr == want[state], state


def test_code_hash_ignores_comments_not_code():
    a = 'int f(int x) { return x + 1; } // one\n/* two */ const char *s = "a // b";\n'
    b = 'int f(int x)\n{\n    return x + 1;   /* changed comment */\n}\nconst char *s = "a // b";\n'
    c = 'int f(int x) { return x + 2; }\nconst char *s = "a // b";\n'
    d = 'int f(int x) { return x + 1; }\nconst char *s = "a / b";\n'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert bench.code_text(a) != bench.code_text(d)


def test_mix_bound():
    """Reads at r, writes at w, one after the other: pure streams give their
    own rate; a 2:1 mix lies between, nearer the read rate."""
    assert bench.mix_bound(100, 0, 6.6, 5.7) == pytest.approx(6.6)
    assert bench.mix_bound(0, 100, 6.6, 5.7) == pytest.approx(5.7)
    b = bench.mix_bound(28, 14, 6600.0, 5700.0)
    assert b == pytest.approx(42 / (28 / 6600 + 14 / 5700))
    assert 5700 < b < 6600


def test_bucket_chunk_len():
    assert bench.bucket_chunk_len(262_144) == 512
    assert bench.bucket_chunk_len(1 << 20) == 1024
    assert bench.bucket_chunk_len(3_000_000) == 2048
    assert bench.bucket_chunk_len(1 << 26) == 2048
    assert bench.bucket_chunk_len(1000) == 512
    for p in (1, 10**5, 10**6, 10**7, 10**9):
        c = bench.bucket_chunk_len(p)
        assert c in (512, 1024, 2048) and c % 64 == 0


def test_headline_is_the_median_allocation(monkeypatch):
    """measure_workload reports the allocation whose roofline fraction is
    the median, with min, median and max of all of them; the JSON record's
    value and ms_per_step are that allocation's."""
    import argparse
    from synth import workloads as W
    w = W.get("gpt2")
    n = w.shard_len
    fr = {0: 0.70, 1: 0.76, 2: 0.73}

    def fake(w_, args, alloc):
        ms = w_.bytes_per_param() * n / (fr[alloc] * bench.HBM_PEAK_GBS * 1e9) * 1e3
        return {"alloc": alloc, "n": n, "chunks": 7, "dst": "tensors", "max_chunk": 2048,
                "bytes_per_param": w_.bytes_per_param(), "launches": 1, "ms_per_step": ms,
                "kernel_ms": ms, "step_ms": [ms] * 3, "bytes_launch": w_.bytes_per_param() * n,
                "extended": None, "next_t": 9, "achieved": fr[alloc] * bench.HBM_PEAK_GBS}

    monkeypatch.setattr(bench, "time_allocation", fake)
    args = argparse.Namespace(allocations=3, scheduled=False, state="fp32", rank=0, graph=False,
                              bucket_params=0, bucket_call="one")
    r = bench.measure_workload(w, args)
    assert r["alloc"] == 2
    fa = r["frac_by_allocation"]
    assert (fa["min"], fa["median"], fa["max"]) == pytest.approx((0.70, 0.73, 0.76))
    assert fa["values"] == pytest.approx([0.70, 0.76, 0.73])
    rec = bench.workload_record(w, args, r)
    assert rec["roofline"]["frac"] == pytest.approx(0.73)
    assert rec["value"] == pytest.approx(n / (r["ms_per_step"] * 1e-3))
    assert rec["config"]["workload"] == "gpt2-small rank-0 shard"


def test_vendor_mix_bounds_use_the_best_rates():
    """The write side of a mix bound is the faster of the write probe and the
    vendor fill; a pure stream at the best rate sits at 1."""
    probes = {"probe_read": {"gbs": 7000.0}, "probe_write": {"gbs": 6500.0}}
    assert bench.best_rates(probes) == (7000.0, 6500.0)
    assert bench.best_rates(probes, {"torch_fill_": {"gbs": 6800.0}}) == (7000.0, 6800.0)
    assert bench.best_rates(probes, {"torch_fill_": {"gbs": 6000.0}}) == (7000.0, 6500.0)


def test_mix_model_and_sum_stream_ratios():
    """The step's mix bound uses its own read and write bytes per launch (the
    7B shard: 28 B read, 14 B written per element); the sum-stream ratios are
    the step's rate over the 8- and 16-array sums of the same run."""
    import types
    w = bench.W.get("llama7b")
    args = types.SimpleNamespace(state="fp32", micro_batches=1)
    n = 1000
    probes = {"probe_read": {"gbs": 7000.0}, "probe_write": {"gbs": 6000.0},
              "probe_copy": {"gbs": 5000.0}}
    sums = {"k1": {"gbs": 6400.0}, "k8": {"gbs": 6250.0}, "k16": {"gbs": 5000.0}}
    rec = {"roofline": {"achieved": 5000.0}}
    bench.add_mix_model(rec, w, args, n, probes, None, sums)
    mm = rec["roofline"]["mix_model"]
    assert (mm["read_bytes"], mm["write_bytes"]) == (28 * n, 14 * n)
    assert mm["bound_gbs"] == pytest.approx(42 / (28 / 7000 + 14 / 6000))
    assert rec["roofline"]["vs_sum_streams"] == pytest.approx({"k8": 0.8, "k16": 1.0})
    rec2 = {"roofline": {"achieved": 5000.0}}
    bench.add_mix_model(rec2, w, args, n, probes)
    assert "vs_sum_streams" not in rec2["roofline"]

"""Host-side parts of bench.py (CPU): the one-GPU guard, the rocprofv3
summary (HBM byte counters scaled by a plain copy of known size, MFMA busy
share) and the source-hash gate on stored traffic figures."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

DKV = "void treeattn::dkv_kernel<__bf16, 128>(treeattn::DkvArgs<__bf16, 128>)"
FWD = "void treeattn::fwd_kernel<__bf16, 128, 12>(treeattn::FwdArgs<__bf16, 128>)"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _ctr(kernel, name, value):
    return {"Kernel_Name": kernel, "Counter_Name": name, "Counter_Value": str(value)}


@pytest.fixture
def tmp_profiles(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    return tmp_path


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_byte_counters_are_scaled_by_the_copy(tmp_profiles):
    # The 1 GiB copy reads as 524288 KiB fetched (half) and 1048576 KiB
    # written (exact), so fetch counts are doubled and writes kept.
    _write_csv(tmp_profiles / "f" / "run_counter_collection.csv", [
        _ctr(COPY, "FETCH_SIZE", 524288), _ctr(DKV, "FETCH_SIZE", 1000),
        _ctr(DKV, "FETCH_SIZE", 3000)])
    _write_csv(tmp_profiles / "w" / "run_counter_collection.csv", [
        _ctr(COPY, "WRITE_SIZE", 1048576), _ctr(DKV, "WRITE_SIZE", 10),
        _ctr(DKV, "WRITE_SIZE", 30)])
    text = bench.summarize([str(tmp_profiles / "f"), str(tmp_profiles / "w")], "the command")
    assert "command: the command" in text
    with open(bench.traffic_file("prompt_heavy")) as f:
        rec = json.load(f)
    assert rec["calibration"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    k = rec["kernels"]["dkv"]
    assert k["read_bytes"] == [1000 * 1024 * 2, 3000 * 1024 * 2]
    assert k["write_bytes"] == [10 * 1024, 30 * 1024]
    # per launch: (reads + writes) / launches
    assert k["hbm_bytes_per_launch"] == round((4000 * 2048 + 40 * 1024) / 2)
    assert k["source_hash"] == bench.kernel_source_hash("dkv")
    assert "fwd" not in rec["kernels"]


def test_mfma_busy_share(tmp_profiles):
    # GRBM_GUI_ACTIVE sums the 8 XCDs' active cycles; with 1024 SIMDs the
    # matrix units could be busy for GRBM/8*1024 SIMD cycles.
    _write_csv(tmp_profiles / "p" / "run_counter_collection.csv", [
        _ctr(FWD, "GRBM_GUI_ACTIVE", 8 * 1000), _ctr(FWD, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 250),
        _ctr(DKV, "GRBM_GUI_ACTIVE", 8 * 400), _ctr(DKV, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 300)])
    text = bench.summarize([str(tmp_profiles / "p")], "c")
    assert "fwd: 0.250" in text
    assert "dkv: 0.750" in text
    assert not os.listdir(bench.PROFILES)


def test_engine_clock(tmp_profiles):
    # 8 XCDs of 2.0e9 cycles each over one second is 2.0 GHz; two dispatches
    # of one kernel are pooled by cycles and time.
    def row(kernel, cycles, t0, t1):
        r = _ctr(kernel, "GRBM_GUI_ACTIVE", cycles)
        r.update(Start_Timestamp=str(t0), End_Timestamp=str(t1))
        return r
    _write_csv(tmp_profiles / "c" / "run_counter_collection.csv", [
        row(DKV, 8 * 2.0e6, 0, 1_000_000), row(DKV, 8 * 1.0e6, 5_000_000, 5_500_000),
        row(COPY, 8 * 2.4e5, 0, 100_000), row(COPY, 8 * 500, 0, 100),
        row("(anonymous namespace)::mfma_loop_random(float*)", 8 * 1.5e6, 0, 1_000_000)])
    text = bench.summarize([str(tmp_profiles / "c")], "c")
    assert "dkv: 2.000 over 2 dispatches, 1.500 ms" in text
    assert "copy: 2.400 over 1 dispatches" in text
    assert "mfma_loop_random: 1.500 over 1 dispatches" in text


def test_wave_state_shares(tmp_profiles):
    _write_csv(tmp_profiles / "s" / "run_counter_collection.csv", [
        _ctr(DKV, "SQ_WAVE_CYCLES", 1000), _ctr(DKV, "SQ_WAIT_ANY", 400),
        _ctr(DKV, "SQ_WAIT_INST_ANY", 250), _ctr(DKV, "SQ_ACTIVE_INST_ANY", 350),
        _ctr(DKV, "SQ_ACTIVE_INST_SCA", 70)])
    text = bench.summarize([str(tmp_profiles / "s")], "c")
    assert "dkv: wait 0.40, wait for issue 0.25, issuing 0.35 (scalar 0.20 of it)" in text


def test_kernel_stats_table(tmp_profiles):
    _write_csv(tmp_profiles / "k" / "run_kernel_stats.csv", [
        {"Name": DKV, "Calls": "4", "AverageNs": "2500000", "TotalDurationNs": "10000000",
         "Percentage": "60.0"},
        {"Name": FWD, "Calls": "2", "AverageNs": "1000000", "TotalDurationNs": "2000000",
         "Percentage": "12.0"}])
    text = bench.summarize([str(tmp_profiles / "k")], "c")
    lines = {l.split()[0]: l for l in text.splitlines() if l[:3] in ("dkv", "fwd")}
    assert lines["dkv"].split()[1:4] == ["4", "2.500", "10.000"]
    assert "(12 waves)" in lines["fwd"]


def test_stored_traffic_needs_the_current_sources_and_workload(tmp_profiles):
    os.makedirs(bench.PROFILES)
    rec = {"kernels": {"dkv": {"hbm_bytes_per_launch": 123,
                               "source_hash": bench.kernel_source_hash("dkv")}},
           "workload": "response_heavy"}

    def store(r, name):
        with open(bench.traffic_file(name), "w") as f:
            json.dump(r, f)

    store(rec, "response_heavy")
    assert bench.stored_traffic("dkv", "response_heavy") == 123
    assert bench.stored_traffic("dkv", "prompt_heavy") is None
    assert bench.stored_traffic("fwd", "response_heavy") is None
    store(rec, "prompt_heavy")  # a record under the wrong name is ignored
    assert bench.stored_traffic("dkv", "prompt_heavy") is None
    rec["kernels"]["dkv"]["source_hash"] = "0" * 16
    store(rec, "response_heavy")
    assert bench.stored_traffic("dkv", "response_heavy") is None


def test_summary_records_the_profiled_workload(tmp_profiles):
    _write_csv(tmp_profiles / "f" / "r_counter_collection.csv", [
        _ctr(COPY, "FETCH_SIZE", 524288), _ctr(DKV, "FETCH_SIZE", 1000)])
    _write_csv(tmp_profiles / "w" / "r_counter_collection.csv", [
        _ctr(COPY, "WRITE_SIZE", 1048576), _ctr(DKV, "WRITE_SIZE", 10)])
    bench.summarize([str(tmp_profiles / "f"), str(tmp_profiles / "w")],
                    "rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --workload long_mixed")
    with open(bench.traffic_file("long_mixed")) as f:
        assert json.load(f)["workload"] == "long_mixed"


def test_per_launch_traffic_report(tmp_profiles):
    """The roofline's per-launch record: the stored counters of each launch of
    one step (two profiled steps, launches in call order), the algorithmic
    bytes and the achieved bandwidth."""
    from shared_prompt_tree_amd import workloads as wl

    os.makedirs(bench.PROFILES)
    rec = {"workload": "prompt_heavy",
           "kernels": {"dkv": {"hbm_bytes_per_launch": 1,
                               "source_hash": bench.kernel_source_hash("dkv"),
                               "read_bytes": [10e9, 100e9, 12e9, 102e9],
                               "write_bytes": [1e9, 2e9, 3e9, 4e9]}}}
    with open(bench.traffic_file("prompt_heavy"), "w") as f:
        json.dump(rec, f)
    st = bench.stored_launch_traffic("dkv", "prompt_heavy")
    assert st == [(11e9, 2e9), (101e9, 3e9)]
    assert bench.stored_launch_traffic("dkv", "response_heavy") is None
    tree = wl.make_tree(wl.SPECS["prompt_heavy"])
    # prefill dK/dV: Q, dO (2 x 32768 x 32 x 128 x 2 B), LSE and D (2 x 32768
    # x 32 x 4 B), K, V in and dK, dV out (4 x 32768 x 8 x 128 x 2 B), float32
    # seeds in (2 x 32768 x 8 x 128 x 4 B)
    want = 2 * 268435456 + 2 * 4194304 + 4 * 67108864 + 2 * 134217728
    assert bench.algorithmic_bytes(tree, "dkv", "prefill_bwd") == want
    launches = bench.launch_report(tree, "dkv", [2.0, 20.0], st)
    assert [x["call"] for x in launches] == ["replay_bwd", "prefill_bwd"]
    pre = launches[1]
    assert pre["hbm_bytes"] == 104e9 and pre["hbm_gbps"] == round(104e9 / 20e-3 / 1e9, 1)
    assert pre["hbm_over_algorithmic"] == round(104e9 / want, 2)
    assert launches[0]["hbm_read_bytes"] == 11e9
    none = bench.launch_report(tree, "dkv", [2.0, 20.0], None)
    assert none[0]["hbm_bytes"] is None and none[0]["algorithmic_bytes"] > 0


def test_causal_tile_visits_closed_form():
    """Key tiles read by the rows of a causal segment: the closed form equals
    the brute-force sum of ceil(k / 256)."""
    for n in (0, 1, 255, 256, 257, 511, 512, 1000, 32768, 32769):
        assert bench.causal_tile_visits(n) == sum(-(-k // 256) for k in range(1, n + 1))


def test_strategy_flops_per_pair():
    """The fused dQ strategy moves the 6d of the dQ pass into the dK/dV
    kernel as 2d: 10d in one kernel, none in the other; forward unchanged."""
    assert bench.flops_per_pair_dim("dkv", True) == 10 and bench.flops_per_pair_dim("dq", True) == 0
    assert bench.flops_per_pair_dim("dkv", False) == 8 and bench.flops_per_pair_dim("dq", False) == 6
    assert bench.flops_per_pair_dim("fwd", True) == bench.flops_per_pair_dim("fwd", False) == 4


def test_assign_grid_largest_first():
    """Largest-first placement (AugTree section 3.4, Eq. 6, the greedy form):
    the classic greedy result on a textbook set (5, 4, 3, 3, 3 on two lanes:
    8 and 10 against the optimum 9 and 9), within Graham's 4/3 - 1/(3m)
    bound of the exhaustive optimum on random sets, conserving the total."""
    import itertools
    import random

    from shared_prompt_tree_amd import workloads as wl

    assert sorted(wl.assign_grid([5, 4, 3, 3, 3], 2)) == [8, 10]
    assert max(wl.assign_grid([7] * 10, 4)) == 21
    rng = random.Random(3)
    for _ in range(40):
        m = rng.randint(2, 3)
        costs = [rng.randint(1, 20) for _ in range(rng.randint(m, 8))]
        loads = wl.assign_grid(costs, m)
        assert abs(sum(loads) - sum(costs)) < 1e-9
        best = min(max(sum(c for c, a in zip(costs, asg) if a == j) for j in range(m))
                   for asg in itertools.product(range(m), repeat=len(costs)))
        assert best <= max(loads) <= (4 / 3 - 1 / (3 * m)) * best + 1e-9


def test_schedule_balance_of_large_replays():
    """On the large workloads the largest-first placement of the replay items
    per XCD is within 2% of perfect balance: a static assignment of the
    items to compute units could not shorten these launches."""
    from shared_prompt_tree_amd import workloads as wl

    for name in ("prompt_heavy", "response_heavy", "long_mixed"):
        tree = wl.make_tree(wl.SPECS[name])
        for kind in ("dq", "dkv"):
            assert 1.0 <= wl.schedule_balance(tree, kind) < 1.02, (name, kind)


def test_mfma_ceiling_library_exports_and_checks_arguments():
    # The measurement library builds with the others and rejects a bad
    # argument on the host, before any HIP call (so this runs without a GPU).
    import ctypes
    path = os.path.join(ROOT, "shared_prompt_tree_amd", "lib", "libmfmaceiling.so")
    assert os.path.exists(path), "build with python -m shared_prompt_tree_amd.build"
    lib = ctypes.CDLL(path)
    f = lib.mfma_ceiling_run
    f.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    tf, first, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    assert f(1, 0.0, ctypes.byref(tf), ctypes.byref(first), ctypes.byref(n)) == -1
    assert f(1, 1.0, None, ctypes.byref(first), ctypes.byref(n)) == -1

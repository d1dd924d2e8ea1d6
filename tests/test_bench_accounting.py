"""bench.py host logic (no GPU): the traffic file from rocprofv3 counter CSVs
and the FLOP accounting."""
import csv
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, counter, rows):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, vals) in enumerate(rows):
            for v in vals:  # one line per XCD-level instance: summed per dispatch
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_write_traffic_scales_by_the_copy(tmp_path):
    bench = _bench()
    part = "_ZN2sk12_GLOBAL__N_119partial_bf16_kernelIDF16bLi192ELi128EEEvNS_11PartialArgsE"
    merge = "void sk::merge_pieces_kernel<128, 128>(sk::PartialArgs)"
    comb = "_ZN2sk14combine_kernelIDF16bLi4ELb1EEEvNS_11CombineArgsE"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    # two split launches of the partial kernel, each followed by its piece
    # merge (partial mean 300 KiB, merge 10), a larger combine that must not
    # count, an unsplit launch (no merge after it) that must not count, and
    # the copy read as half its size
    _write(fetch, "FETCH_SIZE", [(part, [100.0, 150.0]), (merge, [10.0]), (part, [200.0, 150.0]), (merge, [10.0]),
                                 (comb, [5e5]), (part, [9e5]), (comb, [5e5]), (copy, [262144.0, 262144.0])])
    _write(write, "WRITE_SIZE", [(part, [40.0]), (merge, [4.0]), (part, [60.0]), (merge, [4.0]), (comb, [7e5]),
                                 (part, [9e5]), (comb, [7e5]), (copy, [1048576.0]), ("zero_fill", [1048576.0])])
    out = bench.write_traffic(fetch, write, path=str(tmp_path / "t.json"))
    assert out["fetch_size_kib_per_dispatch"] == {"partial_bf16_kernel": 300.0, "merge_pieces_kernel": 10.0}
    assert out["write_size_kib_per_dispatch"] == {"partial_bf16_kernel": 50.0, "merge_pieces_kernel": 4.0}
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    assert out["hbm_bytes_per_launch"] == (310 * 2 + 54) * 1024
    assert out["kernel_source_sha256"] == bench.kernel_source_hash()
    with open(tmp_path / "t.json") as f:
        assert json.load(f) == out


def test_write_traffic_needs_every_kernel(tmp_path):
    import pytest

    bench = _bench()
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    _write(fetch, "FETCH_SIZE", [("partial_bf16_kernel", [1.0]), ("copy", [2.0])])
    _write(write, "WRITE_SIZE", [("partial_bf16_kernel", [1.0]), ("copy", [2.0])])
    with pytest.raises(SystemExit):
        bench.write_traffic(fetch, write, path=str(tmp_path / "t.json"))


def test_visible_pairs_match_the_oracle():
    """bench.py's FLOP accounting counts the pairs the oracle's visibility
    rule leaves visible, on every workload of the parity suite."""
    import sys

    sys.path.insert(0, ROOT)
    from oracle import adapter
    from oracle import splitkv as oracle
    from split_kv_attention_amd import workloads

    bench = _bench()
    for w in workloads.CONFIGS:
        expect = sum(oracle.visible_pairs(s) for s in adapter.seq_specs(w))
        assert bench.visible_pairs(w) == expect, w.name


def test_more_than_one_gpu_is_refused():
    """bench.py runs on one GPU; --gpus N > 1 exits with a message before
    touching a device."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_runs_every_unit_on_a_pool():
    """The pooled oracle baseline covers every (sequence, head, 32-row) unit
    of a small packed workload and reports its pool and host."""
    import dataclasses
    import sys

    sys.path.insert(0, ROOT)
    from split_kv_attention_amd import workloads

    bench = _bench()
    w = dataclasses.replace(workloads.LONG_PREFILL, name="small", heads=2, sq=(70,), sk=(300,))
    inputs = workloads.make_inputs(w, "cpu", seed=1)
    r = bench.cpu_baseline(w, inputs, 128, budget_s=120.0, max_workers=2)
    assert r["units_total"] == 2 * 3 and r["units_done"] == r["units_total"]
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert r["cores"] == min(len(os.sched_getaffinity(0)), 2)
    for key in ("cpu_model", "numpy", "blas", "affinity_cpus", "sample"):
        assert r[key], key


def test_cpu_baseline_samples_whole_sequences_of_a_large_dense_batch():
    """Past the host-memory cap the baseline keeps whole sequences (seeded)
    and reports the sample against the whole workload's units."""
    import dataclasses
    import sys

    sys.path.insert(0, ROOT)
    from split_kv_attention_amd import workloads

    bench = _bench()
    w = dataclasses.replace(workloads.DECODE_BF16, name="small_decode", heads=2, sq=(1,) * 6, sk=(200,) * 6)
    inputs = workloads.make_inputs(w, "cpu", seed=2)
    one_seq = w.heads * 200 * (w.d_qk + w.d_v) * 2
    r = bench.cpu_baseline(w, inputs, 128, budget_s=120.0, max_workers=2, max_host_bytes=2.5 * one_seq)
    assert r["units_total"] == 6 * 2
    assert r["units_done"] == 2 * 2  # two whole sequences fit under the cap
    assert "2 of 6 sequences" in r["sample"]

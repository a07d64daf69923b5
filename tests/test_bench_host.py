"""Host logic of bench.py (no GPU): the one-GPU refusal, counter ingestion and the
algorithmic byte counts the roofline fields use."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synthetic import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes():
    w = WORKLOADS["long_16k_causal"]
    # Q, K, V read and O written in bf16, LSE in fp32: 8*B*H*N*d + 4*B*H*N
    assert bench.algorithmic_bytes(w) == 8 * 16 * 16384 * 128 + 4 * 16 * 16384 == 269484032
    # grouped-query: K and V have H_kv heads
    assert bench.algorithmic_bytes(w, kv_heads=4) == 4 * (16 + 4) * 16384 * 128 + 4 * 16 * 16384
    vl = WORKLOADS["varlen16_causal"]
    assert bench.algorithmic_bytes(vl, lengths=[10, 20]) == 8 * 16 * 30 * 128 + 4 * 16 * 30
    # backward: read Q, K, V, O, dO and LSE, write dQ, dK, dV, D written and read once
    rows = 16 * 16384
    assert bench.bwd_algorithmic_bytes(w) == 2 * 128 * (4 * rows + 4 * rows) + 12 * rows
    # varlen backward: the same per token, over all tokens of all sequences
    vrows = 16 * 30
    assert bench.bwd_algorithmic_bytes(vl, lengths=[10, 20]) == 2 * 128 * (4 * vrows + 4 * vrows) + 12 * vrows


def _write_counters(path, counter, attn_kib, copy_kib):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for v in attn_kib:
            wr.writerow({"Kernel_Name": "void fa2_fwd_kernel<128, 64, true, false, 2, 4, 8>(Params)",
                         "Counter_Name": counter, "Counter_Value": v})
        wr.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter, "Counter_Value": copy_kib})
        wr.writerow({"Kernel_Name": "small_kernel", "Counter_Name": counter, "Counter_Value": 1.0})


def test_ingest_counters_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # The copy moves 1 GiB: FETCH_SIZE reads half of it in KiB (factor 2), WRITE_SIZE all.
    _write_counters(fetch, "FETCH_SIZE", [100.0, 300.0, 200.0], bench.COPY_BYTES / 1024 / 2)
    _write_counters(write, "WRITE_SIZE", [50.0, 50.0, 70.0], bench.COPY_BYTES / 1024)
    bench.ingest_counters(str(fetch), str(write), steps=3)
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["kernel_source_sha256"] == bench.kernel_source_hash()
    assert t["fetch_copy_factor"] == pytest.approx(2.0) and t["write_copy_factor"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2)     # median x factor
    assert t["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0000")
    assert bench.load_traffic() is None                                        # stale after a change


def test_stored_traffic_matches_the_current_kernel_or_is_ignored():
    t = bench.load_traffic()
    if t is not None:
        assert t["fetch_bytes_per_launch"] > 0 and t["write_bytes_per_launch"] > 0


def test_default_warmup_covers_about_half_a_second():
    assert bench.default_warmup(1e-3) == 5 + 500                     # 1 ms steps: ~0.5 s
    assert bench.default_warmup(0.17e-3) * 0.17e-3 >= bench.WARMUP_SECONDS
    assert bench.default_warmup(2.0) == 10                           # long steps: at least 10
    assert bench.default_warmup(0.0) == 5 + 20000                    # bounded for empty steps


def test_parse_amdsmi_metric():
    def gfx(v):
        return {"clk": {"value": v, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"}}
    doc = {"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 1330, "unit": "W"}},
                         "clock": {"gfx_0": gfx(1800), "gfx_1": gfx(2000), "mem_0": gfx(2000),
                                   "gfx_2": {"clk": "N/A"}}}]}
    clocks, power = bench.parse_amdsmi_metric(json.dumps(doc))
    assert clocks == [1800.0, 2000.0] and power == 1330.0           # memory clock and N/A skipped
    # a bare list of GPUs, no power reading
    clocks, power = bench.parse_amdsmi_metric(json.dumps([{"clock": {"gfx_0": gfx(2100)}}]))
    assert clocks == [2100.0] and power is None
    assert bench.parse_amdsmi_metric("not json") == (None, None)
    assert bench.parse_amdsmi_metric(json.dumps({"gpu_data": []})) == (None, None)


def test_bwd_and_fwd_bwd_are_exclusive():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--bwd", "--fwd-bwd"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "exclusive" in r.stderr


def test_host_cpu_info_fields():
    info = bench.host_cpu_info()
    assert info["logical_cpus"] == os.cpu_count()
    assert 1 <= info["affinity_cpus"] <= info["logical_cpus"]
    if "physical_cores" in info:
        assert 1 <= info["physical_cores"] <= info["logical_cpus"]


def test_stored_traffic_matches_the_current_kernel_source():
    """The committed HBM-traffic profile is keyed to the kernel source it was measured on; the
    bench line reports it only while that source is unchanged."""
    t = bench.load_traffic()
    if t is None:
        pytest.skip("profiles/fa2_fwd_long16k_traffic.json was measured on another kernel source "
                    "(the bench line then reports traffic: null)")
    total = t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    assert total >= bench.algorithmic_bytes(WORKLOADS["long_16k_causal"])

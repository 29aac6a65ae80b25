"""Host-side parts of bench.py: the one-GPU guard and the traffic arithmetic
(no GPU is touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                           capture_output=True, text=True, timeout=120,
                           env={**os.environ, **env})
        assert r.returncode == 2, r
        assert "more than one GPU" in r.stderr
        assert r.stdout == ""


def test_traffic_bytes_scale_fetch_and_write():
    # FETCH_SIZE counts half the loaded bytes (scaled by 2), WRITE_SIZE all of them
    assert bench.FETCH_SCALE == 2.0 and bench.WRITE_SCALE == 1.0
    for wl, kernels in bench.TRAFFIC_KIB.items():
        for k, t in kernels.items():
            if t is None:  # the kernel changed since its counters were taken
                assert bench.traffic_bytes(wl, k) is None
                continue
            f, w = t
            assert bench.traffic_bytes(wl, k) == round((2 * f + w) * 1024)
    # the reduce moves its algorithmic bytes, W + 1 slices of R x N fp32, up to
    # the counters' noise
    assert abs(bench.traffic_bytes("rs_long", "reduce") - 9 * 16384 * 5120 * 4) < 1e-4 * 9 * 16384 * 5120 * 4
    assert abs(bench.traffic_bytes("rs", "reduce") - 5 * 1024 * 4096 * 4) < 5e-3 * 5 * 1024 * 4096 * 4


def test_workload_ids_name_the_configs():
    import seeded_inputs as si
    want = {"ag": "ag_qwen3_32b_ffn_up_w8_8192x3200x5120", "rs": "rs_w4_4096x4096x2048",
            "ar": "rs_w4_4096x4096x2048", "rs_long": "rs_ffn_down_128k_w8_131072x5120x3200",
            "moe": "ag_moe_w8_t4096_e64_top8_h2048_n768"}
    assert {k: si.WORKLOADS[v].name for k, v in bench.WORKLOAD_ID.items() if v is not None} == want
    # the one workload that is no config: the memory counters' calibration
    assert [k for k, v in bench.WORKLOAD_ID.items() if v is None] == ["fetch_calibration"]


def test_device_timeout_voids_the_values():
    """A fused step whose flag wait timed out on the device skipped units: its
    throughput is not reported, for the headline or for another landing."""
    from tile_level_communication_amd import tlc
    line = {"value": 900.0, "device_status": [tlc.ERR_TIMEOUT, 190, 3, 0]}
    bench.void_on_device_error(line, tlc)
    assert line["value"] is None and "timeout" in line["error"]
    ok = {"value": 900.0, "device_status": [0, 0, 0, 0]}
    bench.void_on_device_error(ok, tlc)
    assert ok == {"value": 900.0, "device_status": [0, 0, 0, 0]}
    others = bench.other_landings(1e12, 1e-3, {tlc.LAND_CU: (2e-3, [tlc.ERR_TIMEOUT, 1, 2, 0]),
                                               tlc.LAND_COLOCATED: (1e-3, [0, 0, 0, 0])},
                                  {tlc.LAND_CU: 1e-3, tlc.LAND_COLOCATED: 0.5e-3})
    assert others["cu"]["value"] is None
    # a failed leg gives none of its derived figures, and names its status
    for k in ("ms_per_step", "overlap_efficiency", "pct_peak"):
        assert others["cu"][k] is None
    assert "device status" in others["cu"]["error"]
    assert others["colocated"]["value"] == 1000.0 and others["colocated"]["overlap_efficiency"] == 1.0
    assert others["colocated"]["pct_peak"] == 40.0 and "error" not in others["colocated"]
    # the headline fields of a failed line go too
    line = {"value": 900.0, "pct_peak": 36.0, "overlap_efficiency": 0.8, "exposed_copy_ms": 0.05,
            "device_status": [tlc.ERR_TIMEOUT, 1, 2, 0]}
    bench.void_on_device_error(line, tlc)
    assert all(line[k] is None for k in ("value", "pct_peak", "overlap_efficiency", "exposed_copy_ms"))


def test_order_and_legs_options():
    a = bench.parse(["--order", "natural", "--rank", "3", "--legs", "headline", "--no-rs"])
    assert bench.ORDERS[a.order] == 0 and a.rank == 3 and a.legs == "headline" and a.no_rs
    a = bench.parse([])
    assert a.order == "rank_offset" and a.legs == "all" and not a.no_rs and a.land == "memcpy"


def test_cpu_baseline_moe_reports_the_oracle_sample():
    import seeded_inputs as si
    r = bench.cpu_baseline("moe", si.workload_inputs(4), 0.05, 0, si.WORKLOADS[4].topk)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] >= 1
    assert "top-8 of 64" in r["sample"] and "H=2048, N=768" in r["sample"]
    # the host it ran on, and the same oracle on one thread
    assert r["nproc"] == os.cpu_count() and r["cpu_model"]
    assert r["one_thread"]["cores"] == 1 and r["one_thread"]["value"] > 0


def test_schedule_option_maps_to_the_library():
    from tile_level_communication_amd import tlc
    for name, want in (("static", tlc.SCHED_STATIC), ("dynamic", tlc.SCHED_DYNAMIC),
                       ("streamk", tlc.SCHED_STREAMK)):
        a = bench.parse(["--schedule", name])
        assert bench.SCHEDULES[a.schedule] == want


def test_moe_hbm_view_arithmetic():
    """The grouped GEMM's memory-side figures: algorithmic bytes of X, W and Y per
    second of the launch, and the calibrated counter traffic per second."""
    import types
    prob = types.SimpleNamespace(T=4096, H=2048, E=64, N=768, k=8)
    args = bench.parse(["--workload", "moe"])
    v = bench.moe_hbm_view(100e-6, prob, args)
    alg = 4096 * 2048 * 2 + 64 * 2048 * 768 * 2 + 4096 * 8 * 768 * 4
    assert v["algorithmic_bytes"] == alg and v["bound"] == "hbm" and v["peak"] == 8000.0
    assert abs(v["achieved"] - alg / 100e-6 / 1e9) < 0.1
    assert abs(v["traffic_gbs"] - bench.traffic_bytes("moe", "gemm") / 100e-6 / 1e9) < 0.1

"""Host-side logic of bench.py that needs no GPU: the single-GPU refusal, the
algorithmic work each roofline figure divides by, and the scaling of the
rocprofv3 byte counters by the device-copy calibration.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert p.stdout == ""  # no JSON line
    assert "one GPU" in p.stderr


def test_a_launch_with_world_size_above_one_is_refused(monkeypatch, capsys):
    monkeypatch.setenv("WORLD_SIZE", "2")
    assert bench.main(["--gpus", "1"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("fmt", ["int4", "int4_asym", "int5"])
def test_expert_weight_bytes_equal_the_generated_arrays(fmt):
    """The byte figures of the decode rooflines are the sizes of the arrays the
    kernels read: packed codes, scales and zero points or fifth bits."""
    cfg = synth.config("tiny", E=2, fmt=fmt)
    w = synth.make_inputs(cfg).weights
    per_matrix = {name: sum(a[0].nbytes for key, a in w.items() if key.split("_")[0] == name)
                  for name in ("gate", "up", "down")}
    assert bench.expert_weight_bytes(cfg, 1) == per_matrix["down"]
    assert bench.expert_weight_bytes(cfg, 2) == per_matrix["gate"] + per_matrix["up"]
    assert bench.expert_weight_bytes(cfg) == sum(per_matrix.values()) == synth.weight_bytes_per_expert(cfg)


def test_gemm_flops_add_up_to_the_layer():
    cfg = synth.config("prefill6144")
    pairs = cfg.T * cfg.k
    gu, unit_gu, bound_gu = bench.kernel_work("gemm_gateup", cfg, pairs, cfg.E)
    dn, unit_dn, bound_dn = bench.kernel_work("gemm_down", cfg, pairs, cfg.E)
    assert (unit_gu, bound_gu, unit_dn, bound_dn) == ("flop", "mfma", "flop", "mfma")
    assert gu == 2 * dn  # two matrices of the same shape against one
    assert gu + dn == bench.layer_work(cfg, cfg.E)[0]
    # 2 flops per multiply-add, three H x I products per pair
    assert gu + dn == 2 * 3 * pairs * cfg.H * cfg.I


def test_decode_bytes_cover_weights_of_the_selected_experts_only():
    cfg = synth.config("decode")
    one = bench.kernel_work("decode_route_gateup", cfg, cfg.T * cfg.k, 1)[0]
    ten = bench.kernel_work("decode_route_gateup", cfg, cfg.T * cfg.k, 10)[0]
    assert ten - one == 9 * bench.expert_weight_bytes(cfg, 2)
    assert bench.kernel_work("not_a_kernel", cfg, 1, 1) == (None, None, None)


def test_roofline_of_divides_work_by_the_launch_duration(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    cfg = synth.config("prefill6144")
    pairs = cfg.T * cfg.k
    r = bench.roofline_of("gemm_gateup", 100.0, cfg, pairs, cfg.E, "prefill6144")
    flops = 4.0 * pairs * cfg.H * cfg.I
    assert r["achieved"] == pytest.approx(flops / 100e-6 / 1e12, abs=0.01)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.PEAK_MFMA_TFLOPS, abs=1e-4)
    assert (r["bound"], r["unit"], r["traffic"]) == ("mfma", "TFLOP/s", None)
    d = synth.config("decode")
    r = bench.roofline_of("gemv_down", 10.0, d, d.T * d.k, 20, "decode")
    assert r["unit"] == "GB/s" and r["bound"] == "hbm"
    assert r["achieved"] == pytest.approx(r["work_per_launch"] / 10e-6 / 1e9, abs=0.01)
    assert bench.roofline_of("permute_hist", 5.0, cfg, pairs, cfg.E, "prefill6144") is None


def _write_pmc(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_record_traffic_scales_counters_by_the_copy_calibration(tmp_path):
    gib_kib = float(1 << 20)
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # The fetch counter reads half of the copy's true bytes, the write counter all of them.
    _write_pmc(fetch, "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", gib_kib / 2), ("__amd_rocclr_copyBuffer", 10.0),
        ("void strata::moe_gemm_wide<0, 2, 0>(strata::GemmArgs)", 1000.0),
        ("void strata::moe_gemm_wide<0, 2, 0>(strata::GemmArgs)", 3000.0),
        ("void strata::moe_gemm_wide<1, 2, 0>(strata::GemmArgs)", 500.0),
        ("strata::seg_hist_kernel(int const*, int, int, int*)", 7.0)])
    _write_pmc(write, "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", gib_kib),
        ("void strata::moe_gemm_wide<0, 2, 0>(strata::GemmArgs)", 100.0),
        ("void strata::moe_gemm_wide<0, 2, 0>(strata::GemmArgs)", 300.0),
        ("void strata::moe_gemm_wide<1, 2, 0>(strata::GemmArgs)", 50.0)])
    rec = bench.record_traffic(str(fetch), str(write), prefill_workload="prefill6144")
    assert rec["_calibration"]["fetch_scale"] == 2.0 and rec["_calibration"]["write_scale"] == 1.0
    gu = rec["gemm_gateup@prefill6144"]
    assert gu["fetch_bytes"] == 2000 * 1024 * 2 and gu["write_bytes"] == 200 * 1024
    assert gu["bytes_per_launch"] == gu["fetch_bytes"] + gu["write_bytes"]
    assert gu["dispatches"] == 2 and gu["source_sha"] == bench.source_sha("gemm_gateup")
    assert gu["layout"] == "tiled"
    assert bench.record_traffic(str(fetch), str(write), "prefill6144", layout="rows")["gemm_down@prefill6144"][
        "layout"] == "rows"
    dn = rec["gemm_down@prefill6144"]
    assert dn["bytes_per_launch"] == 500 * 1024 * 2 + 50 * 1024
    # kernels with no counter rows get no record
    assert not any(key.startswith(("gemv_", "decode_")) for key in rec)


def test_counted_traffic_is_dropped_once_the_kernel_source_changes(monkeypatch, tmp_path):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.counted_traffic("gemm_down", "prefill6144") is None  # no file
    rec = {"gemm_down@prefill6144": {"bytes_per_launch": 123, "source_sha": bench.source_sha("gemm_down"),
                                     "layout": "tiled"},
           "gemm_gateup@prefill6144": {"bytes_per_launch": 456, "source_sha": "0" * 16, "layout": "tiled"}}
    path.write_text(json.dumps(rec))
    assert bench.counted_traffic("gemm_down", "prefill6144") == 123
    assert bench.counted_traffic("gemm_gateup", "prefill6144") is None  # stale source
    assert bench.counted_traffic("gemm_down", "prefill512") is None  # other workload
    assert bench.counted_traffic("gemm_down", "prefill6144", "rows") is None  # counted with the other layout


def test_committed_traffic_records_are_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        data = json.load(f)
    cal = data.pop("_calibration")
    assert cal["copy_bytes"] == 1 << 30
    kernels = {k for k, _ in bench.COUNTED_KERNELS.values()}
    for key, r in data.items():
        kernel, workload = key.split("@")
        assert kernel in kernels and workload in synth.CONFIGS
        # each of the three figures is rounded on its own
        assert abs(r["bytes_per_launch"] - (r["fetch_bytes"] + r["write_bytes"])) <= 1
        assert r["fetch_bytes"] > 0 and r["write_bytes"] > 0
        assert len(r["source_sha"]) == 16
        assert r["layout"] in ("tiled", "rows")

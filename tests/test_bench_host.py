"""Host-side logic of bench.py (no GPU): the one-GPU contract, the conversion of the
HBM byte counters into bytes per launch, and the guard that drops stored byte counts once a
kernel's sources change."""
import csv
import importlib.util
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    """--gpus above 1 exits (status 2) with a message, before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scaled_by_the_calibration_copy(tmp_path):
    """Each counter is scaled so that the 256 MiB calibration copy reads as 256 MiB: a copy
    whose FETCH_SIZE reads 131072 KiB gives the factor 2, one whose WRITE_SIZE reads 262144
    KiB the factor 1.  A kernel's bytes are the mean over its dispatches times that factor,
    and reads plus writes make its total."""
    b = _bench()
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write_counters(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 131072.0),
                                          ("__amd_rocclr_copyBuffer", 8.0),  # small copy: ignored
                                          ("gen_attn_bf16_kernel", 30000.0),
                                          ("gen_attn_bf16_kernel", 40000.0),
                                          ("euler_vec4_kernel", 1000.0)])
    _write_counters(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 262144.0),
                                          ("gen_attn_bf16_kernel", 16000.0),
                                          ("euler_vec4_kernel", 500.0)])
    out_json = str(tmp_path / "traffic.json")
    a = types.SimpleNamespace(calib_mib=256, workload="large", derive_traffic=(fetch, write),
                              traffic_json=out_json)
    b.derive_traffic(a)
    t = json.load(open(out_json))
    assert t["FETCH_SIZE_scale"] == pytest.approx(2.0)
    assert t["WRITE_SIZE_scale"] == pytest.approx(1.0)
    att = t["gen_attn_bf16_kernel"]
    assert att["FETCH_SIZE"] == pytest.approx(35000.0 * 1024 * 2.0)
    assert att["WRITE_SIZE"] == pytest.approx(16000.0 * 1024)
    assert att["bytes"] == pytest.approx(35000.0 * 1024 * 2.0 + 16000.0 * 1024)
    assert t["fm_euler_step"]["bytes"] == pytest.approx(1000.0 * 2048 + 500.0 * 1024)
    assert "qknorm_rope3" not in t  # no dispatch of it in the counters


def test_missing_calibration_copy_is_an_error(tmp_path):
    b = _bench()
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write_counters(fetch, "FETCH_SIZE", [("gen_attn_bf16_kernel", 30000.0)])
    _write_counters(write, "WRITE_SIZE", [("gen_attn_bf16_kernel", 16000.0)])
    a = types.SimpleNamespace(calib_mib=256, workload="large", derive_traffic=(fetch, write),
                              traffic_json=str(tmp_path / "t.json"))
    with pytest.raises(SystemExit, match="calibration copy"):
        b.derive_traffic(a)


def test_stored_bytes_follow_the_sources(tmp_path):
    """A stored figure is reported only for the same workload and while the kernel's source
    and the library headers hash to what they were when the counters were taken."""
    b = _bench()
    key = "gen_attn_bf16_kernel"
    path = str(tmp_path / "traffic.json")
    good = {"workload": "large", key: {"bytes": 123.0, "source_sha256": b._kernel_source_hash(key)}}
    with open(path, "w") as f:
        json.dump(good, f)
    a = types.SimpleNamespace(traffic_json=path, workload="large")
    assert b.measured_bytes(a, key) == 123.0
    assert b.measured_bytes(types.SimpleNamespace(traffic_json=path, workload="mid"), key) is None
    stale = dict(good)
    stale[key] = {"bytes": 123.0, "source_sha256": "0" * 64}
    with open(path, "w") as f:
        json.dump(stale, f)
    assert b.measured_bytes(a, key) is None
    assert b.measured_bytes(types.SimpleNamespace(traffic_json=str(tmp_path / "none.json"),
                                                  workload="large"), key) is None


def test_source_hash_covers_the_headers(tmp_path, monkeypatch):
    """Editing a shared header changes every kernel's source hash."""
    b = _bench()
    fake = tmp_path / "repo"
    csrc = fake / "pixel_space_flow_amd" / "csrc"
    csrc.mkdir(parents=True)
    (fake / "include").mkdir()
    for name in set(b.KERNEL_SOURCES.values()):
        (csrc / name).write_text("// " + name)
    (csrc / "gemm_tile.h").write_text("// tile core")
    (fake / "include" / "neo.h").write_text("// abi")
    monkeypatch.setattr(b, "ROOT", str(fake))
    before = {k: b._kernel_source_hash(k) for k in b.KERNEL_SOURCES}
    (csrc / "gemm_tile.h").write_text("// tile core, edited")
    after = {k: b._kernel_source_hash(k) for k in b.KERNEL_SOURCES}
    assert all(before[k] != after[k] for k in before)


def test_algorithmic_work_of_the_benchmark_workload():
    """The per-launch work the roofline figures divide by, against their closed forms at
    4096 image tokens, a 512-token prefix, 32/8 heads and 3 x 2048^2 pixels:
    4 * 32 * 128 * 4096 * 4608 flops; 4096 tokens * (40 rows * 128 * 2 B read and written +
    12 B of positions); 12 B per pixel."""
    import workloads as W
    b = _bench()
    w = W.make("large", pixels=False)
    flops, pro, euler, attn = b.algorithmic(w)
    assert flops == 4 * 32 * 128 * 4096 * 4608 == pytest.approx(309.24e9, rel=1e-4)
    assert pro == 4096 * (40 * 128 * 2 * 2 + 12) == pytest.approx(83.94e6, rel=1e-4)
    assert euler == 3 * 2048 * 2048 * 12 == pytest.approx(150.99e6, rel=1e-4)
    assert attn == (4096 * (32 + 8) * 2 + 512 * 8 * 2) * 128 * 2 == pytest.approx(85.98e6, rel=1e-4)


def test_per_call_summary():
    """Median, mean, minimum and 90th percentile of per-call durations, ms in, us out."""
    bench = _bench()
    st = bench.stats_us([0.3, 0.1, 0.2, 0.4, 1.0])
    assert st["median"] == pytest.approx(300.0)
    assert st["mean"] == pytest.approx(400.0)
    assert st["min"] == pytest.approx(100.0)
    assert st["calls"] == 5
    assert 400.0 <= st["p90"] <= 1000.0


def test_path_figures_from_durations():
    """Rates of the step path from per-kernel durations: attention TFLOP/s and its share of
    the 2.5 PFLOP/s peak, the bandwidth-bound kernels' GB/s, tokens/s of the step."""
    bench = _bench()
    import workloads as W
    w = W.make("large", pixels=False)
    w.pixel_shape = (1, 3, 2048, 2048)
    flops, pro_bytes, euler_bytes, _ = bench.algorithmic(w)
    k = {"gen_attn": {"median": 250.0}, "qknorm_rope3": {"median": 20.0},
         "fm_euler_step": {"median": 30.0}}
    f = bench.path_figures(w, k, "median")
    assert f["attention_tflops"] == pytest.approx(flops / 250e-6 / 1e12)
    assert f["attention_frac"] == pytest.approx(flops / 250e-6 / 2.5e15)
    assert f["prologue_gbs"] == pytest.approx(pro_bytes / 20e-6 / 1e9)
    assert f["image_tokens_per_s"] == pytest.approx(4096 / 300e-6)
    assert 0.0 < f["step_frac"] < 1.0


def test_cpu_baseline_protocol():
    """The oracle's timing leg on the small workload: all-core and one-thread figures,
    median of three runs, the attention time scaled from the sampled query tokens."""
    bench = _bench()
    import oracle
    import workloads as W
    from tests import harness as H
    w = W.make("small")
    kp, vp = H.frozen_prefix(w)
    c = bench.cpu_baseline(w, kp, vp, 8, 2)
    assert c["kind"] == "oracle" and c["unit"] == "image-tokens/s"
    assert c["cores"] == (os.cpu_count() or 1) and c["one_thread"]["cores"] == 1
    s = c["seconds"]
    assert s["step"] == pytest.approx(s["prologue"] + s["attention_scaled"] + s["euler"])
    assert c["value"] == pytest.approx(w.Tq / s["step"])
    assert "8 of 256" in c["sample"]
    assert oracle.num_threads() == (os.cpu_count() or 1)

"""Host logic of the rocprofv3 summaries (CPU): the copy-calibrated HBM traffic figure and its
per-launch context fit, on synthetic counter CSVs whose answer is known."""
import csv
import json

from memory_bound_autoregressive_amd import profiling


def _write(path, rows, fields):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_scales_by_the_copy_and_fits_context(tmp_path):
    kib = 1024.0
    copy_bytes = 1 << 28
    # the copy's FETCH_SIZE reads half the true bytes (scale 2), WRITE_SIZE reads them right
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(tmp_path / "cf.csv", [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
                                  "Counter_Value": copy_bytes / 2 / kib}], fields)
    _write(tmp_path / "cw.csv", [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
                                  "Counter_Value": copy_bytes / kib}], fields)
    a, b, wr = 3.8e9, 131072.0, 4096.0  # true bytes of launch n: a + b (n + 1) read, wr written
    n = 50
    fetch = [{"Dispatch_Id": 10 + 2 * i, "Kernel_Name": "void bw::k_persist<...>", "Counter_Name": "FETCH_SIZE",
              "Counter_Value": (a + b * (i + 1)) / 2 / kib} for i in range(n)]
    fetch.append({"Dispatch_Id": 11, "Kernel_Name": "other", "Counter_Name": "FETCH_SIZE", "Counter_Value": 1e9})
    # the reset kernel shares the name prefix; the template's "<" keeps it out of the figure
    fetch.append({"Dispatch_Id": 3, "Kernel_Name": "bw::k_persist_reset(bw::PersistParams)", "Counter_Name": "FETCH_SIZE",
                  "Counter_Value": 16.0})
    write = [{"Dispatch_Id": 10 + 2 * i, "Kernel_Name": "void bw::k_persist<...>", "Counter_Name": "WRITE_SIZE",
              "Counter_Value": wr / kib} for i in range(n)]
    _write(tmp_path / "f.csv", fetch[::-1], fields)  # dispatch order comes from Dispatch_Id, not row order
    _write(tmp_path / "w.csv", write, fields)
    res = profiling.traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                            str(tmp_path / "cw.csv"), copy_bytes, "k_persist<", sources=profiling.STEP_SOURCES,
                            fit_context=True, context_start=0)
    assert abs(res["fetch_scale"] - 2.0) < 1e-12 and abs(res["write_scale"] - 1.0) < 1e-12
    mean_true = a + b * (n + 1) / 2 + wr
    assert abs(res["hbm_bytes_per_launch"] - mean_true) / mean_true < 1e-9
    fit = res["fit"]
    assert abs(fit["bytes_at_context_0"] - (a + wr)) / a < 1e-9
    assert abs(fit["bytes_per_context_token"] - b) / b < 1e-6
    assert fit["contexts"] == [1, n] and fit["rms_residual_bytes"] < 1.0
    assert res["contexts"] == [1, n]
    json.dumps(res)


def test_bench_takes_counted_traffic_only_at_its_context_and_sources(tmp_path, monkeypatch):
    """bench.py's `traffic` field: the committed profile whose contexts lie within 64 positions of
    the traced pass and whose kernel-source digest matches the current sources; else null."""
    import bench
    from memory_bound_autoregressive_amd.build import source_digest

    prof = tmp_path / "profiles"
    prof.mkdir()
    digest = source_digest(profiling.STEP_SOURCES)

    def put(name, lo, hi, bytes_, dig=digest):
        with open(prof / name, "w") as f:
            json.dump({"contexts": [lo, hi], "hbm_bytes_per_launch": bytes_, "kernel_sources": list(profiling.STEP_SOURCES),
                       "kernel_source_digest": dig}, f)

    put("step_dense9b_traffic.json", 2049, 2058, 4.19e9)
    put("step_dense9b_traffic_ctx2600.json", 2601, 2610, 4.27e9)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    cfg = {"kv_dtype": "bf16"}
    assert bench.committed_traffic("dense-9b", cfg, 2104.5) == round(4.19e9)
    assert bench.committed_traffic("dense-9b", cfg, 2607.5) == round(4.27e9)
    assert bench.committed_traffic("dense-9b", cfg, 2674.5) is None  # 64.5 past the profile's contexts
    assert bench.committed_traffic("dense-9b", {"kv_dtype": "fp8"}, 2607.5) is None  # another cache dtype
    assert bench.committed_traffic("verify-9b", cfg, 2607.5) is None  # no single-launch profile
    put("step_dense9b_traffic_ctx2600.json", 2601, 2610, 4.27e9, dig="0" * 16)  # sources changed since
    assert bench.committed_traffic("dense-9b", cfg, 2607.5) is None

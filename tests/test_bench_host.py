"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop
counts, the HBM-traffic calibration from rocprofv3 counter CSVs, and the
rule that a traffic figure taken on other kernel sources is not reported."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_and_flops_of_the_decode_shape():
    # K=5120 N=13824 g=128: K*N/2 codes + N*G*2 fp16 scales + N*G/2 zero-points
    # + 2K activation bytes + 2N output bytes
    G = 5120 // 128
    assert bench.algorithmic_bytes(1) == 5120 * 13824 // 2 + 13824 * G * 2 + 13824 * G // 2 \
        + 2 * 5120 + 2 * 13824 == 36809728
    assert bench.algorithmic_bytes(1, scale_bytes=4, has_zp=False) == \
        5120 * 13824 // 2 + 13824 * G * 4 + 2 * 5120 + 2 * 13824
    two = bench.algorithmic_bytes(32, n_weights=2)
    assert two - 2 * 32 * 5120 - 2 * 32 * 13824 == 2 * (36809728 - 2 * 5120 - 2 * 13824)
    assert bench.flops(128) == 2 * 128 * 13824 * 5120
    assert bench.mlp_weight_bytes(4096, 13696, 128) == \
        2 * bench.algorithmic_bytes(0, 4096, 13696) + bench.algorithmic_bytes(0, 13696, 4096)


def _counter_csv(path, counter, rows):
    """rows: (kernel name, dispatch id, [instance values]) -> rocprofv3 CSV."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for name, disp, values in rows:
            for v in values:
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


def test_traffic_calibration_from_counter_csvs(tmp_path):
    """Per dispatch the instances are summed; the median over dispatches is
    scaled by copy_bytes / (copy reading in bytes)."""
    gemm = "void w4a16::stream_kernel<4, 5, 8, 8, true, 128, false, false, 0>(w4a16::GemmArgs)"
    copy = "w4a16::probe_copy_kernel(unsigned int __vector(4) const*, ...)"
    cb = bench.COPY_PROBE_BYTES
    fdir, wdir = tmp_path / "f", tmp_path / "w"
    (fdir / "sub").mkdir(parents=True)
    wdir.mkdir()
    # FETCH_SIZE reads half the copy's bytes (KiB): factor 2; dispatches of
    # the GEMM sum to 100, 110 and 120 KiB (median 110)
    _counter_csv(fdir / "sub" / "f_counter_collection.csv", "FETCH_SIZE",
                 [(gemm, 1, [60, 40]), (gemm, 2, [55, 55]), (gemm, 3, [100, 20]),
                  (copy, 4, [cb / 2048 / 2, cb / 2048 / 2])])
    # WRITE_SIZE reads the copy's bytes exactly: factor 1
    _counter_csv(wdir / "w_counter_collection.csv", "WRITE_SIZE",
                 [(gemm, 1, [27]), (gemm, 2, [27]), (copy, 3, [cb / 1024])])
    r = bench.summarize_traffic(str(fdir), str(wdir))
    assert r["FETCH_SIZE"]["gemm_kib_per_dispatch"] == 110
    assert r["FETCH_SIZE"]["scale_factor"] == pytest.approx(2.0)
    assert r["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(110 * 1024 * 2)
    assert r["WRITE_SIZE"]["scale_factor"] == pytest.approx(1.0)
    assert r["bytes_per_launch"] == pytest.approx(110 * 1024 * 2 + 27 * 1024)
    assert r["kernel_source_hash"] == bench.kernel_source_hash()
    # a run without the copy kernel cannot be calibrated
    _counter_csv(wdir / "w_counter_collection.csv", "WRITE_SIZE", [(gemm, 1, [27])])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(fdir), str(wdir))


def test_traffic_reported_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic() is None                       # no file
    f.write_text(json.dumps({"kernel_source_hash": "0" * 16, "bytes_per_launch": 1.0}))
    assert bench.load_traffic() is None                       # other sources
    f.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(),
                             "bytes_per_launch": 37e6}))
    assert bench.load_traffic() == 37e6



def test_sample_statistics():
    st = bench.stats([5.0, 1.0, 3.0, 2.0, 4.0])
    assert (st["median"], st["min"], st["max"], st["n"]) == (3.0, 1.0, 5.0, 5)
    assert st["p10"] == pytest.approx(1.4) and st["p90"] == pytest.approx(4.6)


def test_sweep_covers_the_variants():
    """The M sweep holds the sizes of the metric, the odd edge tiles and the
    symmetric and fp32-scale variants."""
    import numpy as np
    ms = {m for m, _, _ in bench.SWEEP}
    assert {1, 2, 4, 7, 8, 16, 32, 33, 64, 128} <= ms
    assert (1, np.float16, False) in bench.SWEEP and (128, np.float32, True) in bench.SWEEP


def test_fusion_bytes_from_counter_csvs(tmp_path):
    """summarize_fusion walks the library's dispatches in order (repacks and
    other kernels skipped): per group, each path's kernels per call (1, 3, 1,
    2), then the calibration copies."""
    cb = bench.COPY_PROBE_BYTES
    iters = 2
    for counter, d, copy_kib in (("FETCH_SIZE", tmp_path / "f", cb / 1024 / 2),
                                 ("WRITE_SIZE", tmp_path / "w", cb / 1024)):
        d.mkdir()
        rows, disp = [], 0

        def add(name, kib):
            nonlocal disp
            disp += 1
            rows.append((name, disp, [kib]))
        add("w4a16::repack_weights_kernel(...)", 999)          # skipped
        add("at::native::fill_kernel", 999)                    # not the library's
        for g in bench.FUSION_GROUPS:
            for name, k in bench.FUSION_PATHS:
                for _ in range(iters):
                    for j in range(k):
                        add(f"w4a16::kernel_{name}_{j}", 10 * (j + 1) + g)
        for _ in range(4):
            add("w4a16::probe_copy_kernel(...)", copy_kib)
        _counter_csv(d / "c_counter_collection.csv", counter, rows)
    r = bench.summarize_fusion(str(tmp_path / "f"), str(tmp_path / "w"))
    # FETCH scale 2, WRITE scale 1: a path of k kernels reads sum(10(j+1)+g) KiB each
    for g in bench.FUSION_GROUPS:
        for name, k in bench.FUSION_PATHS:
            kib = sum(10 * (j + 1) + g for j in range(k))
            assert r["groups"][str(g)][name] == pytest.approx(kib * 1024 * 2 + kib * 1024)
    # a dispatch count that does not fit the sequence is refused
    _counter_csv(tmp_path / "w" / "c_counter_collection.csv", "WRITE_SIZE",
                 [("w4a16::kernel_x", 1, [1.0]), ("w4a16::probe_copy_kernel", 2, [cb / 1024])])
    with pytest.raises(SystemExit):
        bench.summarize_fusion(str(tmp_path / "f"), str(tmp_path / "w"))

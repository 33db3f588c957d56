"""Host logic of bench.py's counter summaries, on synthetic rocprofv3 CSV output: dispatches
are keyed by kernel (template instance, decode layer count), HBM bytes are scaled by what the
counter reads for the calibration copy, MFMA FLOPs are the op counts times 512, the busy
fraction divides busy cycles by the per-XCD active cycles times the SIMDs, and a summary is
used only while the kernel sources hash the same."""
import csv
import os

import pytest

import bench

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
INTRA = "void gdn::intra_chunk_kernel<unsigned short, 128, 128, 64, false>(gdn::PrefillParams)"
INTRA_NORM = "void gdn::intra_chunk_kernel<unsigned short, 128, 128, 64, true>(gdn::PrefillParams)"
INTER = "void gdn::inter_chunk_kernel<unsigned short, 128, 128, 64, true>(gdn::PrefillParams)"
INTER_F32 = "void gdn::inter_chunk_kernel<float, 128, 128, 64, false>(gdn::PrefillParams)"
LAYERS = "void gdn::decode_layers_kernel<unsigned short, 128, 128>(gdn::DecodeTable)"
DECODE = "void gdn::decode_kernel<unsigned short, 128, 128>(gdn::DecodeParams)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": name,
                        "Counter_Name": counter, "Counter_Value": value})


def test_kernel_keys():
    assert bench._kernel_key(INTRA, "131072") == "intra"
    assert bench._kernel_key(INTRA_NORM, "131072") == "intra_qknorm"
    assert bench._kernel_key(INTER, "131072") == "inter"
    assert bench._kernel_key(INTER_F32, "131072") == "inter_f32"
    assert bench._kernel_key(INTRA.replace("unsigned short", "float"), "1") == "intra_f32"
    # a 30-layer launch: 256 workgroups of 256 threads per layer
    assert bench._kernel_key(LAYERS, str(30 * 256 * 256)) == "decode_layers_L30"
    assert bench._kernel_key(DECODE, str(256 * 256)) == "decode_L1"
    assert bench._kernel_key(COPY, "512") == "copy"
    assert bench._kernel_key("void at::native::fill_kernel", "1") is None


def test_hbm_summary_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "hbm.txt"))
    cal_kib = bench.COPY_CALIBRATION_BYTES / 1024
    # FETCH_SIZE reads half the true bytes, WRITE_SIZE the true bytes (as measured on MI355X)
    write_csv(tmp_path / "f", [(COPY, 512, "FETCH_SIZE", cal_kib / 2), (COPY, 512, "FETCH_SIZE", 3.0),
                               (INTRA, 1, "FETCH_SIZE", 100.0), (INTRA, 1, "FETCH_SIZE", 300.0),
                               (INTER, 1, "FETCH_SIZE", 50.0)])
    write_csv(tmp_path / "w", [(COPY, 512, "WRITE_SIZE", cal_kib), (INTRA, 1, "WRITE_SIZE", 10.0),
                               (INTER, 1, "WRITE_SIZE", 20.0)])
    bench.summarize_counters(str(tmp_path / "f"), str(tmp_path / "w"))
    doc = bench.load_traffic()
    assert doc["fetch_scale"] == pytest.approx(0.5) and doc["write_scale"] == pytest.approx(1.0)
    assert doc["intra_fetch_bytes"] == pytest.approx(200.0 * 1024 / 0.5)   # mean of two, rescaled
    assert doc["inter_write_bytes"] == pytest.approx(20.0 * 1024)
    assert doc["prefill_bytes_per_launch"] == pytest.approx((400 + 100 + 10 + 20) * 1024)


def test_mfma_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "MFMA_FILE", str(tmp_path / "mfma.txt"))
    xcd, simd = bench.MI355X_XCDS, bench.MI355X_SIMDS
    active = 1000.0   # per XCD
    write_csv(tmp_path / "m", [
        (INTER, 1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2000.0), (INTER, 1, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0),
        (INTER, 1, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * active * simd), (INTER, 1, "GRBM_GUI_ACTIVE", active * xcd),
        (INTRA, 1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 500.0), (INTRA, 1, "SQ_INSTS_VALU_MFMA_MOPS_F32", 30.0),
        (INTRA, 1, "SQ_VALU_MFMA_BUSY_CYCLES", 0.1 * active * simd), (INTRA, 1, "GRBM_GUI_ACTIVE", active * xcd),
        (LAYERS, 30 * 256 * 256, "SQ_VALU_MFMA_BUSY_CYCLES", 0.0), (LAYERS, 30 * 256 * 256, "GRBM_GUI_ACTIVE", 5.0)])
    bench.summarize_mfma(str(tmp_path / "m"))
    doc = bench.load_mfma()
    assert doc["inter_flops_bf16"] == 2000 * 512 and doc["intra_flops_f32"] == 30 * 512
    assert doc["inter_busy_frac"] == pytest.approx(0.25) and doc["intra_busy_frac"] == pytest.approx(0.1)
    assert doc["decode_layers_L30_busy_frac"] == 0.0
    assert doc["prefill_flops_bf16_per_launch"] == 2500 * 512
    f = bench.mfma_counter_fields(doc, 100.0)   # a 100 us call
    assert f["achieved_tflops"] == pytest.approx((2530 * 512) / 100e-6 / 1e12, abs=0.01)


def test_summaries_are_ignored_once_the_kernels_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "MFMA_FILE", str(tmp_path / "mfma.txt"))
    write_csv(tmp_path / "m", [(INTER, 1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1.0), (INTER, 1, "GRBM_GUI_ACTIVE", 8.0)])
    bench.summarize_mfma(str(tmp_path / "m"))
    assert bench.load_mfma() is not None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_mfma() is None
    assert bench.mfma_counter_fields(None, 100.0) is None

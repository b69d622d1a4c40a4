"""bench.py's rocprofv3 summary on synthetic rocprofv3 CSV output (CPU only).

The HBM figures scale each launch's FETCH_SIZE / WRITE_SIZE by what the same
counters read for the 1 GiB device copy in the same run.  The runs also hold
other large kernels (torch's input generation, the attainable-peak GEMM),
so the calibration copy must be found by its kernel, not as the largest
kernel outside the library, and those kernels stay out of the duration
table.
"""
import csv
import os

import pytest

import bench
from combine_top_route_amd import synthetic as S

WL = S.WORKLOADS["q30b"]
GEMM = "void moe::(anonymous namespace)::wgrad_kernel<1>(moe::(anonymous namespace)::WgradArgs)"
COPY = "__amd_rocclr_copyBuffer"
BLAS = "Custom_Cijk_Alik_Bljk_BBS_BH_MT256x256x64_MI16x16x1_UserArgs_shortname0_gfx950"
TORCH = "void at::native::vectorized_elementwise_kernel<8, at::native::FillFunctor<c10::BFloat16>>()"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def _counters(d, key, values):
    """values: (kernel, KiB per dispatch) rows of one counter run."""
    _write(os.path.join(d, "q30b_counter_collection.csv"), ["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                                            "Counter_Value"],
           [(i, k, key, v) for i, (k, v) in enumerate(values)])


def _make(tmp_path, with_copy=True):
    stats = str(tmp_path / "prof")
    _write(os.path.join(stats, "q30b_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "Percentage"],
           [(GEMM, 19, 950000.0, 20.0), (BLAS, 11, 800000.0, 8.0), (TORCH, 4, 100000.0, 1.5)])
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    mib = 1024  # KiB per MiB
    copy = [(COPY, 512 * mib)] if with_copy else []
    # the square GEMM reads more than the copy's counter shows (778 MiB > 512 MiB)
    _counters(fetch, "FETCH_SIZE", [(GEMM, 700 * mib), (GEMM, 702 * mib), (BLAS, 778 * mib), (TORCH, 0)] + copy)
    copyw = [(COPY, 1024 * mib)] if with_copy else []
    _counters(write, "WRITE_SIZE", [(GEMM, 768 * mib), (GEMM, 768 * mib), (BLAS, 128 * mib),
                                    (TORCH, 1024 * mib)] + copyw)
    return stats, fetch, write


def test_calibration_copy_found_by_kernel(tmp_path):
    stats, fetch, write = _make(tmp_path)
    out = str(tmp_path / "summary.md")
    bench.rocprof_summary(WL, out, stats, fetch, write)
    text = open(out).read()
    assert "fetch factor 2.0000" in text and "write factor 1.0000" in text
    # 701 MiB counted per dispatch, scaled by 2 (1 GiB read, 512 MiB counted)
    line = next(l for l in text.splitlines() if l.startswith("traffic: gemm_gateup_wgrad"))
    parts = dict(p.split("=") for p in line.split()[2:])
    assert float(parts["fetch"]) == pytest.approx(701 * 2**20 * 2.0, rel=1e-6)
    assert float(parts["write"]) == pytest.approx(768 * 2**20, rel=1e-6)


def test_duration_table_holds_library_kernels_only(tmp_path):
    stats, fetch, write = _make(tmp_path)
    out = str(tmp_path / "summary.md")
    bench.rocprof_summary(WL, out, stats, fetch, write)
    rows = [l for l in open(out).read().splitlines() if l.startswith("| ") and "`" in l]
    assert len(rows) == 1 and rows[0].startswith("| gemm_gateup_wgrad | `wgrad_kernel<1>` | 19 | 950.0 |")
    assert "own kernels (9.50% of GPU time)" in open(out).read()


def test_missing_calibration_copy_is_an_error(tmp_path):
    stats, fetch, write = _make(tmp_path, with_copy=False)
    with pytest.raises(SystemExit):
        bench.rocprof_summary(WL, str(tmp_path / "summary.md"), stats, fetch, write)

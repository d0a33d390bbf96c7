"""Host-side logic of bench.py (no GPU): the algorithmic byte counts, the rocprofv3 counter
parsing, and the refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_alg_bytes_dense_entries():
    B, H, W, C = 4, 64, 64, 1024
    n = B * H * W * C
    assert bench.alg_bytes("biwkv", B, H, W, C, 2) == 2 * 2 * n + 4 * n + 8 * C
    assert bench.alg_bytes("causal", B, H, W, C, 2) == bench.alg_bytes("biwkv", B, H, W, C, 2)
    assert bench.alg_bytes("gated", B, H, W, C, 2) == 3 * 2 * n + 4 * n + 8 * C
    assert bench.alg_bytes("mix", B, H, W, C, 4) == 4 * n + 4 * bench.N_MIX * n + 4 * bench.N_MIX * C
    # k, v, g read, dk, dv written, w, u read, dw, du written
    assert bench.alg_bytes("backward", B, H, W, C, 2) == (2 + 2 + 4 + 4 + 4) * n + 16 * C
    with pytest.raises(ValueError):
        bench.alg_bytes("nope", B, H, W, C, 2)


@pytest.mark.parametrize("B,H,W,C,shift,gamma", [(2, 6, 5, 40, 1, 0.25), (1, 7, 7, 30, 2, 0.2), (3, 4, 9, 17, 3, 0.125)])
def test_alg_bytes_fused_counts_only_in_grid_sources(B, H, W, C, shift, gamma):
    """The fused entry reads only sources inside the grid: the count of zero-filled outputs of the
    oracle's Q-Shift (on an input with no zeros) is what the byte count leaves out."""
    x = np.ones((B, H * W, C), dtype=np.float32)
    zeros = int((oracle.qshift(x, H, W, shift, gamma) == 0).sum())
    n = B * H * W * C
    assert bench.alg_bytes("fused", B, H, W, C, 2, shift, gamma) == 2 * 2 * (n - zeros) + 4 * n + 8 * C
    assert bench.alg_bytes("qshift", B, H, W, C, 4, shift, gamma) == 4 * (n - zeros) + 4 * n


@pytest.mark.parametrize("B,N,C,shift,gamma", [(2, 30, 40, 1, 0.25), (1, 49, 384, 1, 0.25), (3, 10, 17, 3, 0.2)])
def test_alg_bytes_bidir_counts_only_in_sequence_sources(B, N, C, shift, gamma):
    x = np.ones((B, N, C), dtype=np.float32)
    zeros = int((oracle.qshift_bidir(x, shift, gamma) == 0).sum())
    n = B * N * C
    assert bench.alg_bytes("bidir", B, 1, N, C, 2, shift, gamma) == 2 * 2 * (n - zeros) + 4 * n + 8 * C


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_counter_means_takes_the_largest_grid(tmp_path):
    rows = [
        {"Dispatch_Id": 1, "Kernel_Name": "void biwkv_row_kernel<1>", "Grid_Size": 100, "Counter_Name": "FETCH_SIZE", "Counter_Value": 5},
        {"Dispatch_Id": 2, "Kernel_Name": "void biwkv_row_kernel<1>", "Grid_Size": 4096, "Counter_Name": "FETCH_SIZE", "Counter_Value": 30},
        {"Dispatch_Id": 2, "Kernel_Name": "void biwkv_row_kernel<1>", "Grid_Size": 4096, "Counter_Name": "FETCH_SIZE", "Counter_Value": 10},
        {"Dispatch_Id": 3, "Kernel_Name": "void biwkv_row_kernel<1>", "Grid_Size": 4096, "Counter_Name": "FETCH_SIZE", "Counter_Value": 60},
        {"Dispatch_Id": 3, "Kernel_Name": "void biwkv_row_kernel<1>", "Grid_Size": 4096, "Counter_Name": "WRITE_SIZE", "Counter_Value": 999},
        {"Dispatch_Id": 4, "Kernel_Name": "copyBuffer", "Grid_Size": 9999, "Counter_Name": "FETCH_SIZE", "Counter_Value": 7},
    ]
    _write_counters(str(tmp_path), rows)
    # dispatch 2 sums its instances (40), dispatch 3 reads 60; dispatch 1 (smaller grid) is skipped
    assert bench._counter_means(str(tmp_path), "FETCH_SIZE", "biwkv_row_kernel") == pytest.approx(50.0)


def test_counter_per_call_sums_the_kernels_of_a_call(tmp_path):
    rows = []
    for call in range(3):
        base = 10 * call
        for i, (name, val) in enumerate([("bwd_chunk_sums_kernel", 100), ("bwd_tile_kernel<2>", 200),
                                         ("bwd_tile_kernel<3>", 300), ("bwd_reduce_kernel", 4)]):
            rows.append({"Dispatch_Id": base + i, "Kernel_Name": name, "Grid_Size": 1, "Counter_Name": "FETCH_SIZE",
                         "Counter_Value": val})
    rows.append({"Dispatch_Id": 99, "Kernel_Name": "copyBuffer", "Grid_Size": 1, "Counter_Name": "FETCH_SIZE",
                 "Counter_Value": 12345})
    _write_counters(str(tmp_path), rows)
    assert bench._counter_per_call(str(tmp_path), "FETCH_SIZE", "bwd_", "bwd_reduce_kernel") == pytest.approx(604.0)


def test_backward_call_marker_counts_both_forms(tmp_path):
    """The backward's once-per-call kernel is its dw / du fold, named differently after the one-launch
    and the multi-launch form; the marker counts either, once per call."""
    rows = []
    for call, names in enumerate([[("bwd_one_kernel", 500), ("bwd_one_reduce_kernel", 6)],
                                  [("bwd_chunk_sums_kernel", 100), ("bwd_tile_kernel<3>", 300),
                                   ("bwd_reduce_kernel", 4)]]):
        for i, (name, val) in enumerate(names):
            rows.append({"Dispatch_Id": 10 * call + i, "Kernel_Name": name, "Grid_Size": 1,
                         "Counter_Name": "FETCH_SIZE", "Counter_Value": val})
    _write_counters(str(tmp_path), rows)
    got = bench._counter_per_call(str(tmp_path), "FETCH_SIZE", bench.KERNEL_NAMES["backward"],
                                  bench.CALL_MARKER["backward"])
    assert got == pytest.approx((506 + 404) / 2)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16


def test_kernel_of_entry_tells_the_tile_kernel_variants_apart():
    """A run of the fused entry also times the plain forward: counters must pick the fused
    kernel's dispatches only (by the FUSED, CAUSAL, GATED template flags)."""
    ns = "void (anonymous namespace)::biwkv_row_kernel<1, 64, 64, 512, {f}, true, {c}, {g}, 0>((anonymous namespace)::RowParams)"
    fused = ns.format(f="true", c="false", g="false")
    plain = ns.format(f="false", c="false", g="false")
    causal = ns.format(f="false", c="true", g="false")
    gated = ns.format(f="false", c="false", g="true")
    assert bench.kernel_of_entry(fused, "fused") and not bench.kernel_of_entry(plain, "fused")
    assert bench.kernel_of_entry(plain, "biwkv") and not bench.kernel_of_entry(fused, "biwkv")
    assert bench.kernel_of_entry(fused, "bidir")
    assert bench.kernel_of_entry(causal, "causal") and not bench.kernel_of_entry(causal, "biwkv")
    assert bench.kernel_of_entry(gated, "gated") and not bench.kernel_of_entry(gated, "fused")
    assert bench.kernel_of_entry("void (anonymous namespace)::qshift_kernel<4, false>(unsigned int const*)", "qshift")
    assert not bench.kernel_of_entry("void (anonymous namespace)::qshift_kernel<4, false>(x)", "biwkv")


def test_summarize_sq_derives_per_wave_figures(tmp_path, capsys):
    # three passes, two dispatches of one kernel: means per counter, then the stated formulas
    rows = {
        "p1": {"SQ_WAVES": (100, 100), "SQ_INSTS_VALU": (2000, 2200), "SQ_INSTS_VALU_TRANS_F32": (300, 300),
               "SQ_INSTS_SALU": (500, 500), "SQ_INSTS_LDS": (10, 10), "SQ_INSTS_VMEM_RD": (640, 640),
               "SQ_INSTS_VMEM_WR": (320, 320), "SQ_INSTS_SMEM": (70, 70)},
        "p2": {"SQ_WAVE_CYCLES": (1000, 1000), "SQ_BUSY_CYCLES": (50, 50), "SQ_ACTIVE_INST_VALU": (200, 200)},
        "p3": {"SQ_LDS_BANK_CONFLICT": (7, 9), "SQ_LDS_IDX_ACTIVE": (100, 100)},
    }
    dirs = []
    for name, ctrs in rows.items():
        d = tmp_path / name
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
            for cname, vals in ctrs.items():
                for v in vals:
                    w.writerow(["my_kernel(int)", cname, v])
        dirs.append(str(d))
    bench.summarize_sq(*dirs)
    out = capsys.readouterr().out
    assert "my_kernel" in out
    assert "per wave: VALU 21 (transcendental 3), SALU 5, LDS 0.1, vector loads 6.4" in out
    # 4 * 1000 / (50 * 32) = 2.50 waves per SIMD; 4 * 200 / (50 * 32) = 0.50 VALU-active
    assert "resident waves per SIMD 2.50; VALU-active share 0.50; LDS bank-conflict cycles 8 of 100" in out

"""Host-side checks of the benchmark's bookkeeping (no GPU).

The grid sizes below are the work-item counts rocprofv3 recorded for these
kernels on MI355X (profiles/qmm_configs_traffic.md,
profiles/qmm_dense_decode_step_traffic.md); bench.launch_grid must reproduce
them from the kernel name and the matrix heights, including the split grids
whose blocks after the last whole round over the CUs hold one row per lane.
"""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

RECORDED_GRIDS = [
    # (kernel, matrix heights, recorded work-items)
    ("qmm_dense_kernel<1, 1, 5, 1, 1, 2, 1, 64>", [20480], 327680),            # gate+up, M = 1
    ("qmm_dense_kernel<1, 1, 5, 4, 1, 2, 1, 64>", [2560], 163840),             # down, M = 1
    ("qmm_dense_kernel<1, 1, 1, 5, 1, 1, 1, 64>", [2560], 204800),             # o, M = 1
    ("qmm_dense_kernel<1, 1, 1, 5, 1, 1, 1, 64>", [512], 40960),               # k, M = 1
    ("qmm_dense_kernel<1, 1, 1, 5, 1, 1, 1, 64>", [2560, 512, 512], 614400),   # grouped q/k/v, M = 1
    ("qmm_dense_split_kernel<5, 2, 5, 1, 1, 2, 1, 64>", [20480], 196608),      # gate+up, M = 5
    ("qmm_dense_split_kernel<5, 2, 1, 4, 1, 2, 1, 64>", [2560], 98304),        # down, M = 5
    ("qmm_dense_split_kernel<5, 2, 1, 5, 1, 1, 1, 64>", [2560], 122880),       # o, M = 5
    ("qmm_dense_kernel<4, 2, 4, 1, 1, 2, 1, 64>", [16384], 131072),            # square, M = 4
    ("qmm_dense_kernel<1, 1, 4, 1, 1, 2, 1, 64>", [16384], 262144),            # square, M = 1
]


@pytest.mark.parametrize("kernel,Ns,items", RECORDED_GRIDS)
def test_launch_grid_matches_recorded_dispatches(kernel, Ns, items):
    assert bench.launch_grid(kernel, Ns) == items


def test_step_bytes_of_the_decode_step():
    # 42 layers of q, k, v, o (2560 / 512 / 512 / 2560 <- 2560), gate+up
    # (20480 <- 2560) and down (2560 <- 10240): codes (N K / 2 bytes), scales
    # and biases (2 bytes per 64 codes each), x (M K bf16) and y (M N bf16)
    shapes = [(2560, 2560), (512, 2560), (512, 2560), (2560, 2560), (20480, 2560), (2560, 10240)]
    per_layer = sum(n * k // 2 + 2 * (n * k // 64) * 2 + k * 2 + n * 2 for n, k in shapes)
    assert bench.step_bytes(1, 42) == 42 * per_layer == 2233921536


def test_floors_scale_with_the_activation_rows():
    # flops: 2 (M + 1) per weight; issue: 42 + 16 M cycles per word and wave
    gu = ("gate_up",)
    assert bench.unit_flops(5, gu) == 2 * bench.unit_flops(2, gu) == 12 * 20480 * 2560
    r = bench.unit_issue_floor_us(5, gu) / bench.unit_issue_floor_us(1, gu)
    assert abs(r - (42 + 16 * 5) / (42 + 16)) < 1e-12
    # gate+up at M = 1: 20480 * 2560 / 8 words over 64 lanes and 1024 SIMDs
    # at 58 cycles per word and wave, 2.4 GHz
    expect = 20480 * 2560 / 8 / 64 / 1024 * 58 / 2400.0
    assert abs(bench.unit_issue_floor_us(1, gu) - expect) < 1e-9


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_counter_summary_tables(tmp_path):
    # one kernel, two dispatches per counter (the summary takes the median);
    # a non-library kernel in the same file is left out
    from decode_w4a16_affine_amd import profiling
    name = "void w4k::qmm_dense_kernel<5, 2, 1, 5, 1, 1, 1, 64>(int)"
    counters = {"SQ_WAVES": 320, "SQ_WAVE_CYCLES": 1000, "SQ_INSTS_VALU": 6400, "SQ_INSTS_LDS": 640,
                "SQ_LDS_BANK_CONFLICT": 320, "SQ_WAIT_ANY": 250, "SQ_WAIT_INST_ANY": 350, "SQ_ACTIVE_INST_ANY": 400,
                "SQ_ACTIVE_INST_VALU": 300, "SQ_INST_LEVEL_VMEM": 120}
    path = tmp_path / "c.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for dispatch in range(2):
            for c, v in counters.items():
                w.writerow([20480, name, c, v * (1 + dispatch)])   # medians: 1.5 x
            w.writerow([256, "void other_kernel()", "SQ_WAVES", 1])
    out = tmp_path / "c.md"
    profiling.summarize_sq(str(path), str(out), "cmd")
    text = out.read_text()
    assert "other_kernel" not in text
    rows = [l for l in text.splitlines() if l.startswith("| `qmm_dense_kernel<5, 2, 1, 5, 1, 1, 1, 64>`")]
    assert len(rows) == 3   # instructions, memory waits, wave states
    first = [c.strip() for c in rows[0].split("|")[1:-1]]
    # waves 480, VALU / wave 20, LDS / wave 2, conflict cycles / LDS instr 0.5, wave cycles / wave 3.125 -> 3
    assert first[1:4] == ["20480", "480", "20"] and first[5:8] == ["2", "0.50", "3"]
    # SQ_WAIT_ANY / wave cycles, vector-memory reads / wave (not collected), loads in flight
    assert [c.strip() for c in rows[1].split("|")[1:-1]][2:] == ["0.25", "0", "0.12"]
    states = [c.strip() for c in rows[2].split("|")[1:-1]]
    # fractions of SQ_WAVE_CYCLES; no SQ_ACTIVE_INST_LDS was collected
    assert states[3:9] == ["0.25", "0.35", "0.40", "0.30", "-", "0.12"]


def test_prefill_matrix_factor_follows_the_dispatch():
    # gate+up 20480 <- 2560 and down 2560 <- 10240 at the benchmark's M
    f = bench.prefill_matrix_factor
    assert f(16, 20480) is None and f(16, 2560) is None       # decode kernels on 8-row chunks
    assert f(64, 20480) == 1.5                                 # 160 tiles of 64 rows
    assert f(64, 2560) == 2.0                                  # per-wave form
    assert f(512, 20480) == 1.25 and f(4096, 20480) == 1.25    # 128-row tiles
    assert f(512, 2560) == 1.5                                 # 80 tiles of 128 rows, 160 of 64
    assert f(384, 2560) == 2.0 and f(1024, 2560) == 1.25 and f(4096, 2560) == 1.25

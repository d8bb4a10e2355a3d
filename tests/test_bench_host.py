"""CPU checks of bench.py's bookkeeping: the algorithmic multiply-add and byte counts behind
every TFLOP/s, GB/s and roofline figure (pinned to the values the pages print and to closed
forms of the convolution shapes), the output shapes, the kernel each workload runs, and the
one-GPU guard."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

import bench
import oracle
from implicit_gemm_convolution_conv3d_amd import workloads as wl

ROOT = Path(__file__).resolve().parent.parent
PAGES = json.loads((ROOT / "tests" / "golden" / "page_values.json").read_text())


def test_pool_macs_match_the_page():
    macs, nbytes = bench.work(wl.WORKLOADS[2])
    assert macs == PAGES["pool_conv_macs"]["value"]          # 23,806,476,288
    # x + w + conv_b + bias + out, each once
    assert nbytes == 4 * (128 * 8 * 16 * 64 * 64 + 16 * 8 * 27 + 16 + 16 + 128)


def test_pool_macs_count_only_the_windows_conv_outputs():
    # 3x3x3 pool over a 14x62x62 conv output: floor mode reads 12x60x60 of it
    macs, _ = bench.work(wl.WORKLOADS[7])
    assert macs == 128 * 16 * (12 * 60 * 60) * 8 * 27
    # 2x2x2 pool on even sizes reads every conv output: the page's count
    assert bench.work(wl.WORKLOADS[9])[0] == PAGES["pool_conv_macs"]["value"]


def test_conv3d_macs_match_the_page():
    macs, nbytes = bench.work(wl.WORKLOADS[3])
    assert macs == (PAGES["conv3d_mish_tanh_output_elements"]["value"]
                    * PAGES["conv3d_mish_tanh_macs_per_output"]["value"])
    assert nbytes == 4 * (16 * 32 * 32 * 64 * 64 + 64 * 32 * 27 + 64 + 16 * 64 * 30 * 62 * 62)


def test_dwsep_counts_closed_form():
    # per output pixel: 9 depthwise MACs per input channel + Cin * Cout pointwise MACs
    macs, nbytes = bench.work(wl.WORKLOADS[4])
    assert macs == 16 * 512 * 512 * (64 * 9 + 64 * 128) == 36_775_657_472
    assert nbytes == 4 * (16 * 64 * 512 * 512 + 64 * 9 + 128 * 64 + 16 * 128 * 512 * 512)
    macs5, nbytes5 = bench.work(wl.WORKLOADS[5])
    assert macs5 == 8 * 333 * 517 * (96 * 9 + 96 * 192)
    assert nbytes5 == 4 * (8 * 96 * 333 * 517 + 96 * 9 + 192 * 96 + 8 * 192 * 333 * 517 + 96 + 192)


@pytest.mark.parametrize("index", sorted(wl.WORKLOADS))
def test_output_dims_use_the_oracles_formula(index):
    w = wl.WORKLOADS[index]
    d, p = w.dims, w.params
    if w.op.startswith("dwsep"):
        args = (p["K"], p["stride"], p["pad"], p["dilation"])
        expect = tuple(oracle.out_len(d[a], *args) for a in ("H", "W"))
    else:
        s, pad = p.get("stride", 1), p.get("pad", 0)
        expect = tuple(oracle.out_len(d[a], p["k"], s, pad) for a in ("D", "H", "W"))
    assert bench.out_dims(w) == expect


def test_split_workloads_count_the_same_work():
    for fp32, split in ((4, 10), (5, 11), (3, 12), (2, 13)):
        assert bench.work(wl.WORKLOADS[fp32]) == bench.work(wl.WORKLOADS[split])


def test_kernel_names():
    names = {i: bench.kernel_name(w) for i, w in wl.WORKLOADS.items()}
    assert names[2] == "conv3d_pool_sum_kernel"
    assert names[3] == "conv3d_mish_tanh_kernel"
    assert names[4] == names[5] == "dwsep_persistent_kernel"
    assert names[6] == "conv3d_staged_kernel"
    assert names[7] == "conv3d_pool_staged_kernel"
    assert names[8] == "dwsep_staged_kernel"
    assert names[10] == names[11] == "dwsep_split_kernel"
    assert names[12] == "conv3d_split_kernel"
    assert names[13] == "conv3d_pool_split_kernel"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_matrix_work_excludes_the_depthwise_step():
    # the pointwise GEMM alone runs on the matrix cores: 2 * pixels * Cin * Cout FLOP
    assert bench.gemm_macs(wl.WORKLOADS[4]) == 16 * 512 * 512 * 64 * 128
    assert bench.gemm_macs(wl.WORKLOADS[5]) == 8 * 333 * 517 * 96 * 192
    # the Conv3d layers are one contraction
    for i in (1, 2, 3, 6, 7, 9):
        assert bench.gemm_macs(wl.WORKLOADS[i]) == bench.work(wl.WORKLOADS[i])[0]
    assert bench.graded_bound(wl.WORKLOADS[4]) == bench.graded_bound(wl.WORKLOADS[5]) == "hbm"
    assert bench.graded_bound(wl.WORKLOADS[2]) == bench.graded_bound(wl.WORKLOADS[3]) == "mfma"


def test_workload_figures_grade_against_the_right_roof():
    import numpy as np
    w4 = wl.WORKLOADS[4]
    ms = np.array([0.80, 0.70, 0.75])
    rec = bench.workload_figures(w4, ms, ms, None)
    assert rec["ms_median"] == 0.75
    macs, nbytes = bench.work(w4)
    assert rec["frac_hbm"] == round(nbytes / 0.75e-3 / 8e12, 4)
    assert rec["frac_fp32_mfma"] == round(2 * 16 * 512 * 512 * 64 * 128 / 0.75e-3 / 157.3e12, 4)
    assert rec["graded"]["bound"] == "hbm" and rec["graded"]["frac"] == rec["frac_hbm"]
    rec3 = bench.workload_figures(wl.WORKLOADS[3], ms, ms, ms)
    assert rec3["graded"]["bound"] == "mfma" and rec3["vector_gflop"] == 0
    assert bench.workload_figures(wl.WORKLOADS[1], ms, ms, None)["graded"] is None

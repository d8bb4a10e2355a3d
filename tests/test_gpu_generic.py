"""GPU parity of the general-parameter kernels (any kernel size, stride, padding, dilation,
pooling window; Conv3d kernel sizes 3/5/7 at strides 1/2 run the LDS-staged kernel, other
ones the direct kernel) against the fp64 CPU oracle, through the C ABI.  Same tolerances as the
tuned kernels: |gpu - ref| <= 1e-4 + 1e-4 |ref| elementwise for conv3d_mish_tanh and
dwsep_conv2d, relative 1e-4 per batch scalar for the pooled sum.  Every case here uses
parameters outside the tuned kernels' range (k != 3, stride > 1, pad > 2, pool != 2,
dilation > 1), so the general kernels are the ones that run."""
import numpy as np
import pytest

import bench
import oracle
from implicit_gemm_convolution_conv3d_amd import workloads as wl

from test_gpu_full_parity import Tally, _torch
from test_gpu_parity import assert_close, cf, dev, POOL_RTOL

pytestmark = pytest.mark.gpu

ACT_CASES = [
    # (N, C, D, H, W, O, k, stride, pad, bias)
    (1, 4, 7, 9, 20, 8, 1, 1, 0, True),       # 1x1x1 kernel
    (2, 5, 8, 10, 37, 19, 5, 1, 2, True),     # k = 5, ragged channels and columns
    (1, 6, 9, 11, 40, 40, 3, 2, 1, False),    # stride 2, three channel blocks, no bias
    (1, 3, 7, 8, 21, 16, 2, 3, 0, True),      # even kernel, stride 3
    (1, 4, 5, 6, 17, 33, 3, 1, 4, True),      # padding wider than the kernel reach
    (1, 2, 12, 12, 12, 5, 7, 2, 3, True),     # k = 7
    (1, 6, 10, 12, 70, 20, 7, 1, 3, True),    # k = 7 stride 1, two column tiles, ragged W
    (2, 9, 9, 9, 33, 16, 5, 2, 0, False),     # k = 5 stride 2, one channel block, no padding
    (1, 5, 4, 5, 9, 7, 3, 1, 3, True),        # k = 3 with padding 3: more padding than input
]


@pytest.mark.parametrize("case", ACT_CASES)
def test_conv3d_mish_tanh_general(case):
    N, C, D, H, W, O, k, s, p, bias = case
    inp = wl.conv3d_act_inputs(400 + sum(case), N, C, D, H, W, O, k=k, bias=bias)
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"], s, p)
    y = cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), s, p)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "conv3d_mish_tanh general %s" % (case,))


POOL_CASES = [
    # (N, C, D, H, W, O, k, pool, divisor, conv_bias)
    (2, 4, 8, 9, 21, 16, 3, 3, 2.0, True),     # 3x3x3 pool, floor mode drops a column
    (2, 3, 9, 9, 40, 7, 5, 2, -1.5, True),     # k = 5, negative divisor
    (1, 4, 6, 8, 10, 20, 1, 4, 3.0, False),    # k = 1, pool 4, two channel groups
    (1, 2, 35, 35, 40, 3, 1, 32, 2.0, True),   # the largest pooling window
    (3, 5, 5, 5, 5, 4, 3, 1, 0.5, True),       # pool 1: the mean of every conv output
]


@pytest.mark.parametrize("case", POOL_CASES)
def test_pool_general(case):
    N, C, D, H, W, O, k, pool, div, cbias = case
    inp = wl.conv3d_pool_inputs(500 + int(sum(case)), N, C, D, H, W, O, k=k, conv_bias=cbias)
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(inp["x"], inp["w"], inp["conv_b"], div, pool,
                                                 inp["bias"])
    out = cf().conv3d_div_maxpool_gap_bias_sum(dev(inp["x"]), dev(inp["w"]), dev(inp["conv_b"]),
                                               div, pool, dev(inp["bias"]))
    got = out.cpu().numpy().astype(np.float64)
    rel = np.abs(got - ref) / np.abs(ref)
    assert rel.max() <= POOL_RTOL, (case, got, ref)


MAXPOOL_CASES = [
    # (N, C, D, H, W, O, k, pool, divisor, conv_bias): the pooled tensor
    (1, 5, 9, 15, 40, 16, 3, 3, 2.0, True),     # pool 3: windows straddle 16-column blocks
    (2, 3, 11, 23, 30, 20, 5, 4, -1.5, True),   # k = 5, pool 4, negative divisor, two groups
    (1, 6, 6, 14, 70, 9, 1, 2, 3.0, False),     # k = 1, pool 2, several column tiles
    (1, 4, 12, 30, 33, 16, 3, 3, 0.5, True),    # pooled rows past one workgroup's four
]


@pytest.mark.parametrize("case", MAXPOOL_CASES)
def test_maxpool_tensor_general(case):
    N, C, D, H, W, O, k, pool, div, cbias = case
    inp = wl.conv3d_pool_inputs(550 + int(sum(case)), N, C, D, H, W, O, k=k, conv_bias=cbias)
    ref = oracle.conv3d_div_maxpool(inp["x"], inp["w"], inp["conv_b"], div, pool)
    y = cf().conv3d_div_maxpool(dev(inp["x"]), dev(inp["w"]), dev(inp["conv_b"]), div, pool)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "pooled tensor general %s" % (case,))


DW_CASES = [
    # (N, C, H, W, O, K, stride, pad, dilation, bias)
    (2, 8, 13, 30, 16, 1, 1, 0, 1, True),      # pointwise only (K = 1)
    (1, 20, 15, 33, 40, 5, 1, 2, 1, False),    # K = 5
    (1, 12, 20, 41, 200, 7, 2, 3, 1, True),    # K = 7, stride 2, two output-channel groups
    (2, 7, 11, 17, 9, 3, 1, 2, 2, True),       # dilation 2
    (1, 4, 9, 19, 8, 3, 2, 1, 1, False),       # stride 2
    (1, 6, 8, 8, 70, 3, 1, 4, 1, True),        # padding 4
    (1, 10, 9, 40, 24, 4, 1, 2, 1, True),      # even kernel K = 4
    (2, 13, 12, 70, 130, 6, 2, 3, 2, False),   # K = 6, stride 2, dilation 2, ragged slices
    (1, 16, 20, 30, 8, 2, 1, 0, 3, True),      # K = 2, dilation 3, no padding
    (1, 9, 7, 200, 72, 7, 1, 3, 1, True),      # K = 7, four column tiles
]


@pytest.mark.parametrize("case", DW_CASES)
def test_dwsep_general(case):
    N, C, H, W, O, K, s, p, d, bias = case
    inp = wl.dwsep_inputs(600 + sum(case), N, C, H, W, O, K=K, bias=bias)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], s,
                              p, d)
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                          dev(inp["pw_b"]), s, p, d)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "dwsep general %s" % (case,))


def test_conv3d_mish_tanh_general_larger():
    """k = 5, stride 2, pad 2 on a multi-tile shape: every output."""
    inp = wl.conv3d_act_inputs(77, 2, 16, 24, 48, 48, 32, k=5)
    y = cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), 2, 2)
    assert tuple(y.shape) == (2, 32, 12, 24, 24)
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"], 2, 2)
    assert_close(y.cpu().numpy(), ref, "conv3d k5 s2")


def test_dwsep_general_larger():
    """K = 5, stride 2, dilation 2 on a multi-tile shape: every output."""
    inp = wl.dwsep_inputs(78, 2, 32, 96, 130, 64, K=5, bias=True)
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                          dev(inp["pw_b"]), 2, 4, 2)
    assert tuple(y.shape) == (2, 64, 48, 65)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], 2, 4, 2)
    assert_close(y.cpu().numpy(), ref, "dwsep K5 s2 d2")


@pytest.mark.parametrize("index", [6, 8])
def test_general_workload_every_output(index):
    """The general-parameter workloads at the size bench.py times them: every output, compared
    one batch item at a time."""
    torch = _torch()
    w = wl.WORKLOADS[index]
    inp = w.inputs()
    p = w.params
    if w.op == "conv3d_mish_tanh":
        y = cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), p["stride"],
                                  p["pad"])
        ref_of = lambda n: oracle.conv3d_mish_tanh(inp["x"][n:n + 1], inp["w"], inp["b"],
                                                   p["stride"], p["pad"])
    else:
        y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                              dev(inp["pw_b"]), p["stride"], p["pad"], p["dilation"])
        ref_of = lambda n: oracle.dwsep_conv2d(inp["x"][n:n + 1], inp["dw_w"], inp["dw_b"],
                                               inp["pw_w"], inp["pw_b"], p["stride"], p["pad"],
                                               p["dilation"])
    assert cf().last_kernel() == bench.kernel_name(w)
    host = y.cpu().numpy()
    del y
    torch.cuda.empty_cache()
    t = Tally("workload %d %s" % (index, w.name))
    for n in range(host.shape[0]):
        t.add(host[n:n + 1], ref_of(n), "batch item %d" % n)
    assert t.count == host.size
    t.report()


def test_general_pool_workload_every_scalar():
    """The 3x3x3-pool workload at the size bench.py times it: all 128 scalars."""
    w = wl.WORKLOADS[7]
    inp = w.inputs()
    p = w.params
    out = cf().conv3d_div_maxpool_gap_bias_sum(dev(inp["x"]), dev(inp["w"]), dev(inp["conv_b"]),
                                               p["divisor"], p["pool"], dev(inp["bias"]))
    assert cf().last_kernel() == bench.kernel_name(w)
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(inp["x"], inp["w"], inp["conv_b"], p["divisor"],
                                                 p["pool"], inp["bias"])
    rel = np.abs(got - ref) / np.abs(ref)
    assert rel.max() <= POOL_RTOL, (got, ref)

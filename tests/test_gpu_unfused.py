"""GPU parity of the unfused path's separate steps (conv + bias, elementwise tanh(mish), the
pooled channel sum from a stored conv output, depthwise alone, pointwise alone) against the
fp64 oracle, through the C ABI, and of their compositions against the fused oracle.  Each
step's reference is the oracle's own definition: conv3d; mish_tanh; the pooled sum of a
1x1x1 identity convolution; dwsep with identity pointwise weights (depthwise alone) or with
a 1x1 unit depthwise kernel (pointwise alone).  Tolerances as for the fused kernels."""
import numpy as np
import pytest

import oracle
from implicit_gemm_convolution_conv3d_amd import workloads as wl

from test_gpu_parity import assert_close, cf, dev, POOL_RTOL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", [(2, 5, 7, 9, 37, 19, 3, 1, 0), (1, 32, 6, 9, 70, 64, 3, 1, 1),
                                  (1, 4, 8, 10, 21, 8, 5, 2, 2)])
def test_conv3d_bias(case):
    N, C, D, H, W, O, k, s, p = case
    inp = wl.conv3d_act_inputs(800 + sum(case), N, C, D, H, W, O, k=k)
    ref = oracle.conv3d(inp["x"], inp["w"], inp["b"], s, p)
    y = cf().conv3d_bias(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), s, p)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "conv3d_bias %s" % (case,))


def test_mish_tanh_elementwise():
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.standard_normal(10001) * 8,
                        np.array([0, 20, 20.0001, -20, 30, -200, 88, -88], np.float64)]
                       ).astype(np.float32)
    ref = oracle.mish_tanh(v.astype(np.float64))
    y = cf().mish_tanh(dev(v))
    assert_close(y.cpu().numpy(), ref, "mish_tanh")
    t = dev(v)
    cf().mish_tanh(t, out=t)  # in place
    assert_close(t.cpu().numpy(), ref, "mish_tanh in place")


@pytest.mark.parametrize("case", [(3, 16, 14, 20, 21, 2, 2.0), (2, 5, 9, 10, 31, 3, -1.5)])
def test_div_maxpool_gap_bias_sum_from_conv(case):
    N, C, OD, OH, OW, pool, div = case
    rng = np.random.default_rng(10 + sum(case[:5]))
    conv = rng.standard_normal((N, C, OD, OH, OW)).astype(np.float32)
    bias = rng.standard_normal(C).astype(np.float32)
    ident = np.zeros((C, C, 1, 1, 1), np.float32)
    ident[np.arange(C), np.arange(C)] = 1.0
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(conv, ident, None, div, pool, bias)
    got = cf().div_maxpool_gap_bias_sum(dev(conv), div, pool, dev(bias)).cpu().numpy()
    assert np.max(np.abs(got - ref) / np.abs(ref)) <= POOL_RTOL


@pytest.mark.parametrize("case", [(2, 8, 13, 70, 3, 1, 1, 1, True), (1, 6, 20, 41, 5, 2, 2, 1, False),
                                  (1, 4, 11, 17, 3, 1, 2, 2, True)])
def test_depthwise_conv2d(case):
    N, C, H, W, K, s, p, d, bias = case
    inp = wl.dwsep_inputs(900 + sum(case), N, C, H, W, C, K=K, bias=bias)
    ident = np.eye(C, dtype=np.float32).reshape(C, C, 1, 1)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], ident, None, s, p, d)
    y = cf().depthwise_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), s, p, d)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "depthwise %s" % (case,))


@pytest.mark.parametrize("case", [(2, 8, 13, 70, 16, True), (1, 64, 17, 64, 128, False),
                                  (1, 96, 7, 45, 192, True), (1, 20, 9, 33, 40, False)])
def test_pointwise_conv2d(case):
    N, C, H, W, O, bias = case
    inp = wl.dwsep_inputs(950 + sum(case), N, C, H, W, O, bias=bias)
    unit = np.ones((C, 1, 1, 1), np.float32)
    ref = oracle.dwsep_conv2d(inp["x"], unit, None, inp["pw_w"], inp["pw_b"], 1, 0, 1)
    y = cf().pointwise_conv2d(dev(inp["x"]), dev(inp["pw_w"]), dev(inp["pw_b"]))
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "pointwise %s" % (case,))


def test_unfused_compositions_match_fused_oracle():
    """conv -> mish_tanh, conv -> pooled sum, depthwise -> pointwise against the fused oracle."""
    inp = wl.conv3d_act_inputs(31, 1, 8, 6, 10, 40, 32)
    y = cf().mish_tanh(cf().conv3d_bias(dev(inp["x"]), dev(inp["w"]), dev(inp["b"])))
    assert_close(y.cpu().numpy(), oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"]),
                 "conv3d -> mish_tanh")
    pin = wl.conv3d_pool_inputs(32, 2, 4, 8, 12, 22, 16)
    conv = cf().conv3d_bias(dev(pin["x"]), dev(pin["w"]), dev(pin["conv_b"]))
    got = cf().div_maxpool_gap_bias_sum(conv, 2.0, 2, dev(pin["bias"])).cpu().numpy()
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(pin["x"], pin["w"], pin["conv_b"], 2.0, 2,
                                                 pin["bias"])
    assert np.max(np.abs(got - ref) / np.abs(ref)) <= POOL_RTOL
    din = wl.dwsep_inputs(33, 1, 24, 19, 40, 48, bias=True)
    y = cf().pointwise_conv2d(cf().depthwise_conv2d(dev(din["x"]), dev(din["dw_w"]),
                                                    dev(din["dw_b"])),
                              dev(din["pw_w"]), dev(din["pw_b"]))
    ref = oracle.dwsep_conv2d(din["x"], din["dw_w"], din["dw_b"], din["pw_w"], din["pw_b"])
    assert_close(y.cpu().numpy(), ref, "depthwise -> pointwise")

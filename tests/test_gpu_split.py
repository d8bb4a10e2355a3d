"""GPU parity of the split-bf16 modes (dwsep_conv2d_split_bf16: the pointwise GEMM;
conv3d_mish_tanh_split_bf16: the Conv3d implicit GEMM) -- opt-in modes that run the
contraction as a three-term bf16 split of fp32 on the matrix cores -- against the fp64 CPU
oracle through the C ABI.  The Conv3d mode's contract is
    |y - y_exact| <= 1e-4 + 1e-4 |y_exact| + 2^-13 * sum over taps and channels |x * w|
(3 * 2^-16 per product, times tanh(mish)'s slope of at most 1.1), with the sum taken from the
oracle's Conv3d of |x| and |w|.  The dwsep mode's contract, with d[c] the exact depthwise
output at the pixel, is
    |y[o] - y_exact[o]| <= 1e-4 + 1e-4 |y_exact[o]| + 2^-14 * sum_c |d[c] * pw[o,c]|
(bf16 rounding to nearest leaves |v - hi - lo| <= 2^-16 |v| and |lo| <= 2^-8 |v|, so each
product loses at most 3 * 2^-16 |v*w|).  The sum is computed here from the oracle's depthwise
output (the oracle's depthwise-separable conv with an identity pointwise step).  Cases cover
ragged tiles, channel counts off the k-steps and chunks, several output-channel slices, every
padding the split kernels take, every output of the full-size workloads, and a closed form
that fixes which of the split's product terms are present."""
import numpy as np
import pytest

import bench
import oracle
from implicit_gemm_convolution_conv3d_amd import workloads as wl

from conftest import PARITY_REPORT
from test_gpu_parity import _torch, cf, dev

pytestmark = pytest.mark.gpu

SPLIT_SLACK = 2.0 ** -14


def depthwise_exact(inp, stride, pad, dil):
    """The depthwise output [N, C, Ho, Wo] in fp64 from the oracle (identity pointwise)."""
    C = inp["dw_w"].shape[0]
    eye = np.eye(C, dtype=np.float32).reshape(C, C, 1, 1)
    return oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], eye, None, stride, pad, dil)


def assert_split_close(got, ref, abs_dot, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = 1e-4 + 1e-4 * np.abs(ref) + SPLIT_SLACK * abs_dot
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    bad = err > bound
    assert not bad.any(), "%s: %d/%d outside the split contract; worst err %.3g (bound %.3g)" % (
        what, bad.sum(), bad.size, err.reshape(-1)[np.argmax(err / bound)],
        bound.reshape(-1)[np.argmax(err / bound)])


SPLIT_CASES = [
    # (N, C, H, W, O, pad, bias)
    (2, 8, 13, 70, 16, 1, False),          # ragged W and H tiles, one partial k-step
    (1, 20, 9, 33, 40, 1, True),           # Cin % 4 != 0, Cout % 16 != 0
    (1, 64, 17, 64, 128, 1, False),        # the 512^2 workload's channel shape
    (1, 96, 7, 45, 192, 1, True),          # the odd workload's channel shape
    (1, 40, 6, 20, 200, 2, True),          # padding 2, two output-channel slices
    (1, 4, 5, 19, 8, 0, False),            # no padding
    (1, 3, 1, 1, 5, 1, True),              # 1x1 image
    (3, 33, 10, 24, 70, 1, True),          # one channel past a k-step, 3 images
    # split weights near the LDS limit
    (1, 170, 6, 24, 100, 1, True),         # 128-channel group, aligned rows
    (1, 110, 5, 21, 150, 1, True),         # 192-channel group, unaligned rows
    (1, 330, 4, 20, 48, 1, False),         # 64-channel group
    # tall images: more tiles than workgroups, so workgroups take several tiles each
    (2, 40, 600, 130, 100, 1, True),       # two chunks, ragged unaligned columns, 2 images
    (1, 48, 1100, 64, 64, 2, True),        # padding 2
]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_split_small(case):
    N, C, H, W, O, pad, bias = case
    inp = wl.dwsep_inputs(700 + sum(case), N, C, H, W, O, bias=bias)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], 1,
                              pad, 1)
    d = depthwise_exact(inp, 1, pad, 1)
    abs_dot = np.einsum("oc,nchw->nohw", np.abs(inp["pw_w"][:, :, 0, 0].astype(np.float64)),
                        np.abs(d))
    y = cf().dwsep_conv2d_split_bf16(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]),
                                     dev(inp["pw_w"]), dev(inp["pw_b"]), 1, pad, 1)
    assert tuple(y.shape) == ref.shape
    assert_split_close(y.cpu().numpy(), ref, abs_dot, "split %s" % (case,))


def test_split_general_parameters_run_fp32():
    """Geometries outside the split kernel (here K = 5, stride 2) run the fp32 kernels and meet
    the fp32 tolerance."""
    inp = wl.dwsep_inputs(790, 1, 12, 20, 41, 24, K=5, bias=True)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], 2, 2,
                              1)
    y = cf().dwsep_conv2d_split_bf16(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]),
                                     dev(inp["pw_w"]), dev(inp["pw_b"]), 2, 2, 1)
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-4 + 1e-4 * np.abs(ref))


def test_split_terms_closed_form():
    """Depthwise output d = 1 + 2^-10 everywhere (centre tap 1 + 2^-10 on an all-ones image)
    and pointwise weights w = 1 + 2^-10: hi = 1 and lo = 2^-10 for both, so the three-term
    product is exactly 1 + 2^-9 (the dropped lo*lo term is 2^-20) and each output is
    C (1 + 2^-9), against C (1 + 2^-9 + 2^-20) exactly.  A plain bf16 product would give C."""
    torch = _torch()
    N, C, H, W, O = 1, 32, 6, 70, 16
    e = 2.0 ** -10
    x = torch.ones((N, C, H, W), device="cuda")
    dw = torch.zeros((C, 1, 3, 3), device="cuda")
    dw[:, 0, 1, 1] = 1.0 + e
    pw = torch.full((O, C, 1, 1), 1.0 + e, device="cuda")
    y = cf().dwsep_conv2d_split_bf16(x, dw, None, pw, None, 1, 1, 1)
    assert bool((y == C * (1.0 + 2 * e)).all()), y.unique()
    y32 = cf().dwsep_conv2d(x, dw, None, pw, None, 1, 1, 1)
    exact = C * (1.0 + 2 * e + e * e)
    assert float((y32 - exact).abs().max()) <= 1e-4 + 1e-4 * exact


class SplitTally:
    """Whole-output comparison against a split contract, accumulated over batch items."""

    def __init__(self, what):
        self.what, self.count, self.max_ratio = what, 0, 0.0

    def add(self, got, ref, abs_term, where):
        got = np.asarray(got, np.float64)
        assert got.shape == ref.shape == abs_term.shape, (where, got.shape, ref.shape)
        assert_split_close(got, ref, abs_term, "%s %s" % (self.what, where))
        bound = 1e-4 + 1e-4 * np.abs(ref) + SPLIT_SLACK * abs_term
        self.count += got.size
        self.max_ratio = max(self.max_ratio, float((np.abs(got - ref) / bound).max()))

    def report(self):
        PARITY_REPORT.append("%-44s %12d compared  max err/bound %.4f (split contract)" % (
            self.what, self.count, self.max_ratio))


@pytest.mark.parametrize("index", [10, 11])
def test_split_full_workload_every_output(index):
    """The dwsep split workloads at full size: every output against the split contract, one
    batch item at a time; the sum of |d[c] * pw[o,c]| comes from the oracle's depthwise
    output of the item."""
    torch = _torch()
    w = wl.WORKLOADS[index]
    inp = w.inputs()
    p = w.params
    args = (p["stride"], p["pad"], p["dilation"])
    y = cf().dwsep_conv2d_split_bf16(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]),
                                     dev(inp["pw_w"]), dev(inp["pw_b"]), *args)
    assert cf().last_kernel() == bench.kernel_name(w)
    dd = w.dims
    assert tuple(y.shape) == (dd["N"], dd["O"], dd["H"], dd["W"])
    assert bool(torch.isfinite(y).all())
    # the split kernel ran (its rounding differs from the fp32 kernel's) and is deterministic
    y32 = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                            dev(inp["pw_b"]), *args)
    assert not bool(torch.equal(y, y32))
    del y32
    y2 = cf().dwsep_conv2d_split_bf16(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]),
                                      dev(inp["pw_w"]), dev(inp["pw_b"]), *args)
    assert bool(torch.equal(y, y2))
    del y2
    host = y.cpu().numpy()
    del y
    torch.cuda.empty_cache()
    pw = np.abs(inp["pw_w"][:, :, 0, 0].astype(np.float64))
    t = SplitTally("split workload %d %s" % (index, w.name))
    for n in range(dd["N"]):
        item = dict(inp, x=inp["x"][n:n + 1])
        ref = oracle.dwsep_conv2d(item["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"],
                                  *args)
        d = np.abs(depthwise_exact(item, *args)[0]).reshape(dd["C"], -1)
        abs_dot = (pw @ d).reshape(ref.shape)
        t.add(host[n:n + 1], ref, abs_dot, "batch item %d" % n)
    assert t.count == host.size
    t.report()


def test_split_not_written_past_end():
    torch = _torch()
    inp = wl.dwsep_inputs(791, 1, 5, 7, 21, 19, bias=True)
    n_out = 19 * 7 * 21
    buf = torch.full((n_out + 4096,), 12345.0, device="cuda")
    y = buf[:n_out].view(1, 19, 7, 21)
    cf().dwsep_conv2d_split_bf16(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]),
                                 dev(inp["pw_w"]), dev(inp["pw_b"]), 1, 1, 1, out=y)
    assert bool((buf[n_out:] == 12345.0).all())


CONV_SPLIT_CASES = [
    # (N, C, D, H, W, O, pad, bias)
    (1, 8, 6, 9, 20, 16, 0, True),      # one chunk, one channel group
    (2, 5, 7, 9, 37, 19, 0, True),      # C below the 8-channel chunk, ragged columns
    (1, 13, 5, 6, 70, 40, 1, False),    # two chunks (ragged), two channel groups, pad 1
    (1, 32, 6, 7, 64, 64, 2, True),     # the layer's channel shape, pad 2
    (2, 3, 4, 4, 4, 7, 2, True),        # output larger than input
]


def conv_abs_sum(inp, pad):
    return oracle.conv3d(np.abs(inp["x"]), np.abs(inp["w"]), None, 1, pad)


@pytest.mark.parametrize("case", CONV_SPLIT_CASES)
def test_conv3d_split_small(case):
    N, C, D, H, W, O, pad, bias = case
    inp = wl.conv3d_act_inputs(720 + sum(case), N, C, D, H, W, O, bias=bias)
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"], 1, pad)
    bound_extra = (2.0 ** -13 / SPLIT_SLACK) * conv_abs_sum(inp, pad)
    y = cf().conv3d_mish_tanh_split_bf16(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), 1, pad)
    assert tuple(y.shape) == ref.shape
    assert_split_close(y.cpu().numpy(), ref, bound_extra, "conv3d split %s" % (case,))


def test_conv3d_split_general_parameters_run_fp32():
    inp = wl.conv3d_act_inputs(790, 1, 4, 9, 10, 21, 8, k=5)
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"], 2, 2)
    y = cf().conv3d_mish_tanh_split_bf16(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), 2, 2)
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-4 + 1e-4 * np.abs(ref))


def test_conv3d_split_full_workload_every_output():
    """The Conv3d split workload at full size: every output against the split contract, one
    batch item at a time; sum |x * w| is the oracle's Conv3d of |x| and |w| for the item."""
    torch = _torch()
    w = wl.WORKLOADS[12]
    inp = w.inputs()
    p = w.params
    y = cf().conv3d_mish_tanh_split_bf16(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]),
                                         p["stride"], p["pad"])
    assert cf().last_kernel() == bench.kernel_name(w)
    assert tuple(y.shape) == (16, 64, 30, 62, 62)
    assert bool(torch.isfinite(y).all())
    y32 = cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), p["stride"], p["pad"])
    assert not bool(torch.equal(y, y32))
    del y32
    y2 = cf().conv3d_mish_tanh_split_bf16(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]),
                                          p["stride"], p["pad"])
    assert bool(torch.equal(y, y2))
    del y2
    host = y.cpu().numpy()
    del y
    torch.cuda.empty_cache()
    aw = np.abs(inp["w"])
    t = SplitTally("split workload 12 %s" % w.name)
    for n in range(host.shape[0]):
        xn = inp["x"][n:n + 1]
        ref = oracle.conv3d_mish_tanh(xn, inp["w"], inp["b"], p["stride"], p["pad"])
        extra = oracle.conv3d(np.abs(xn), aw, None, p["stride"], p["pad"])
        t.add(host[n:n + 1], ref, (2.0 ** -13 / SPLIT_SLACK) * extra, "batch item %d" % n)
    assert t.count == host.size
    t.report()


POOL_SPLIT_CASES = [
    # (N, C, D, H, W, O, divisor, conv_bias)
    (2, 8, 8, 12, 20, 16, 2.0, True),     # one chunk, one channel group
    (1, 13, 9, 21, 40, 20, -1.5, True),   # two chunks (ragged), two groups, negative divisor
    (3, 4, 6, 6, 37, 5, 0.75, False),     # ragged pooled rows and columns, few channels
]


def pool_split_bound(inp, ref, divisor):
    """1e-4 |ref| + 2^-14 * sum_o (largest sum |x*w| over the pooled voxels) / |divisor|."""
    s = oracle.conv3d(np.abs(inp["x"]), np.abs(inp["w"]), None, 1, 0)
    PD, PH, PW = (n // 2 for n in s.shape[2:])
    m = s[:, :, :2 * PD, :2 * PH, :2 * PW].reshape(s.shape[0], s.shape[1], -1).max(axis=2)
    return 1e-4 * np.abs(ref) + 2.0 ** -14 * m.sum(axis=1) / abs(divisor)


@pytest.mark.parametrize("case", POOL_SPLIT_CASES)
def test_pool_split_small(case):
    N, C, D, H, W, O, div, cbias = case
    inp = wl.conv3d_pool_inputs(740 + int(sum(case)), N, C, D, H, W, O, conv_bias=cbias)
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(inp["x"], inp["w"], inp["conv_b"], div, 2,
                                                 inp["bias"])
    out = cf().conv3d_div_maxpool_gap_bias_sum_split_bf16(dev(inp["x"]), dev(inp["w"]),
                                                          dev(inp["conv_b"]), div, 2,
                                                          dev(inp["bias"]))
    got = out.cpu().numpy().astype(np.float64)
    bound = pool_split_bound(inp, ref, div)
    assert np.all(np.abs(got - ref) <= bound), (case, got, ref, bound)


def test_pool_split_full_workload_every_scalar():
    """The pooled-sum split workload at full size: all 128 scalars against the split bound."""
    w = wl.WORKLOADS[13]
    inp = w.inputs()
    p = w.params
    out = cf().conv3d_div_maxpool_gap_bias_sum_split_bf16(dev(inp["x"]), dev(inp["w"]),
                                                          dev(inp["conv_b"]), p["divisor"],
                                                          p["pool"], dev(inp["bias"]))
    assert cf().last_kernel() == bench.kernel_name(w)
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(inp["x"], inp["w"], inp["conv_b"],
                                                 p["divisor"], p["pool"], inp["bias"])
    bound = pool_split_bound(inp, ref, p["divisor"])
    err = np.abs(got - ref)
    assert np.all(err <= bound), [(int(i), got[i], ref[i], bound[i])
                                  for i in np.nonzero(err > bound)[0][:8]]
    PARITY_REPORT.append("%-44s %12d compared  max err/bound %.4f (split contract)" % (
        "split workload 13 %s" % w.name, got.size, float((err / bound).max())))
    torch = _torch()
    assert bool(torch.isfinite(out).all())
    out32 = cf().conv3d_div_maxpool_gap_bias_sum(dev(inp["x"]), dev(inp["w"]), dev(inp["conv_b"]),
                                                 p["divisor"], p["pool"], dev(inp["bias"]))
    assert not bool(torch.equal(out, out32))

"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the same
seeded inputs.

Tolerances:
  * conv3d_mish_tanh and dwsep_conv2d: |gpu - ref| <= 1e-4 + 1e-4 * |ref| elementwise;
  * conv3d_div_maxpool_gap_bias_sum: |gpu - ref| <= 1e-4 * |ref| per batch scalar.
Small cases (several tiles, ragged tails, padding, odd channel counts, saturation) are
compared over the whole output; the full-size configurations are compared over their whole
output in test_gpu_full_parity.py."""
import numpy as np
import pytest

import oracle
from implicit_gemm_convolution_conv3d_amd import workloads as wl

pytestmark = pytest.mark.gpu

ATOL = RTOL = 1e-4
POOL_RTOL = 1e-4


def _torch():
    import torch
    return torch


def dev(a):
    if a is None:
        return None
    return _torch().from_numpy(np.ascontiguousarray(a)).to("cuda")


def cf():
    import implicit_gemm_convolution_conv3d_amd as m
    return m


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    assert not bad.any(), "%s: %d/%d outside tolerance; worst err %.3g at ref %.6g" % (
        what, bad.sum(), bad.size, err.max(), ref.reshape(-1)[np.argmax(err)])


def edge_indices(shape, rng, count):
    """Flat indices: random ones plus every combination of first/last along each axis."""
    total = int(np.prod(shape))
    idx = [rng.integers(0, total, count)]
    corners = np.array(np.meshgrid(*[[0, s - 1] for s in shape], indexing="ij")).reshape(len(shape), -1)
    idx.append(np.ravel_multi_index(corners, shape))
    return np.unique(np.concatenate(idx))


def gather(y, idx):
    torch = _torch()
    t = torch.from_numpy(idx).to(y.device)
    return y.reshape(-1)[t].cpu().numpy()


# ----------------------------------------------------------------- conv3d + mish + tanh
ACT_CASES = [
    # (N, C, D, H, W, O, pad, bias)
    (1, 4, 8, 16, 16, 8, 0, True),        # the tiny workload's shape
    (2, 5, 7, 9, 37, 19, 0, True),         # Cin % 4 != 0, Cout % 16 != 0, ragged W tile
    (1, 32, 6, 9, 70, 64, 0, True),        # several W tiles, odd H, full channel group
    (1, 8, 5, 6, 20, 80, 1, False),        # two channel groups, padding 1, no bias
    (2, 3, 4, 4, 4, 16, 2, True),          # padding 2, output larger than input
    (1, 4, 3, 3, 3, 3, 0, True),           # single output voxel
    (1, 8, 5, 6, 133, 32, 1, True),        # rows 4-byte aligned only, three W tiles
]


@pytest.mark.parametrize("case", ACT_CASES)
def test_conv3d_mish_tanh_small(case):
    N, C, D, H, W, O, pad, bias = case
    inp = wl.conv3d_act_inputs(100 + sum(case), N, C, D, H, W, O, bias=bias)
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"], 1, pad)
    y = cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), 1, pad)
    _torch().cuda.synchronize()
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "conv3d_mish_tanh %s" % (case,))


def test_conv3d_mish_tanh_tiny_workload_full():
    w1 = wl.WORKLOADS[1]
    inp = w1.inputs()
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"])
    y = cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]))
    assert tuple(y.shape) == (1, 8, 6, 14, 14)
    assert_close(y.cpu().numpy(), ref, "workload 1")


def test_conv3d_mish_tanh_saturation_paths():
    """Pre-activations far beyond the softplus threshold and deep in the negative tail."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 4, 6, 6, 20)).astype(np.float32)
    w = rng.uniform(-0.2, 0.2, (16, 4, 3, 3, 3)).astype(np.float32)
    b = np.array([30, -30, 200, -200, 20, -20, 21, 19, 0, 1, -1, 5, -5, 88, -88, 10],
                 np.float32)
    ref = oracle.conv3d_mish_tanh(x, w, b)
    y = cf().conv3d_mish_tanh(dev(x), dev(w), dev(b)).cpu().numpy()
    assert_close(y, ref, "saturation")


# ----------------------------------------------------------------- conv3d + pool + sum
POOL_CASES = [
    # (N, C, D, H, W, O, divisor, conv_bias)
    (3, 8, 6, 10, 12, 16, 2.0, True),
    (2, 5, 9, 11, 70, 21, 2.0, True),      # odd conv output (floor mode drops a plane/row/col)
    (2, 4, 4, 20, 36, 16, -2.0, True),     # negative divisor: max becomes min
    (1, 3, 5, 5, 5, 7, 3.0, False),        # single window, non power-of-two divisor
    (4, 8, 16, 30, 64, 16, 2.0, True),     # several ph groups, full-width rows
]


@pytest.mark.parametrize("case", POOL_CASES)
def test_pool_small(case):
    N, C, D, H, W, O, div, cbias = case
    inp = wl.conv3d_pool_inputs(200 + int(sum(case)), N, C, D, H, W, O, conv_bias=cbias)
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(inp["x"], inp["w"], inp["conv_b"], div, 2,
                                                 inp["bias"])
    out = cf().conv3d_div_maxpool_gap_bias_sum(dev(inp["x"]), dev(inp["w"]), dev(inp["conv_b"]),
                                               div, 2, dev(inp["bias"]))
    got = out.cpu().numpy().astype(np.float64)
    rel = np.abs(got - ref) / np.abs(ref)
    assert rel.max() <= POOL_RTOL, (case, got, ref)


# ----------------------------------------------------------------- conv3d + pool (tensor)
MAXPOOL_CASES = [
    # (N, C, D, H, W, O, k, pool, divisor, conv_bias)
    (3, 8, 6, 10, 12, 16, 3, 2, 2.0, True),     # tuned kernel
    (2, 5, 9, 11, 70, 21, 3, 2, 2.0, True),     # floor mode, two channel groups, ragged W
    (2, 4, 4, 20, 36, 16, 3, 2, -2.0, True),    # negative divisor
    (1, 3, 5, 5, 5, 7, 3, 2, 3.0, False),       # single window
    (2, 4, 8, 9, 21, 16, 3, 3, 2.0, True),      # general kernel: pool 3
    (1, 3, 9, 9, 40, 7, 5, 2, -1.5, True),      # general kernel: k = 5
]


@pytest.mark.parametrize("case", MAXPOOL_CASES)
def test_maxpool_tensor_small(case):
    N, C, D, H, W, O, k, pool, div, cbias = case
    inp = wl.conv3d_pool_inputs(700 + int(sum(case)), N, C, D, H, W, O, k=k, conv_bias=cbias)
    ref = oracle.conv3d_div_maxpool(inp["x"], inp["w"], inp["conv_b"], div, pool)
    y = cf().conv3d_div_maxpool(dev(inp["x"]), dev(inp["w"]), dev(inp["conv_b"]), div, pool)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "conv3d_div_maxpool %s" % (case,))


# ----------------------------------------------------------------- depthwise-separable
DW_CASES = [
    # (N, C, H, W, O, pad, bias)
    (2, 8, 13, 70, 16, 1, False),          # ragged W and H tiles
    (1, 20, 9, 33, 40, 1, True),           # Cin % 16 != 0, Cout % 16 != 0
    (1, 64, 17, 64, 128, 1, False),        # the 512^2 workload's channel shape
    (1, 96, 7, 45, 192, 1, True),          # the odd workload's channel shape
    (2, 4, 6, 20, 200, 2, True),           # padding 2, two channel groups
    (1, 4, 5, 19, 8, 0, False),            # no padding
    (1, 3, 1, 1, 5, 1, True),              # 1x1 image
    # wider layers: weights near the LDS limit of the 32-channel-chunk persistent kernel
    # (Cin 97-128) and the 16-channel-chunk persistent kernel (Cin 129-192)
    (1, 100, 7, 37, 100, 1, True),         # 128-channel group, unaligned rows
    (1, 110, 6, 40, 128, 1, False),        # the same, aligned rows
    (1, 150, 6, 36, 128, 1, True),         # 16-channel chunks, aligned rows
    (1, 120, 5, 21, 150, 1, True),         # 192-channel group, unaligned rows
    (1, 140, 5, 24, 192, 1, False),        # 192-channel group, 16-channel chunks
    (1, 200, 9, 44, 40, 1, True),          # 64-channel group, near the LDS limit
    (1, 300, 5, 27, 64, 1, False),         # 64-channel group, 16-channel chunks
]


@pytest.mark.parametrize("case", DW_CASES)
def test_dwsep_small(case):
    N, C, H, W, O, pad, bias = case
    inp = wl.dwsep_inputs(300 + sum(case), N, C, H, W, O, bias=bias)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], 1,
                              pad, 1)
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                          dev(inp["pw_b"]), 1, pad, 1)
    assert tuple(y.shape) == ref.shape
    assert_close(y.cpu().numpy(), ref, "dwsep %s" % (case,))


def test_outputs_not_written_past_their_end():
    """A guard band after y stays untouched for ragged shapes."""
    torch = _torch()
    inp = wl.dwsep_inputs(7, 1, 5, 7, 21, 19, bias=True)
    n_out = 1 * 19 * 7 * 21
    buf = torch.full((n_out + 4096,), 12345.0, device="cuda")
    y = buf[:n_out].view(1, 19, 7, 21)
    cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                      dev(inp["pw_b"]), 1, 1, 1, out=y)
    assert bool((buf[n_out:] == 12345.0).all())
    inp = wl.conv3d_act_inputs(8, 1, 3, 5, 6, 23, 7)
    n_out = 7 * 3 * 4 * 21
    buf = torch.full((n_out + 4096,), 12345.0, device="cuda")
    y = buf[:n_out].view(1, 7, 3, 4, 21)
    cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), out=y)
    assert bool((buf[n_out:] == 12345.0).all())
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"])
    assert_close(y.cpu().numpy(), ref, "guarded conv3d")


def test_empty_batch():
    torch = _torch()
    x = torch.empty((0, 4, 8, 8, 8), device="cuda")
    w = torch.zeros((8, 4, 3, 3, 3), device="cuda")
    assert tuple(cf().conv3d_mish_tanh(x, w).shape) == (0, 8, 6, 6, 6)

"""GPU parity of the kernel variants that only large or unusual shapes select, against the fp64
CPU oracle through the C ABI: the Conv3d kernels' plain-load staging (a chunk of input
channels above 2^31 bytes), the chunked depthwise-separable kernel (pointwise weights too
large for LDS, or an image above 2^31 bytes), the general kernels' direct fallbacks (kernel
size above 7, a chunk beyond 32-bit offsets), the split-bf16 mode's fp32 fallback, and guard
bands after outputs written by the float2 / float4 row epilogues.  Same tolerances as the
other parity tests."""
import numpy as np
import pytest

import oracle
from implicit_gemm_convolution_conv3d_amd import workloads as wl

from test_gpu_parity import POOL_RTOL, assert_close, cf, dev, edge_indices, gather

pytestmark = pytest.mark.gpu


def test_conv3d_plain_load_staging():
    """One image of 512 x 512 x 513 voxels: four channels of it exceed 2^31 bytes, so the
    tuned kernel stages through plain loads; sampled outputs and every corner."""
    inp = wl.conv3d_act_inputs(901, 1, 1, 512, 512, 513, 5)
    y = cf().conv3d_mish_tanh(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]))
    assert tuple(y.shape) == (1, 5, 510, 510, 511)
    idx = edge_indices(y.shape, np.random.default_rng(5), 4000)
    ref = oracle.conv3d_mish_tanh_at(inp["x"], inp["w"], inp["b"], idx)
    assert_close(gather(y, idx), ref, "conv3d plain-load staging")


def test_pool_plain_load_staging():
    inp = wl.conv3d_pool_inputs(902, 1, 1, 512, 512, 513, 3)
    out = cf().conv3d_div_maxpool_gap_bias_sum(dev(inp["x"]), dev(inp["w"]), dev(inp["conv_b"]),
                                               2.0, 2, dev(inp["bias"]))
    ref = oracle.conv3d_div_maxpool_gap_bias_sum(inp["x"], inp["w"], inp["conv_b"], 2.0, 2,
                                                 inp["bias"])
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= POOL_RTOL * np.abs(ref)), (got, ref)


CHUNKED_CASES = [
    # (N, C, H, W, O, bias): 520 input channels, pointwise weights above the LDS size
    (1, 520, 9, 70, 40, True),      # unaligned rows (scalar staging loads)
    (2, 520, 6, 72, 24, False),     # aligned rows (float4 staging loads)
    (1, 516, 5, 33, 150, True),     # three output-channel groups
]


@pytest.mark.parametrize("case", CHUNKED_CASES)
def test_dwsep_chunked(case):
    N, C, H, W, O, bias = case
    inp = wl.dwsep_inputs(910 + sum(case), N, C, H, W, O, bias=bias)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"])
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                          dev(inp["pw_b"]))
    assert_close(y.cpu().numpy(), ref, "dwsep chunked %s" % (case,))
    # the split-bf16 mode falls back to the same fp32 kernels here
    y2 = cf().dwsep_conv2d_split_bf16(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]),
                                      dev(inp["pw_w"]), dev(inp["pw_b"]))
    assert bool((y2 == y).all())


def test_pointwise_chunked():
    inp = wl.dwsep_inputs(920, 1, 520, 7, 40, 36, K=1, bias=True)
    eye_dw = np.ones((520, 1, 1, 1), np.float32)
    ref = oracle.dwsep_conv2d(inp["x"], eye_dw, None, inp["pw_w"], inp["pw_b"], 1, 0, 1)
    y = cf().pointwise_conv2d(dev(inp["x"]), dev(inp["pw_w"]), dev(inp["pw_b"]))
    assert_close(y.cpu().numpy(), ref, "pointwise chunked")


def test_dwsep_large_image():
    """64 channels of 2048 x 4100 pixels: the image exceeds 2^31 bytes, so the persistent
    kernel's 32-bit offsets do not apply and the chunked kernel runs; sampled outputs."""
    inp = wl.dwsep_inputs(921, 1, 64, 2048, 4100, 16, bias=True)
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                          dev(inp["pw_b"]))
    idx = edge_indices(y.shape, np.random.default_rng(6), 4000)
    ref = oracle.dwsep_conv2d_at(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], idx)
    assert_close(gather(y, idx), ref, "dwsep large image")


def test_dwsep_image_at_offset_limit():
    """64 channels of 2048 x 4095 pixels: 2 146 959 360 bytes, just inside the 32-bit buffer
    range, so the persistent kernel runs; its rows are only 4-byte aligned, so it stages with
    16-byte loads inside each row and single loads where the row ends, up to the last row of
    the range; sampled outputs and every corner."""
    inp = wl.dwsep_inputs(922, 1, 64, 2048, 4095, 16, bias=True)
    assert 4 * inp["x"].size < 2 ** 31 - 1
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                          dev(inp["pw_b"]))
    idx = edge_indices(y.shape, np.random.default_rng(7), 4000)
    # every output channel at the last 2 rows x 32 columns, which read the end of the range
    o, h, w = np.meshgrid(np.arange(16), [2046, 2047], np.arange(4063, 4095), indexing="ij")
    tail = np.ravel_multi_index((o.ravel(), h.ravel(), w.ravel()), (16, 2048, 4095))
    idx = np.unique(np.concatenate([idx, tail]))
    ref = oracle.dwsep_conv2d_at(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], idx)
    assert_close(gather(y, idx), ref, "dwsep image at the offset limit")


def test_dwsep_general_direct_fallbacks():
    # kernel size 9: above the staged kernel's 7
    inp = wl.dwsep_inputs(922, 1, 6, 20, 30, 10, K=9, bias=True)
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], 1, 4, 1)
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                          dev(inp["pw_b"]), 1, 4, 1)
    assert_close(y.cpu().numpy(), ref, "dwsep K9")
    # K = 5 on an 8192 x 8200 single-channel image: an 8-channel chunk exceeds 32-bit offsets
    inp = wl.dwsep_inputs(923, 1, 1, 8192, 8200, 3, K=5, bias=False)
    y = cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), None, dev(inp["pw_w"]), None, 2, 2, 1)
    assert tuple(y.shape) == (1, 3, 4096, 4100)
    idx = edge_indices(y.shape, np.random.default_rng(7), 3000)
    ref = oracle.dwsep_conv2d_at(inp["x"], inp["dw_w"], None, inp["pw_w"], None, idx, 2, 2, 1)
    assert_close(gather(y, idx), ref, "dwsep K5 s2 beyond 32-bit chunk offsets")


@pytest.mark.parametrize("entry,shape,k,stride,pad", [
    ("conv3d_mish_tanh", (1, 3, 5, 6, 16), 3, 1, 0),             # tuned, float2 rows, partial quad
    ("conv3d_mish_tanh", (1, 3, 5, 6, 22), 3, 1, 2),             # tuned, float4 rows (OW = 24)
    ("conv3d_mish_tanh", (1, 3, 9, 10, 26), 5, 2, 2),            # staged, OW = 13: single floats
    ("conv3d_mish_tanh", (1, 3, 9, 10, 32), 5, 1, 2),            # staged, float4 rows
    ("conv3d_mish_tanh_split_bf16", (1, 9, 5, 6, 16), 3, 1, 0),  # split, float2 rows
])
def test_conv3d_row_stores_stay_inside(entry, shape, k, stride, pad):
    """A guard band after y stays untouched by the vector-store row epilogues."""
    import torch
    N, C, D, H, W = shape
    O = 19
    inp = wl.conv3d_act_inputs(930 + W, N, C, D, H, W, O, k=k)
    od, oh, ow = ((s + 2 * pad - k) // stride + 1 for s in (D, H, W))
    n_out = N * O * od * oh * ow
    buf = torch.full((n_out + 4096,), 12345.0, device="cuda")
    y = buf[:n_out].view(N, O, od, oh, ow)
    getattr(cf(), entry)(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), stride, pad, out=y)
    assert bool((buf[n_out:] == 12345.0).all())
    ref = oracle.conv3d_mish_tanh(inp["x"], inp["w"], inp["b"], stride, pad)
    if entry == "conv3d_mish_tanh":
        assert_close(y.cpu().numpy(), ref, "guarded %s %s" % (entry, shape))
    else:
        assert np.all(np.abs(y.cpu().numpy() - ref) <= 1e-3)


def test_dwsep_staged_stores_stay_inside():
    import torch
    inp = wl.dwsep_inputs(940, 1, 6, 9, 35, 21, K=5, bias=True)
    ho, wo = 5, 18  # stride 2, pad 2
    n_out = 21 * ho * wo
    buf = torch.full((n_out + 4096,), 12345.0, device="cuda")
    y = buf[:n_out].view(1, 21, ho, wo)
    cf().dwsep_conv2d(dev(inp["x"]), dev(inp["dw_w"]), dev(inp["dw_b"]), dev(inp["pw_w"]),
                      dev(inp["pw_b"]), 2, 2, 1, out=y)
    assert bool((buf[n_out:] == 12345.0).all())
    ref = oracle.dwsep_conv2d(inp["x"], inp["dw_w"], inp["dw_b"], inp["pw_w"], inp["pw_b"], 2, 2, 1)
    assert_close(y.cpu().numpy(), ref, "guarded staged dwsep")

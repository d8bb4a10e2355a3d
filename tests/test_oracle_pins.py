"""Pins for the fp64 CPU oracle: checks against what the pages and the mathematics fix,
independent of the oracle's own code (closed forms, identities, the pages' printed
values, and numpy brute force on tiny inputs).  CPU only."""
import json
import math
import os

import numpy as np
import pytest
from numpy.lib.stride_tricks import sliding_window_view

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


# ---------------------------------------------------------------- numpy brute force
def np_conv3d(x, w, b=None, stride=1, pad=0):
    """Independent fp64 Conv3d: zero-pad, sliding windows, einsum."""
    x = x.astype(np.float64)
    w = w.astype(np.float64)
    k = w.shape[-1]
    xp = np.pad(x, ((0, 0), (0, 0), (pad, pad), (pad, pad), (pad, pad)))
    win = sliding_window_view(xp, (k, k, k), axis=(2, 3, 4))[:, :, ::stride, ::stride, ::stride]
    y = np.einsum("ncdhwijk,ocijk->nodhw", win, w)
    if b is not None:
        y = y + b.astype(np.float64)[None, :, None, None, None]
    return y


def np_dwsep(x, dw_w, dw_b, pw_w, pw_b, stride=1, pad=1, dil=1):
    x = x.astype(np.float64)
    K = dw_w.shape[-1]
    xp = np.pad(x, ((0, 0), (0, 0), (pad, pad), (pad, pad)))
    span = dil * (K - 1) + 1
    win = sliding_window_view(xp, (span, span), axis=(2, 3))[:, :, ::stride, ::stride, ::dil, ::dil]
    dw = np.einsum("nchwij,cij->nchw", win, dw_w[:, 0].astype(np.float64))
    if dw_b is not None:
        dw = dw + dw_b.astype(np.float64)[None, :, None, None]
    y = np.einsum("oc,nchw->nohw", pw_w[:, :, 0, 0].astype(np.float64), dw)
    if pw_b is not None:
        y = y + pw_b.astype(np.float64)[None, :, None, None]
    return y


def mish_tanh_closed_form(v):
    """tanh(v * tanh(ln(1+e^v))) via tanh(ln u) = (u^2-1)/(u^2+1), u = 1+e^v (pure Python)."""
    if v > 20.0:
        t = 1.0 - 2.0 / (math.exp(2 * v) + 1.0) if v < 300 else 1.0
        m = v * t
    else:
        u = 1.0 + math.exp(v)
        m = v * (u * u - 1.0) / (u * u + 1.0)
    e = math.exp(2 * m)
    return (e - 1.0) / (e + 1.0)


rng = np.random.default_rng(7)


# ---------------------------------------------------------------- shapes (page values)
def test_shapes_match_pages():
    g = GOLDEN["conv3d_mish_tanh_output_shape"]["value"]
    assert [oracle.out_len(n, 3) for n in g["input"][2:]] == g["output"][2:]
    g2 = GOLDEN["pool_conv_output_shape"]["value"]
    conv = [oracle.out_len(n, 3) for n in g2["input"][2:]]
    assert conv == g2["conv_output"][2:]
    pooled = [oracle.out_len(n, 2, 2) for n in conv]
    assert pooled == GOLDEN["pool_pooled_shape"]["value"][2:]
    assert int(np.prod(pooled)) == GOLDEN["pool_pooled_count"]["value"]
    g3 = GOLDEN["dwsep_output_shape"]["value"]
    assert [oracle.out_len(n, 3, 1, 1, 1) for n in g3["input"][2:]] == g3["output"][2:]
    # The odd workload keeps its size at pad 1.
    assert oracle.out_len(333, 3, 1, 1, 1) == 333 and oracle.out_len(517, 3, 1, 1, 1) == 517


def test_page_counts():
    g = GOLDEN["conv3d_mish_tanh_output_shape"]["value"]["output"]
    assert int(np.prod(g)) == GOLDEN["conv3d_mish_tanh_output_elements"]["value"]
    assert 32 * 27 == GOLDEN["conv3d_mish_tanh_macs_per_output"]["value"]
    conv = GOLDEN["pool_conv_output_shape"]["value"]["conv_output"]
    assert int(np.prod(conv)) * 8 * 27 == GOLDEN["pool_conv_macs"]["value"]


# ---------------------------------------------------------------- (a) conv3d + mish + tanh
@pytest.mark.parametrize("stride,pad", [(1, 0), (2, 1), (1, 2), (3, 0)])
def test_conv3d_matches_numpy(stride, pad):
    x = rng.standard_normal((2, 3, 7, 6, 9)).astype(np.float32)
    w = rng.uniform(-1, 1, (4, 3, 3, 3, 3)).astype(np.float32)
    b = rng.uniform(-1, 1, 4).astype(np.float32)
    ref = np_conv3d(x, w, b, stride, pad)
    got = oracle.conv3d(x, w, b, stride, pad)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_conv3d_delta_kernel_is_shift():
    """w[o] = e_(c0,kd0,kh0,kw0), b = 0 gives x[n,c0] shifted by (kd0,kh0,kw0), exactly."""
    x = rng.standard_normal((2, 3, 6, 7, 8)).astype(np.float32)
    taps = [(0, 0, 0, 0), (1, 2, 0, 1), (2, 1, 2, 2), (0, 0, 1, 2)]
    w = np.zeros((len(taps), 3, 3, 3, 3), np.float32)
    for o, (c, a, bb, cc) in enumerate(taps):
        w[o, c, a, bb, cc] = 1.0
    y = oracle.conv3d(x, w, None)
    for o, (c, a, bb, cc) in enumerate(taps):
        np.testing.assert_array_equal(y[:, o], x[:, c, a:a + 4, bb:bb + 5, cc:cc + 6])


def test_conv3d_padding_reads_zero():
    """With pad 1 and a corner delta, the first output plane reads the zero border."""
    x = rng.standard_normal((1, 1, 4, 4, 4)).astype(np.float32)
    w = np.zeros((1, 1, 3, 3, 3), np.float32)
    w[0, 0, 0, 0, 0] = 1.0
    y = oracle.conv3d(x, w, None, 1, 1)
    assert y.shape == (1, 1, 4, 4, 4)
    assert np.all(y[0, 0, 0] == 0) and np.all(y[0, 0, :, 0] == 0) and np.all(y[0, 0, :, :, 0] == 0)
    np.testing.assert_array_equal(y[0, 0, 1:, 1:, 1:], x[0, 0, :3, :3, :3])


def test_conv3d_linearity():
    x1 = rng.standard_normal((1, 2, 5, 5, 5)).astype(np.float32)
    x2 = rng.standard_normal((1, 2, 5, 5, 5)).astype(np.float32)
    w = rng.uniform(-1, 1, (3, 2, 3, 3, 3)).astype(np.float32)
    s = (x1.astype(np.float64) + x2).astype(np.float32)
    # fp32 rounding of the sum is the only difference; compare with the exact fp64 sum.
    lhs = oracle.conv3d(x1, w) + oracle.conv3d(x2, w)
    rhs = np_conv3d(x1.astype(np.float64) + x2.astype(np.float64), w)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    assert np.abs(oracle.conv3d(s, w) - lhs).max() < 1e-5


def test_mish_tanh_zero_and_limits():
    x = rng.standard_normal((1, 2, 5, 5, 5)).astype(np.float32)
    w = np.zeros((3, 2, 3, 3, 3), np.float32)
    y = oracle.conv3d_mish_tanh(x, w, np.zeros(3, np.float32))
    assert np.all(y == 0.0)  # mish(0) = 0, tanh(0) = 0
    y = oracle.conv3d_mish_tanh(x, w, np.array([30.0, -200.0, 21.0], np.float32))
    assert np.all(y[:, 0] == 1.0)               # overflow side: tanh(30) rounds to 1
    assert np.all(np.abs(y[:, 1]) < 1e-80)      # underflow side: mish(-200) ~ -200*e^-200
    np.testing.assert_allclose(y[:, 2], math.tanh(21.0 * math.tanh(21.0)), rtol=1e-15)


def test_mish_tanh_closed_form_and_range():
    v = np.concatenate([np.linspace(-30, 30, 2001), [-1.1924312, 0.0, 19.999, 20.0, 20.001]])
    got = oracle.mish_tanh(v)
    ref = np.array([mish_tanh_closed_form(t) for t in v])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    # min of mish is -0.3088434 at v = -1.1924312; tanh of it bounds y from below.
    ymin = math.tanh(-0.30884340)
    assert got.min() >= ymin - 1e-7 and got.max() <= 1.0
    assert abs(oracle.mish_tanh(np.array([-1.1924312]))[0] - ymin) < 1e-7


def test_mish_tanh_sampled_matches_full():
    x = rng.standard_normal((2, 3, 6, 7, 8)).astype(np.float32)
    w = rng.uniform(-0.3, 0.3, (5, 3, 3, 3, 3)).astype(np.float32)
    b = rng.uniform(-0.3, 0.3, 5).astype(np.float32)
    full = oracle.conv3d_mish_tanh(x, w, b)
    idx = rng.choice(full.size, 200, replace=False)
    np.testing.assert_array_equal(oracle.conv3d_mish_tanh_at(x, w, b, idx), full.reshape(-1)[idx])
    ref = np.vectorize(mish_tanh_closed_form)(np_conv3d(x, w, b))
    np.testing.assert_allclose(full, ref, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- (b) conv3d + pool + sum
def np_pool_definitional(x, w, cb, divisor, pool, bias):
    co = np_conv3d(x, w, cb) / divisor
    N, O, OD, OH, OW = co.shape
    PD, PH, PW = OD // pool, OH // pool, OW // pool
    c = co[:, :, :PD * pool, :PH * pool, :PW * pool]
    c = c.reshape(N, O, PD, pool, PH, pool, PW, pool)
    mp = c.max(axis=(3, 5, 7))
    g = mp.mean(axis=(2, 3, 4)) + bias.reshape(-1).astype(np.float64)[None]
    return g.sum(axis=1)


def np_pool_rewrite(x, w, cb, pool, bias):
    """Page l2_p8 rewrite: out[n] = S[n]/(2*count) + sum_c bias[c], S = sum of window maxima
    of the undivided conv (+ conv bias); valid only for divisor 2."""
    co = np_conv3d(x, w, cb)
    N, O, OD, OH, OW = co.shape
    PD, PH, PW = OD // pool, OH // pool, OW // pool
    c = co[:, :, :PD * pool, :PH * pool, :PW * pool].reshape(N, O, PD, pool, PH, pool, PW, pool)
    S = c.max(axis=(3, 5, 7)).sum(axis=(1, 2, 3, 4))
    return S / (2.0 * PD * PH * PW) + bias.astype(np.float64).sum()


@pytest.mark.parametrize("shape", [(2, 3, 8, 10, 12), (1, 2, 9, 7, 11), (3, 4, 6, 6, 6)])
def test_pool_rewrite_and_definition(shape):
    N, C, D, H, W = shape
    x = rng.standard_normal(shape).astype(np.float32)
    w = rng.uniform(-0.3, 0.3, (5, C, 3, 3, 3)).astype(np.float32)
    cb = rng.uniform(-0.3, 0.3, 5).astype(np.float32)
    bias = rng.standard_normal((5, 1, 1, 1)).astype(np.float32)
    got = oracle.conv3d_div_maxpool_gap_bias_sum(x, w, cb, 2.0, 2, bias)
    np.testing.assert_allclose(got, np_pool_rewrite(x, w, cb, 2, bias), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, np_pool_definitional(x, w, cb, 2.0, 2, bias), rtol=1e-12,
                               atol=1e-12)


def test_pool_divides_before_max():
    """A negative divisor turns max into min: only the definitional order gets it right."""
    x = rng.standard_normal((2, 2, 6, 6, 6)).astype(np.float32)
    w = rng.uniform(-0.3, 0.3, (3, 2, 3, 3, 3)).astype(np.float32)
    cb = rng.uniform(-0.3, 0.3, 3).astype(np.float32)
    bias = rng.standard_normal(3).astype(np.float32)
    got = oracle.conv3d_div_maxpool_gap_bias_sum(x, w, cb, -2.0, 2, bias)
    np.testing.assert_allclose(got, np_pool_definitional(x, w, cb, -2.0, 2, bias), rtol=1e-12)
    swapped = -np_pool_rewrite(x, w, cb, 2, np.zeros(3, np.float32)) + bias.astype(np.float64).sum()
    assert np.abs(got - swapped).min() > 1e-3


def test_pool_closed_forms():
    x = rng.standard_normal((2, 2, 8, 8, 8)).astype(np.float32)
    cb = np.array([0.25, -0.5, 0.125], np.float32)
    bias = np.array([1.0, 2.0, -4.0], np.float32)
    w0 = np.zeros((3, 2, 3, 3, 3), np.float32)
    got = oracle.conv3d_div_maxpool_gap_bias_sum(x, w0, cb, 2.0, 2, bias)
    np.testing.assert_allclose(got, cb.sum() / 2 + bias.sum(), rtol=1e-15)
    # constant input a: every conv output is a*sum(w[c]) + cb[c]
    a = 0.75
    xc = np.full((2, 2, 8, 8, 8), a, np.float32)
    w = rng.uniform(-0.3, 0.3, (3, 2, 3, 3, 3)).astype(np.float32)
    per_c = a * w.astype(np.float64).reshape(3, -1).sum(1) + cb
    got = oracle.conv3d_div_maxpool_gap_bias_sum(xc, w, cb, 2.0, 2, bias)
    np.testing.assert_allclose(got, (per_c / 2).sum() + bias.sum(), rtol=1e-13)


def test_pool_ramp_delta_floor_mode():
    """x = +-w ramp along W, delta kernel: window maxima sit at odd (or even) columns.
    W=13 gives a conv width 11 and floor-mode pooling keeps 5 windows."""
    N, C, D, H, W = 1, 1, 6, 6, 13
    ramp = np.broadcast_to(np.arange(W, dtype=np.float32), (N, C, D, H, W)).copy()
    w = np.zeros((2, 1, 3, 3, 3), np.float32)
    w[:, 0, 0, 0, 0] = 1.0
    bias = np.zeros(2, np.float32)
    PW = (W - 2) // 2
    got = oracle.conv3d_div_maxpool_gap_bias_sum(ramp, w, None, 2.0, 2, bias)
    # max over (2pw, 2pw+1) of ow is 2pw+1; mean over pw is PW; halved; two channels.
    np.testing.assert_allclose(got, 2 * PW / 2.0, rtol=1e-15)
    got = oracle.conv3d_div_maxpool_gap_bias_sum(-ramp, w, None, 2.0, 2, bias)
    np.testing.assert_allclose(got, 2 * (-(PW - 1)) / 2.0, rtol=1e-15)


def np_conv_div_maxpool(x, w, cb, divisor, pool):
    """Independent pooled tensor: numpy conv, + cb, / divisor, windows reshaped, max."""
    co = np_conv3d(x, w, cb) / divisor
    N, O, OD, OH, OW = co.shape
    PD, PH, PW = (OD - pool) // pool + 1, (OH - pool) // pool + 1, (OW - pool) // pool + 1
    c = co[:, :, :PD * pool, :PH * pool, :PW * pool]
    return c.reshape(N, O, PD, pool, PH, pool, PW, pool).max(axis=(3, 5, 7))


@pytest.mark.parametrize("shape,k,pool,div", [((2, 3, 8, 10, 12), 3, 2, 2.0),
                                              ((1, 2, 9, 7, 11), 3, 2, -2.0),
                                              ((2, 2, 11, 10, 13), 3, 3, 0.5),
                                              ((1, 3, 7, 8, 9), 1, 4, 3.0),
                                              ((1, 2, 10, 9, 12), 5, 2, 2.0)])
def test_pooled_tensor_matches_numpy(shape, k, pool, div):
    N, C, D, H, W = shape
    x = rng.standard_normal(shape).astype(np.float32)
    w = rng.uniform(-0.3, 0.3, (5, C, k, k, k)).astype(np.float32)
    cb = rng.uniform(-0.3, 0.3, 5).astype(np.float32)
    got = oracle.conv3d_div_maxpool(x, w, cb, div, pool)
    ref = np_conv_div_maxpool(x, w, cb, div, pool)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_pooled_tensor_ramp_closed_form():
    """Delta kernel on a ramp along W: window maxima are the odd columns (2pw+1), halved;
    floor mode keeps (W-2)//2 windows of the 11-wide conv output."""
    N, C, D, H, W = 1, 1, 6, 6, 13
    ramp = np.broadcast_to(np.arange(W, dtype=np.float32), (N, C, D, H, W)).copy()
    w = np.zeros((2, 1, 3, 3, 3), np.float32)
    w[:, 0, 0, 0, 0] = 1.0
    got = oracle.conv3d_div_maxpool(ramp, w, None, 2.0, 2)
    PW = (W - 2) // 2
    assert got.shape == (1, 2, 2, 2, PW)
    np.testing.assert_array_equal(got, np.broadcast_to((2 * np.arange(PW) + 1) / 2.0, got.shape))


def test_pooled_tensor_reduces_to_pooled_sum():
    """Channel sum of (mean of the pooled tensor + bias) is the fused pooled-sum output."""
    x = rng.standard_normal((3, 2, 7, 9, 10)).astype(np.float32)
    w = rng.uniform(-0.3, 0.3, (4, 2, 3, 3, 3)).astype(np.float32)
    cb = rng.uniform(-0.3, 0.3, 4).astype(np.float32)
    bias = rng.standard_normal(4).astype(np.float32)
    mp = oracle.conv3d_div_maxpool(x, w, cb, 2.0, 2)
    via = (mp.mean(axis=(2, 3, 4)) + bias.astype(np.float64)[None]).sum(axis=1)
    np.testing.assert_allclose(oracle.conv3d_div_maxpool_gap_bias_sum(x, w, cb, 2.0, 2, bias),
                               via, rtol=1e-13)


# ---------------------------------------------------------------- (c) depthwise-separable
@pytest.mark.parametrize("K,stride,pad,dil,bias", [(3, 1, 1, 1, False), (3, 1, 1, 1, True),
                                                   (3, 2, 1, 1, True), (5, 1, 2, 2, False),
                                                   (1, 1, 0, 1, True), (3, 1, 0, 1, False)])
def test_dwsep_matches_numpy(K, stride, pad, dil, bias):
    N, C, H, W, O = 2, 3, 11, 9, 4
    x = rng.standard_normal((N, C, H, W)).astype(np.float32)
    dw = rng.uniform(-1, 1, (C, 1, K, K)).astype(np.float32)
    pw = rng.uniform(-1, 1, (O, C, 1, 1)).astype(np.float32)
    db = rng.uniform(-1, 1, C).astype(np.float32) if bias else None
    pb = rng.uniform(-1, 1, O).astype(np.float32) if bias else None
    ref = np_dwsep(x, dw, db, pw, pb, stride, pad, dil)
    got = oracle.dwsep_conv2d(x, dw, db, pw, pb, stride, pad, dil)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    idx = rng.choice(got.size, 50, replace=False)
    np.testing.assert_array_equal(oracle.dwsep_conv2d_at(x, dw, db, pw, pb, idx, stride, pad, dil),
                                  got.reshape(-1)[idx])


def test_dwsep_center_delta_identity_and_corner_shift():
    C = 4
    x = rng.standard_normal((2, C, 7, 9)).astype(np.float32)
    eye = np.eye(C, dtype=np.float32).reshape(C, C, 1, 1)
    dw = np.zeros((C, 1, 3, 3), np.float32)
    dw[:, 0, 1, 1] = 1.0
    np.testing.assert_array_equal(oracle.dwsep_conv2d(x, dw, None, eye, None), x)
    dw = np.zeros((C, 1, 3, 3), np.float32)
    dw[:, 0, 0, 0] = 1.0   # reads (h-1, w-1): shift down-right, zero border
    y = oracle.dwsep_conv2d(x, dw, None, eye, None)
    assert np.all(y[:, :, 0, :] == 0) and np.all(y[:, :, :, 0] == 0)
    np.testing.assert_array_equal(y[:, :, 1:, 1:], x[:, :, :-1, :-1])


def test_dwsep_pointwise_is_matmul():
    N, C, H, W, O = 2, 5, 4, 6, 7
    x = rng.standard_normal((N, C, H, W)).astype(np.float32)
    alpha = rng.uniform(-1, 1, C).astype(np.float32)
    dw = np.zeros((C, 1, 3, 3), np.float32)
    dw[:, 0, 1, 1] = alpha
    pw = rng.uniform(-1, 1, (O, C, 1, 1)).astype(np.float32)
    pb = rng.uniform(-1, 1, O).astype(np.float32)
    y = oracle.dwsep_conv2d(x, dw, None, pw, pb)
    M = pw[:, :, 0, 0].astype(np.float64) @ np.diag(alpha.astype(np.float64))
    ref = np.einsum("oc,nchw->nohw", M, x.astype(np.float64)) + pb[None, :, None, None]
    ref2 = (M @ x.astype(np.float64).transpose(1, 0, 2, 3).reshape(C, -1)).reshape(O, N, H, W)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, ref2.transpose(1, 0, 2, 3) + pb[None, :, None, None],
                               rtol=1e-12, atol=1e-12)


def test_dwsep_combined_bias_identity():
    """Page l1_p86 combined bias: b'[o] = sum_c pw[o,c] * dw_b[c] + pw_b[o]."""
    N, C, H, W, O = 1, 3, 5, 6, 4
    x = rng.standard_normal((N, C, H, W)).astype(np.float32)
    dw = rng.uniform(-1, 1, (C, 1, 3, 3)).astype(np.float32)
    pw = rng.uniform(-1, 1, (O, C, 1, 1)).astype(np.float32)
    db = rng.uniform(-1, 1, C).astype(np.float32)
    pb = rng.uniform(-1, 1, O).astype(np.float32)
    y_b = oracle.dwsep_conv2d(x, dw, db, pw, pb)
    y_0 = oracle.dwsep_conv2d(x, dw, None, pw, None)
    bprime = pw[:, :, 0, 0].astype(np.float64) @ db.astype(np.float64) + pb
    np.testing.assert_allclose(y_b - y_0, np.broadcast_to(bprime[None, :, None, None], y_b.shape),
                               rtol=1e-12, atol=1e-12)

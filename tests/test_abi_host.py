"""Host-only checks of libconvfuse.so: it loads, exports every function include/convfuse.h
declares, and rejects bad arguments with the documented codes before launching anything.
No GPU is needed: every call here fails validation (or is an N = 0 no-op), so no kernel is
launched with the fake pointers used below."""
import ctypes
import os
import re

import pytest

import implicit_gemm_convolution_conv3d_amd as cf

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "convfuse.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    assert {"conv3d_mish_tanh", "conv3d_div_maxpool_gap_bias_sum", "dwsep_conv2d"} <= names
    assert names == set(cf.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = cf.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.convfuse_abi_version() == 102


def test_library_was_built_from_this_tree():
    from implicit_gemm_convolution_conv3d_amd import _build
    assert cf.build_id() == _build.source_sha()


def _golden(key):
    import json
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_values.json")
    return json.load(open(path))[key]["value"]


def test_out_dims_conv3d_page_shapes():
    # Conv3d + Mish + Tanh: [16,32,32,64,64] with a 3^3 kernel -> [16,64,30,62,62]
    g = _golden("conv3d_mish_tanh_output_shape")
    assert cf.out_dims_conv3d(*g["input"][2:], 3) == tuple(g["output"][2:])
    # the pooling workload's conv: [.,8,16,64,64] -> 14 x 62 x 62, then pool 2 -> 7 x 31 x 31
    g = _golden("pool_conv_output_shape")
    conv = cf.out_dims_conv3d(*g["input"][2:], 3)
    assert conv == tuple(g["conv_output"][2:])
    pooled = cf.out_dims_conv3d(*conv, 2, 2, 0)
    assert pooled == tuple(_golden("pool_pooled_shape")[2:])
    assert pooled[0] * pooled[1] * pooled[2] == _golden("pool_pooled_count")


def test_out_dims_conv2d_page_shapes():
    g = _golden("dwsep_output_shape")
    assert cf.out_dims_conv2d(*g["input"][2:], 3, 1, 1, 1) == tuple(g["output"][2:])
    assert cf.out_dims_conv2d(333, 517, 3, 1, 1, 1) == (333, 517)
    assert cf.out_dims_conv2d(512, 512, 5, 2, 2, 1) == (256, 256)
    assert cf.out_dims_conv2d(20, 9, 3, 1, 2, 2) == (20, 9)
    assert cf.out_dims_conv2d(7, 7, 3, 2, 0, 1) == (3, 3)


@pytest.mark.parametrize("args", [(0, 8, 8, 3, 1, 0), (2, 8, 8, 3, 1, 0), (8, 8, 8, 3, 0, 0),
                                  (8, 8, 8, 3, 1, -1), (8, 8, 8, 0, 1, 0), (8, 1 << 25, 8, 3, 1, 0)])
def test_out_dims_conv3d_rejects(args):
    with pytest.raises(cf.ConvFuseError) as e:
        cf.out_dims_conv3d(*args)
    assert e.value.code == cf.ERR_SHAPE
    assert "convfuse_out_dims_conv3d" in cf.lib().convfuse_last_error().decode()


@pytest.mark.parametrize("args", [(8, 0, 3, 1, 1, 1), (2, 8, 5, 1, 0, 1), (8, 8, 3, 0, 1, 1),
                                  (8, 8, 3, 1, 1, 0), (8, 8, 3, 1, -1, 1)])
def test_out_dims_conv2d_rejects(args):
    with pytest.raises(cf.ConvFuseError) as e:
        cf.out_dims_conv2d(*args)
    assert e.value.code == cf.ERR_SHAPE


def test_out_dims_null_pointers():
    L = cf.lib()
    v = ctypes.c_int64(-7)
    assert L.convfuse_out_dims_conv3d(8, 8, 8, 3, 1, 0, None, ctypes.byref(v),
                                      ctypes.byref(v)) == cf.ERR_NULL
    assert L.convfuse_out_dims_conv2d(8, 8, 3, 1, 1, 1, ctypes.byref(v), None) == cf.ERR_NULL
    assert v.value == -7


@pytest.mark.parametrize("args,expected", [
    ((32, 3, 1, 0, 1), 30), ((64, 3, 1, 0, 1), 62), ((512, 3, 1, 1, 1), 512),
    ((333, 3, 1, 1, 1), 333), ((517, 3, 1, 1, 1), 517), ((14, 2, 2, 0, 1), 7),
    ((62, 2, 2, 0, 1), 31), ((10, 3, 2, 1, 1), 5), ((9, 3, 1, 2, 2), 9), ((1, 1, 1, 0, 1), 1),
])
def test_out_len(args, expected):
    assert cf.conv_out_len(*args) == expected


@pytest.mark.parametrize("args", [(0, 3, 1, 0, 1), (2, 3, 1, 0, 1), (5, 3, 0, 0, 1),
                                  (5, 3, 1, -1, 1), (5, 0, 1, 0, 1), (5, 3, 1, 0, 0)])
def test_out_len_rejects(args):
    with pytest.raises(cf.ConvFuseError) as e:
        cf.conv_out_len(*args)
    assert e.value.code == cf.ERR_SHAPE
    assert "convfuse_conv_out_len" in cf.lib().convfuse_last_error().decode()


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def call_act(x=FAKE, w=FAKE, b=None, y=FAKE, N=1, C=4, D=8, H=8, W=8, O=8, k=3, s=1, p=0):
    return cf.lib().conv3d_mish_tanh(x, w, b, y, N, C, D, H, W, O, k, s, p, None)


def call_pool(x=FAKE, w=FAKE, cb=None, div=2.0, pool=2, bias=FAKE, out=FAKE, N=1, C=4, D=8,
              H=8, W=8, O=8, k=3):
    return cf.lib().conv3d_div_maxpool_gap_bias_sum(x, w, cb, div, pool, bias, out, N, C, D, H,
                                                    W, O, k, None)


def call_dw(x=FAKE, dw=FAKE, db=None, pw=FAKE, pb=None, y=FAKE, N=1, C=4, H=8, W=8, O=8, K=3,
            s=1, p=1, d=1):
    return cf.lib().dwsep_conv2d(x, dw, db, pw, pb, y, N, C, H, W, O, K, s, p, d, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), cf.ERR_NULL), (dict(w=None), cf.ERR_NULL), (dict(y=None), cf.ERR_NULL),
    (dict(C=0), cf.ERR_SHAPE), (dict(O=0), cf.ERR_SHAPE), (dict(N=-1), cf.ERR_SHAPE),
    (dict(D=2), cf.ERR_SHAPE), (dict(W=0), cf.ERR_SHAPE), (dict(p=-1), cf.ERR_SHAPE),
    (dict(s=0), cf.ERR_SHAPE), (dict(C=1 << 40), cf.ERR_SHAPE),
    (dict(N=1 << 20, C=1 << 20, D=1 << 20, H=1 << 20), cf.ERR_SHAPE),
    (dict(s=1 << 25), cf.ERR_SHAPE), (dict(D=1 << 25), cf.ERR_SHAPE),
    (dict(k=1100, D=1 << 12, H=1 << 12, W=1 << 12, C=1, O=1), cf.ERR_UNSUPPORTED),
])
def test_conv3d_mish_tanh_validation(kw, code):
    assert call_act(**kw) == code
    assert cf.lib().convfuse_last_error().decode().startswith("conv3d_mish_tanh")


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), cf.ERR_NULL), (dict(bias=None), cf.ERR_NULL), (dict(out=None), cf.ERR_NULL),
    (dict(div=0.0), cf.ERR_SHAPE), (dict(div=float("inf")), cf.ERR_SHAPE),
    (dict(div=float("nan")), cf.ERR_SHAPE), (dict(D=3), cf.ERR_SHAPE),
    (dict(pool=0), cf.ERR_SHAPE), (dict(pool=9), cf.ERR_SHAPE), (dict(C=0), cf.ERR_SHAPE),
    (dict(pool=33, D=66, H=66, W=66), cf.ERR_UNSUPPORTED),
    (dict(k=1100, D=1 << 12, H=1 << 12, W=1 << 12, C=1, O=1), cf.ERR_UNSUPPORTED),
])
def test_pool_validation(kw, code):
    assert call_pool(**kw) == code
    assert "conv3d_div_maxpool_gap_bias_sum" in cf.lib().convfuse_last_error().decode()


def call_maxpool(x=FAKE, w=FAKE, cb=None, div=2.0, pool=2, y=FAKE, N=1, C=4, D=8, H=8, W=8,
                 O=8, k=3):
    return cf.lib().conv3d_div_maxpool(x, w, cb, div, pool, y, N, C, D, H, W, O, k, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), cf.ERR_NULL), (dict(w=None), cf.ERR_NULL), (dict(y=None), cf.ERR_NULL),
    (dict(div=0.0), cf.ERR_SHAPE), (dict(div=float("nan")), cf.ERR_SHAPE),
    (dict(D=3), cf.ERR_SHAPE), (dict(pool=0), cf.ERR_SHAPE), (dict(pool=9), cf.ERR_SHAPE),
    (dict(C=0), cf.ERR_SHAPE), (dict(O=-1), cf.ERR_SHAPE),
    (dict(pool=33, D=66, H=66, W=66), cf.ERR_UNSUPPORTED),
])
def test_maxpool_validation(kw, code):
    assert call_maxpool(**kw) == code
    assert cf.lib().convfuse_last_error().decode().startswith("conv3d_div_maxpool")


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), cf.ERR_NULL), (dict(dw=None), cf.ERR_NULL), (dict(pw=None), cf.ERR_NULL),
    (dict(y=None), cf.ERR_NULL), (dict(C=0), cf.ERR_SHAPE), (dict(H=0), cf.ERR_SHAPE),
    (dict(p=0, H=2), cf.ERR_SHAPE), (dict(d=0), cf.ERR_SHAPE),
    (dict(s=1 << 25), cf.ERR_SHAPE), (dict(K=1 << 25), cf.ERR_SHAPE),
    (dict(K=40000, p=20000, C=1, O=1), cf.ERR_UNSUPPORTED),
])
def test_dwsep_validation(kw, code):
    assert call_dw(**kw) == code
    assert cf.lib().convfuse_last_error().decode().startswith("dwsep_conv2d")


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), cf.ERR_NULL), (dict(w=None), cf.ERR_NULL), (dict(y=None), cf.ERR_NULL),
    (dict(C=0), cf.ERR_SHAPE), (dict(O=0), cf.ERR_SHAPE), (dict(N=-1), cf.ERR_SHAPE),
    (dict(D=2), cf.ERR_SHAPE), (dict(p=-1), cf.ERR_SHAPE), (dict(s=0), cf.ERR_SHAPE),
    (dict(k=1100, D=1 << 12, H=1 << 12, W=1 << 12, C=1, O=1), cf.ERR_UNSUPPORTED),
])
def test_conv3d_split_validation(kw, code):
    args = dict(x=FAKE, w=FAKE, b=None, y=FAKE, N=1, C=4, D=8, H=8, W=8, O=8, k=3, s=1, p=0)
    args.update(kw)
    a = args
    assert cf.lib().conv3d_mish_tanh_split_bf16(a["x"], a["w"], a["b"], a["y"], a["N"], a["C"],
                                                a["D"], a["H"], a["W"], a["O"], a["k"], a["s"],
                                                a["p"], None) == code
    assert cf.lib().convfuse_last_error().decode().startswith("conv3d_mish_tanh_split_bf16")


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), cf.ERR_NULL), (dict(bias=None), cf.ERR_NULL), (dict(out=None), cf.ERR_NULL),
    (dict(div=0.0), cf.ERR_SHAPE), (dict(div=float("nan")), cf.ERR_SHAPE), (dict(D=3), cf.ERR_SHAPE),
    (dict(pool=0), cf.ERR_SHAPE), (dict(C=0), cf.ERR_SHAPE),
    (dict(pool=33, D=66, H=66, W=66), cf.ERR_UNSUPPORTED),
])
def test_pool_split_validation(kw, code):
    a = dict(x=FAKE, w=FAKE, cb=None, div=2.0, pool=2, bias=FAKE, out=FAKE, N=1, C=4, D=8, H=8,
             W=8, O=8, k=3)
    a.update(kw)
    assert cf.lib().conv3d_div_maxpool_gap_bias_sum_split_bf16(
        a["x"], a["w"], a["cb"], a["div"], a["pool"], a["bias"], a["out"], a["N"], a["C"],
        a["D"], a["H"], a["W"], a["O"], a["k"], None) == code
    assert cf.lib().convfuse_last_error().decode().startswith(
        "conv3d_div_maxpool_gap_bias_sum_split_bf16")


@pytest.mark.parametrize("iters,wgs,out,code", [
    (0, 1, FAKE, cf.ERR_SHAPE), (1 << 22, 1, FAKE, cf.ERR_SHAPE), (1, 0, FAKE, cf.ERR_SHAPE),
    (1, (1 << 20) + 1, FAKE, cf.ERR_SHAPE), (1, 1, None, cf.ERR_NULL),
])
def test_measure_mfma_validation(iters, wgs, out, code):
    assert cf.lib().convfuse_measure_mfma(out, iters, wgs, None) == code
    assert cf.lib().convfuse_last_error().decode().startswith("convfuse_measure_mfma")


def call_dw_split(x=FAKE, dw=FAKE, db=None, pw=FAKE, pb=None, y=FAKE, N=1, C=4, H=8, W=8, O=8,
                  K=3, s=1, p=1, d=1):
    return cf.lib().dwsep_conv2d_split_bf16(x, dw, db, pw, pb, y, N, C, H, W, O, K, s, p, d, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), cf.ERR_NULL), (dict(dw=None), cf.ERR_NULL), (dict(pw=None), cf.ERR_NULL),
    (dict(y=None), cf.ERR_NULL), (dict(C=0), cf.ERR_SHAPE), (dict(O=0), cf.ERR_SHAPE),
    (dict(N=-1), cf.ERR_SHAPE), (dict(H=0), cf.ERR_SHAPE), (dict(p=0, H=2), cf.ERR_SHAPE),
    (dict(d=0), cf.ERR_SHAPE), (dict(s=0), cf.ERR_SHAPE), (dict(p=-1), cf.ERR_SHAPE),
    (dict(s=1 << 25), cf.ERR_SHAPE), (dict(K=1 << 25), cf.ERR_SHAPE),
    (dict(N=1 << 20, C=1 << 20, H=1 << 20), cf.ERR_SHAPE),
    (dict(K=40000, p=20000, C=1, O=1), cf.ERR_UNSUPPORTED),
])
def test_dwsep_split_validation(kw, code):
    assert call_dw_split(**kw) == code
    assert cf.lib().convfuse_last_error().decode().startswith("dwsep_conv2d_split_bf16")


def test_empty_batch_is_a_no_op():
    # N = 0: nothing to compute, no pointer is needed and nothing is launched.
    assert call_act(x=None, w=None, y=None, N=0) == cf.OK
    assert call_pool(x=None, w=None, bias=None, out=None, N=0) == cf.OK
    assert call_maxpool(x=None, w=None, y=None, N=0) == cf.OK
    assert call_dw(x=None, dw=None, pw=None, y=None, N=0) == cf.OK
    assert call_dw_split(x=None, dw=None, pw=None, y=None, N=0) == cf.OK


def test_error_message_is_thread_local():
    import threading
    assert call_act(C=0) == cf.ERR_SHAPE
    seen = {}

    def other():
        seen["msg"] = cf.lib().convfuse_last_error().decode()
        call_dw(C=0)
        seen["after"] = cf.lib().convfuse_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert seen["after"].startswith("dwsep_conv2d")
    assert cf.lib().convfuse_last_error().decode().startswith("conv3d_mish_tanh")


@pytest.mark.parametrize("call,code,prefix", [
    (lambda L: L.conv3d_bias(None, FAKE, None, FAKE, 1, 4, 8, 8, 8, 8, 3, 1, 0, None),
     cf.ERR_NULL, "conv3d_bias"),
    (lambda L: L.conv3d_bias(FAKE, FAKE, None, FAKE, 1, 0, 8, 8, 8, 8, 3, 1, 0, None),
     cf.ERR_SHAPE, "conv3d_bias"),
    (lambda L: L.conv3d_bias(FAKE, FAKE, None, FAKE, 1, 4, 2, 8, 8, 8, 3, 1, 0, None),
     cf.ERR_SHAPE, "conv3d_bias"),
    (lambda L: L.mish_tanh(None, FAKE, 10, None), cf.ERR_NULL, "mish_tanh"),
    (lambda L: L.mish_tanh(FAKE, FAKE, -1, None), cf.ERR_SHAPE, "mish_tanh"),
    (lambda L: L.div_maxpool_gap_bias_sum(FAKE, 0.0, 2, FAKE, FAKE, 1, 4, 8, 8, 8, None),
     cf.ERR_SHAPE, "div_maxpool_gap_bias_sum"),
    (lambda L: L.div_maxpool_gap_bias_sum(FAKE, 2.0, 9, FAKE, FAKE, 1, 4, 8, 8, 8, None),
     cf.ERR_SHAPE, "div_maxpool_gap_bias_sum"),
    (lambda L: L.div_maxpool_gap_bias_sum(FAKE, 2.0, 2, None, FAKE, 1, 4, 8, 8, 8, None),
     cf.ERR_NULL, "div_maxpool_gap_bias_sum"),
    (lambda L: L.depthwise_conv2d(FAKE, None, None, FAKE, 1, 4, 8, 8, 3, 1, 1, 1, None),
     cf.ERR_NULL, "depthwise_conv2d"),
    (lambda L: L.depthwise_conv2d(FAKE, FAKE, None, FAKE, 1, 4, 2, 8, 3, 1, 0, 1, None),
     cf.ERR_SHAPE, "depthwise_conv2d"),
    (lambda L: L.pointwise_conv2d(FAKE, None, None, FAKE, 1, 4, 8, 8, 8, None),
     cf.ERR_NULL, "pointwise_conv2d"),
    (lambda L: L.pointwise_conv2d(FAKE, FAKE, None, FAKE, 1, 4, 0, 8, 8, None),
     cf.ERR_SHAPE, "pointwise_conv2d"),
])
def test_unfused_steps_validation(call, code, prefix):
    assert call(cf.lib()) == code
    assert cf.lib().convfuse_last_error().decode().startswith(prefix)


def test_unfused_steps_empty_is_a_no_op():
    L = cf.lib()
    assert L.conv3d_bias(None, None, None, None, 0, 4, 8, 8, 8, 8, 3, 1, 0, None) == cf.OK
    assert L.mish_tanh(None, None, 0, None) == cf.OK
    assert L.div_maxpool_gap_bias_sum(None, 2.0, 2, None, None, 0, 4, 8, 8, 8, None) == cf.OK
    assert L.depthwise_conv2d(None, None, None, None, 0, 4, 8, 8, 3, 1, 1, 1, None) == cf.OK
    assert L.pointwise_conv2d(None, None, None, None, 0, 4, 8, 8, 8, None) == cf.OK

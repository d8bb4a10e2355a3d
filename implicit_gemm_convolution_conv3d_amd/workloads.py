"""Seeded synthetic inputs for the fused convolution hot path.

This module holds only input shapes, value distributions and the random generator;
it contains none of the convolution arithmetic, so both the GPU path's tests and the
CPU oracle can take their inputs from here.

Recipe (every workload):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64); draws in the order the
    arrays are listed; ``x`` is drawn directly in float32 (standard normal), every
    other array is drawn in float64 and rounded to float32;
  * activations x ~ N(0, 1);
  * Conv3d weights and conv biases ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)) with
    fan_in = Cin * k^3, PyTorch's default Conv initialisation that the pages assume;
  * the extra per-channel bias of the pooling workload ~ N(0, 1);
  * depthwise weights/bias ~ U(-1/3, 1/3) (fan_in 9); pointwise weights ~ U(+-1/sqrt(Cin)),
    pointwise bias ~ U(+-1/sqrt(Cin)).
The five named workloads use seed 20261202 + their index (1..5).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20261202


def _uniform(rng, shape, bound):
    return rng.uniform(-bound, bound, size=shape).astype(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(size=shape).astype(np.float32)


def _x(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def conv3d_act_inputs(seed, N, C, D, H, W, O, k=3, bias=True):
    """x [N,C,D,H,W], w [O,C,k,k,k], b [O] (or None)."""
    rng = np.random.default_rng(seed)
    bound = 1.0 / np.sqrt(C * k ** 3)
    x = _x(rng, (N, C, D, H, W))
    w = _uniform(rng, (O, C, k, k, k), bound)
    b = _uniform(rng, (O,), bound) if bias else None
    return {"x": x, "w": w, "b": b}


def conv3d_pool_inputs(seed, N, C, D, H, W, O, k=3, conv_bias=True):
    """x, w [O,C,k,k,k], conv_b [O] (or None), bias [O,1,1,1] ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    bound = 1.0 / np.sqrt(C * k ** 3)
    x = _x(rng, (N, C, D, H, W))
    w = _uniform(rng, (O, C, k, k, k), bound)
    cb = _uniform(rng, (O,), bound) if conv_bias else None
    bias = _normal(rng, (O, 1, 1, 1))
    return {"x": x, "w": w, "conv_b": cb, "bias": bias}


def dwsep_inputs(seed, N, C, H, W, O, K=3, bias=False):
    """x [N,C,H,W], dw_w [C,1,K,K], dw_b [C]|None, pw_w [O,C,1,1], pw_b [O]|None."""
    rng = np.random.default_rng(seed)
    x = _x(rng, (N, C, H, W))
    dbound = 1.0 / np.sqrt(K * K)
    pbound = 1.0 / np.sqrt(C)
    dw_w = _uniform(rng, (C, 1, K, K), dbound)
    dw_b = _uniform(rng, (C,), dbound) if bias else None
    pw_w = _uniform(rng, (O, C, 1, 1), pbound)
    pw_b = _uniform(rng, (O,), pbound) if bias else None
    return {"x": x, "dw_w": dw_w, "dw_b": dw_b, "pw_w": pw_w, "pw_b": pw_b}


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    op: str
    dims: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)

    @property
    def seed(self):
        return BASE_SEED + self.index

    def inputs(self, seed=None):
        s = self.seed if seed is None else seed
        d = self.dims
        if self.op in ("conv3d_mish_tanh", "conv3d_mish_tanh_split_bf16"):
            return conv3d_act_inputs(s, d["N"], d["C"], d["D"], d["H"], d["W"], d["O"],
                                     self.params["k"], bias=True)
        if self.op in ("conv3d_div_maxpool_gap_bias_sum", "conv3d_div_maxpool",
                       "conv3d_div_maxpool_gap_bias_sum_split_bf16"):
            return conv3d_pool_inputs(s, d["N"], d["C"], d["D"], d["H"], d["W"], d["O"],
                                      self.params["k"], conv_bias=True)
        if self.op in ("dwsep_conv2d", "dwsep_conv2d_split_bf16"):
            return dwsep_inputs(s, d["N"], d["C"], d["H"], d["W"], d["O"], self.params["K"],
                                bias=self.params["bias"])
        raise ValueError(self.op)


WORKLOADS = {
    1: Workload(1, "tiny_conv3d_mish_tanh", "conv3d_mish_tanh",
                dict(N=1, C=4, D=8, H=16, W=16, O=8), dict(k=3, stride=1, pad=0)),
    2: Workload(2, "conv3d_div_maxpool_gap_bias_sum", "conv3d_div_maxpool_gap_bias_sum",
                dict(N=128, C=8, D=16, H=64, W=64, O=16), dict(k=3, divisor=2.0, pool=2)),
    3: Workload(3, "conv3d_mish_tanh", "conv3d_mish_tanh",
                dict(N=16, C=32, D=32, H=64, W=64, O=64), dict(k=3, stride=1, pad=0)),
    4: Workload(4, "dwsep_conv2d_512", "dwsep_conv2d",
                dict(N=16, C=64, H=512, W=512, O=128),
                dict(K=3, stride=1, pad=1, dilation=1, bias=False)),
    5: Workload(5, "dwsep_conv2d_333x517_bias", "dwsep_conv2d",
                dict(N=8, C=96, H=333, W=517, O=192),
                dict(K=3, stride=1, pad=1, dilation=1, bias=True)),
    # General-parameter variants of the same layers (kernel size, stride, pooling window),
    # timed on request; they run the general kernels.
    6: Workload(6, "conv3d_mish_tanh_k5_s2_p2", "conv3d_mish_tanh",
                dict(N=16, C=32, D=32, H=64, W=64, O=64), dict(k=5, stride=2, pad=2)),
    7: Workload(7, "conv3d_div_maxpool3_gap_bias_sum", "conv3d_div_maxpool_gap_bias_sum",
                dict(N=128, C=8, D=16, H=64, W=64, O=16), dict(k=3, divisor=2.0, pool=3)),
    8: Workload(8, "dwsep_conv2d_512_k5_s2", "dwsep_conv2d",
                dict(N=16, C=64, H=512, W=512, O=128),
                dict(K=5, stride=2, pad=2, dilation=1, bias=False)),
    # The pooling layer with its pooled tensor [N,O,7,31,31] as the output (no global mean).
    9: Workload(9, "conv3d_div_maxpool", "conv3d_div_maxpool",
                dict(N=128, C=8, D=16, H=64, W=64, O=16), dict(k=3, divisor=2.0, pool=2)),
    # The two depthwise-separable layers with the pointwise GEMM as a three-term bf16 split of
    # fp32 on the matrix cores (opt-in precision mode with its own error contract).
    10: Workload(10, "dwsep_conv2d_512_split_bf16", "dwsep_conv2d_split_bf16",
                 dict(N=16, C=64, H=512, W=512, O=128),
                 dict(K=3, stride=1, pad=1, dilation=1, bias=False)),
    11: Workload(11, "dwsep_conv2d_333x517_bias_split_bf16", "dwsep_conv2d_split_bf16",
                 dict(N=8, C=96, H=333, W=517, O=192),
                 dict(K=3, stride=1, pad=1, dilation=1, bias=True)),
    12: Workload(12, "conv3d_mish_tanh_split_bf16", "conv3d_mish_tanh_split_bf16",
                 dict(N=16, C=32, D=32, H=64, W=64, O=64), dict(k=3, stride=1, pad=0)),
    13: Workload(13, "conv3d_div_maxpool_gap_bias_sum_split_bf16",
                 "conv3d_div_maxpool_gap_bias_sum_split_bf16",
                 dict(N=128, C=8, D=16, H=64, W=64, O=16), dict(k=3, divisor=2.0, pool=2)),
}

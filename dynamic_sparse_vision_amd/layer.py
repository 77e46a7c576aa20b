"""The DCNv4 layer around the operator: projections in, the spatial
aggregation, projection out.

The module's arguments follow the constructor quoted in the blog "DCNv4架构解析"
(section "动态卷积机制创新": channels, kernel_size, stride, pad, dilation,
group, offset_scale, dw_kernel_size, remove_center, output_bias,
without_pointwise), and the offsets and masks come from one merged linear
layer (walkthrough "DCNv4论文解析", section 2.2, micro design).  Layout is
channel-last throughout, x: (N, H, W, C).

    value       = x @ W_v + b_v                          (skipped: without_pointwise)
    offset_mask = x' @ W_om + b_om,  x' = dwconv(x) or x  (P = roundup8(3*G*K) columns,
                                                           written in the operator's
                                                           padded layout directly;
                                                           x' at the output pixels'
                                                           window centres)
    y           = dcnv4(value, offset_mask)              (the HIP operator, C ABI)
    out         = y @ W_o (+ b_o if output_bias)          (skipped: without_pointwise)

The projections are plain GEMMs and go to the vendor BLAS through torch; the
depthwise convolution goes through torch as well.  Only the aggregation and
its backward run in this library's kernels (``Dcnv4Function``).  The
center_feature_scale option of the pages' constructor is not built: the
pages name it but do not define its arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import dcnv4


class Dcnv4Function(torch.autograd.Function):
    """Autograd wrapper of dcnv4_forward_ex / dcnv4_backward_ex.

    grad_value comes back in fp32 from the library and is rounded once to
    the value's dtype here; grad_offset_mask is already in the offset_mask's
    dtype.
    """

    @staticmethod
    def forward(ctx, value, offset_mask, params: dict):
        ctx.params = params
        ctx.save_for_backward(value, offset_mask)
        return dcnv4.forward(value.contiguous(), offset_mask.contiguous(), **params)

    @staticmethod
    def backward(ctx, grad_out):
        value, offset_mask = ctx.saved_tensors
        gv, gom = dcnv4.backward(value, offset_mask, grad_out.contiguous(), **ctx.params)
        return gv.to(value.dtype), gom, None


def aggregate(value, offset_mask, **params):
    """The operator with autograd (params as for dcnv4.forward)."""
    return Dcnv4Function.apply(value, offset_mask, params)


@dataclass
class LayerConfig:
    channels: int = 64
    kernel_size: int = 3
    stride: int = 1
    pad: int = 1
    dilation: int = 1
    group: int = 4
    offset_scale: float = 1.0
    dw_kernel_size: int | None = None
    remove_center: bool = False
    output_bias: bool = True
    without_pointwise: bool = False
    softmax: bool = False           # the DCNv3 form (masks normalised over K)

    @property
    def K(self) -> int:
        return self.kernel_size * self.kernel_size - int(self.remove_center)

    @property
    def P(self) -> int:
        return dcnv4.dcnv4_om_channels(self.group, self.kernel_size, self.kernel_size,
                                       self.remove_center)

    def op_params(self) -> dict:
        k = self.kernel_size
        return dict(kernel_h=k, kernel_w=k, stride_h=self.stride, stride_w=self.stride,
                    pad_h=self.pad, pad_w=self.pad, dilation_h=self.dilation,
                    dilation_w=self.dilation, group=self.group,
                    group_channels=self.channels // self.group, offset_scale=self.offset_scale,
                    remove_center=self.remove_center, softmax=self.softmax)


def init_weights(cfg: LayerConfig, device, dtype=torch.float32, seed: int = 0) -> dict:
    """Random weights of the layer's shapes (there are no trained weights):
    weights ~ N(0, 1/fan_in), biases ~ N(0, 0.1); the offset/mask linear is
    scaled so that offsets come out at a few pixels; its padding columns are
    zero."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    C, P, GK3 = cfg.channels, cfg.P, 3 * cfg.group * cfg.K

    def rnd(*shape, std):
        return (torch.randn(*shape, generator=g) * std).to(device=device, dtype=dtype)

    w = {}
    if not cfg.without_pointwise:
        w["w_v"] = rnd(C, C, std=C ** -0.5)
        w["b_v"] = rnd(C, std=0.1)
        w["w_o"] = rnd(C, C, std=C ** -0.5)
        if cfg.output_bias:
            w["b_o"] = rnd(C, std=0.1)
    w_om = torch.zeros(C, P)
    b_om = torch.zeros(P)
    w_om[:, :GK3] = torch.randn(C, GK3, generator=g) * (2.0 * C ** -0.5)
    b_om[:GK3] = torch.randn(GK3, generator=g) * 0.1
    w["w_om"] = w_om.to(device=device, dtype=dtype)
    w["b_om"] = b_om.to(device=device, dtype=dtype)
    if cfg.dw_kernel_size:
        kd = cfg.dw_kernel_size
        w["w_dw"] = rnd(C, 1, kd, kd, std=1.0 / kd)
        w["b_dw"] = rnd(C, std=0.1)
    return w


def centre_features(x, cfg: LayerConfig):
    """Features at the window centres of the output pixels: the offsets and
    masks of an output pixel are predicted from the feature at its window
    centre, x[ho*stride, wo*stride] when pad = dilation*(kernel_size-1)/2
    (identity for stride 1)."""
    if cfg.stride == 1 and 2 * cfg.pad == cfg.dilation * (cfg.kernel_size - 1):
        return x
    if 2 * cfg.pad != cfg.dilation * (cfg.kernel_size - 1):
        raise ValueError("the layer needs pad = dilation*(kernel_size-1)/2 (window centre on the grid)")
    N, H, W, C = x.shape
    Ho = (H - 1) // cfg.stride + 1
    Wo = (W - 1) // cfg.stride + 1
    return x[:, ::cfg.stride, ::cfg.stride][:, :Ho, :Wo]


def layer_forward(x, w: dict, cfg: LayerConfig):
    """x (N, H, W, C) -> out (N, Ho, Wo, C); differentiable in x and w."""
    if cfg.without_pointwise:
        value = x
    else:
        value = torch.nn.functional.linear(x, w["w_v"].t(), w["b_v"])
    xo = x
    if cfg.dw_kernel_size:
        xc = x.permute(0, 3, 1, 2)
        xc = torch.nn.functional.conv2d(xc, w["w_dw"], w["b_dw"], padding=(cfg.dw_kernel_size - 1) // 2,
                                        groups=cfg.channels)
        xo = xc.permute(0, 2, 3, 1)
    xo = centre_features(xo, cfg)
    offset_mask = torch.nn.functional.linear(xo, w["w_om"].t(), w["b_om"])
    y = aggregate(value.contiguous(), offset_mask.contiguous(), **cfg.op_params())
    if cfg.without_pointwise:
        return y
    return torch.nn.functional.linear(y, w["w_o"].t(), w.get("b_o"))

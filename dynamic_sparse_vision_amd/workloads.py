"""The benchmark and parity workloads: shapes, dtypes, distributions, seeds.

Feature-map shapes follow the operator benchmarks of "Efficient Deformable
ConvNets" (CSDN walkthrough "DCNv4论文解析", section 3.1: maps of a 224x224
input at /4, /8, /16, /32 with batch 64, and a batch-1 high-resolution map)
with 16 channels per group, the 3x3 grid, stride 1, pad 1, dilation 1 and
offset_scale 1.0.  Inputs are synthetic (``synth``); sigma values are standard
deviations.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import synth


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    W: int
    C: int
    G: int
    dtype: str            # storage dtype: fp32 | fp16 | bf16
    seed: int
    sigma_value: float
    sigma_off: float
    sigma_m: float
    direction: str        # fwd | bwd
    remove_center: bool = False
    integer_offsets: bool = False
    kernel: tuple = (3, 3)
    stride: tuple = (1, 1)
    pad: tuple = (1, 1)
    dilation: tuple = (1, 1)
    offset_scale: float = 1.0
    sigma_grad: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def Cg(self) -> int:
        return self.C // self.G

    @property
    def K(self) -> int:
        return self.kernel[0] * self.kernel[1] - int(self.remove_center)

    @property
    def P(self) -> int:
        return synth.om_channels(self.G, self.K)

    @property
    def Ho(self) -> int:
        kh, s, p, d = self.kernel[0], self.stride[0], self.pad[0], self.dilation[0]
        return (self.H + 2 * p - (d * (kh - 1) + 1)) // s + 1

    @property
    def Wo(self) -> int:
        kw, s, p, d = self.kernel[1], self.stride[1], self.pad[1], self.dilation[1]
        return (self.W + 2 * p - (d * (kw - 1) + 1)) // s + 1

    @property
    def points(self) -> int:
        """Sampled points per call: N * Ho * Wo * G * K * C'."""
        return self.N * self.Ho * self.Wo * self.G * self.K * self.Cg

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def fwd_bytes(self) -> int:
        """Compulsory forward bytes: value + offset_mask + output."""
        s = self.elem_bytes
        return s * (self.N * self.H * self.W * self.C + self.N * self.Ho * self.Wo * (self.P + self.C))

    def bwd_bytes(self) -> int:
        """Compulsory backward bytes: read value, offset_mask, grad_output
        and write grad_offset_mask in the storage dtype; write grad_value in
        fp32."""
        s = self.elem_bytes
        nv = self.N * self.H * self.W * self.C
        no = self.N * self.Ho * self.Wo
        return s * (nv + no * (2 * self.P + self.C)) + 4 * nv

    def kwargs(self) -> dict:
        return dict(kernel_h=self.kernel[0], kernel_w=self.kernel[1],
                    stride_h=self.stride[0], stride_w=self.stride[1],
                    pad_h=self.pad[0], pad_w=self.pad[1],
                    dilation_h=self.dilation[0], dilation_w=self.dilation[1],
                    group=self.G, group_channels=self.Cg,
                    offset_scale=self.offset_scale, remove_center=self.remove_center)

    def make_inputs(self, pad_fill: float = float("nan"), N: int | None = None,
                    with_grad: bool | None = None):
        """float32 numpy (value, offset_mask[, grad_out]) before storage rounding.

        grad_out is drawn when ``with_grad`` (default: backward workloads).

        ``N`` < self.N draws the first N images of the same streams (a bounded
        sample of the same workload)."""
        n = self.N if N is None else N
        v = synth.value_f32((n, self.H, self.W, self.C), self.seed, self.sigma_value)
        om = synth.offset_mask_f32(n, self.Ho, self.Wo, self.G, self.K, self.P, self.seed,
                                   self.sigma_off, self.sigma_m, pad_fill,
                                   self.integer_offsets)
        out = [v, om]
        if with_grad if with_grad is not None else self.direction == "bwd":
            out.append(synth.grad_out_f32((n, self.Ho, self.Wo, self.C), self.seed, self.sigma_grad))
        return tuple(out)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("c1_fwd_fp32_14x14", 1, 14, 14, 64, 4, "fp32", 0, 1.0, 1.5, 1.0, "fwd",
                 note="small forward case"),
        Workload("c2_fwd_fp32_56x56_b64", 64, 56, 56, 64, 4, "fp32", 2, 1.0, 2.0, 0.5, "fwd",
                 note="FlashInternImage-T-like stage 1"),
        Workload("c3a_fwd_fp16_56x56x64_g4", 64, 56, 56, 64, 4, "fp16", 30, 1.0, 2.0, 0.5, "fwd"),
        Workload("c3b_fwd_fp16_28x28x128_g8", 64, 28, 28, 128, 8, "fp16", 31, 1.0, 2.0, 0.5, "fwd"),
        Workload("c3c_fwd_fp16_14x14x256_g16", 64, 14, 14, 256, 16, "fp16", 32, 1.0, 2.0, 0.5, "fwd"),
        Workload("c3d_fwd_fp16_7x7x512_g32", 64, 7, 7, 512, 32, "fp16", 33, 1.0, 2.0, 0.5, "fwd"),
        Workload("c4_fwd_bf16_270x480_k9", 1, 270, 480, 256, 16, "bf16", 40, 1.0, 4.0, 1.0, "fwd",
                 note="stride-4 map of a 1080x1920 frame"),
        Workload("c4_fwd_bf16_270x480_k8", 1, 270, 480, 256, 16, "bf16", 41, 1.0, 4.0, 1.0, "fwd",
                 remove_center=True),
        Workload("c5_bwd_fp32_56x56_b16", 16, 56, 56, 64, 4, "fp32", 5, 1.0, 2.0, 0.5, "bwd",
                 integer_offsets=True),
    ]
}


# ------------------------------------------------- flash deformable attention --

@dataclass(frozen=True)
class FdaWorkload:
    """A flash deformable attention problem: value (N, S, M, D) over the
    levels ``shapes``; Q queries per image (encoder queries: one per value
    pixel, Q = S); L*K points per (query, head)."""
    name: str
    N: int
    shapes: tuple
    M: int
    D: int
    K: int
    dtype: str
    seed: int
    sigma_px: float = 2.0
    sigma_logit: float = 1.0
    Q: int = 0                 # 0: encoder queries (Q = S)
    note: str = field(default="", compare=False)

    @property
    def L(self) -> int:
        return len(self.shapes)

    @property
    def S(self) -> int:
        return sum(h * w for h, w in self.shapes)

    @property
    def queries(self) -> int:
        return self.Q or self.S

    @property
    def P(self) -> int:
        return synth.fdattn_channels(self.L, self.K)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def points(self) -> int:
        """Sampled points per call: N * Q * M * L * K * D."""
        return self.N * self.queries * self.M * self.L * self.K * self.D

    def fwd_bytes(self) -> int:
        """Compulsory forward bytes: value + loc_attn + output."""
        s = self.elem_bytes
        return s * self.N * (self.S * self.M * self.D + self.queries * self.M * (self.P + self.D))

    def bwd_bytes(self) -> int:
        """Compulsory backward bytes: read value, loc_attn, grad_output, write
        grad_loc_attn in the storage dtype and grad_value in fp32."""
        s = self.elem_bytes
        nv = self.N * self.S * self.M * self.D
        nq = self.N * self.queries * self.M
        return s * (nv + nq * (2 * self.P + self.D)) + 4 * nv

    def make_inputs(self, pad_fill: float = float("nan"), N: int | None = None):
        """float32 numpy (value, loc_attn, grad_out) before storage rounding."""
        n = self.N if N is None else N
        v = synth.value_f32((n, self.S, self.M, self.D), self.seed)
        la = synth.fdattn_loc_attn_f32(n, self.queries, self.M, self.shapes, self.K, self.P, self.seed,
                                       self.sigma_px, self.sigma_logit, encoder_queries=self.Q == 0,
                                       pad_fill=pad_fill)
        g = synth.grad_out_f32((n, self.queries, self.M, self.D), self.seed)
        return v, la, g


# Multi-scale maps of an 800x1280 detection input at strides 8, 16, 32, 64
# (the high-resolution input of the walkthrough's operator benchmarks,
# section 3.1), 8 heads of 32 channels (32 channels per head/group there),
# 4 points per level, encoder queries.
FDA_WORKLOADS = {
    w.name: w
    for w in [
        FdaWorkload("fda_enc_800x1280_b4_fp32", 4, ((100, 160), (50, 80), (25, 40), (13, 20)), 8, 32, 4,
                    "fp32", 60, note="encoder self-attention over four levels"),
        FdaWorkload("fda_enc_800x1280_b4_fp16", 4, ((100, 160), (50, 80), (25, 40), (13, 20)), 8, 32, 4,
                    "fp16", 61),
        FdaWorkload("fda_small_fp32", 2, ((12, 20), (6, 10), (3, 5), (2, 3)), 4, 32, 4, "fp32", 62),
    ]
}

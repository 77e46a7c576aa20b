"""A call whose tensors exceed what one launch addresses (2^31 bytes per
buffer) is split into launches of whole images.  The split must not change
any result: N = 10 images of 256x256x512 fp32 (G = 32, C' = 16; 226 MB of
offset_mask per image, so nine images per launch) against the same images
called one at a time, forward and backward: the output and
grad_offset_mask agree bit for bit, grad_value (summed in an order that
depends on wave timing) within the fp32 parity bound.  The first and the
last image of the split call (one in each launch) are also compared with
the oracle, forward and backward, at the fp32 parity tolerance.  The flash
deformable attention case is GPU against GPU only (split call against
single-image calls), whose parity with the oracle the other tests establish.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_vision_amd import dcnv4
from tests.test_gpu_parity import check, say

pytestmark = pytest.mark.gpu

N, H, W, C, G = 10, 256, 256, 512, 32
K = 9


def test_split_launches_match_single_images():
    P = dcnv4.dcnv4_om_channels(G, 3, 3, False)
    per_image = H * W * P * 4
    assert per_image * 9 < 2 ** 31 < per_image * 10, "the call must span two launches"
    say(f"[split] N={N} {H}x{W}x{C} G={G} fp32: offset_mask {per_image / 1e6:.0f} MB per image")
    gen = torch.Generator(device="cuda").manual_seed(7)
    v = torch.randn((N, H, W, C), device="cuda", generator=gen)
    om = 2.0 * torch.randn((N, H, W, P), device="cuda", generator=gen)
    go = torch.randn((N, H, W, C), device="cuda", generator=gen)
    kw = dict(group=G, group_channels=C // G)
    out = dcnv4.forward(v, om, **kw)
    gv, gom = dcnv4.backward(v, om, go, **kw)
    torch.cuda.synchronize()
    for n in range(N):
        o1 = dcnv4.forward(v[n:n + 1], om[n:n + 1], **kw)
        gv1, gom1 = dcnv4.backward(v[n:n + 1], om[n:n + 1], go[n:n + 1], **kw)
        torch.cuda.synchronize()
        assert torch.equal(out[n:n + 1], o1), f"image {n}: output differs"
        assert torch.equal(gom[n:n + 1], gom1), f"image {n}: grad_offset_mask differs"
        assert bool(((gv[n:n + 1] - gv1).abs() <= 1e-5 + 1e-5 * gv1.abs()).all()), f"image {n}: grad_value differs"
    say(f"  {N} images: the split call agrees with the single-image calls")
    for n in (0, N - 1):
        vn, omn, gon = (t[n:n + 1].cpu().numpy() for t in (v, om, go))
        say(f"  image {n} against the oracle")
        check(out[n:n + 1].cpu().numpy(), oracle.forward(vn, omn, **kw), "fp32", f"image {n} forward")
        rgv, rgom = oracle.backward(vn, omn, gon, **kw)
        check(gv[n:n + 1].cpu().numpy(), rgv, "fp32", f"image {n} grad_value")
        check(gom[n:n + 1].cpu().numpy(), rgom, "fp32", f"image {n} grad_offset_mask")
        assert np.all(gom[n:n + 1, ..., 3 * G * K:].cpu().numpy() == 0)


def test_flash_deform_attn_split_launches_match_single_images():
    """The same for flash deformable attention: one level of 1024x600 with
    M = 8 heads of D = 64 fp32 channels is 1.26 GB of value per image, so
    each image is a launch of its own (the level's 616 000 corner bins also
    exceed the LDS sort: grad_value takes the device-atomic path)."""
    from dynamic_sparse_vision_amd import flash_deform_attn as fda

    n, shapes, M, D, Kp, Q = 2, ((1024, 600),), 8, 64, 4, 1500
    S = shapes[0][0] * shapes[0][1]
    assert S * M * D * 4 > 2 ** 30
    P = fda.flash_deform_attn_channels(1, Kp)
    say(f"[split] flash deformable attention N={n} level {shapes[0]} M={M} D={D}: "
        f"{S * M * D * 4 / 1e9:.2f} GB of value per image")
    gen = torch.Generator(device="cuda").manual_seed(8)
    v = torch.randn((n, S, M, D), device="cuda", generator=gen)
    la = torch.rand((n, Q, M, P), device="cuda", generator=gen)
    la[..., 2 * Kp:3 * Kp] = torch.randn((n, Q, M, Kp), device="cuda", generator=gen)
    la[..., 3 * Kp:] = 0.0
    go = torch.randn((n, Q, M, D), device="cuda", generator=gen)
    out = fda.forward(v, shapes, la, Kp)
    gv, gla = fda.backward(v, shapes, la, go, Kp)
    torch.cuda.synchronize()
    for i in range(n):
        o1 = fda.forward(v[i:i + 1], shapes, la[i:i + 1], Kp)
        gv1, gla1 = fda.backward(v[i:i + 1], shapes, la[i:i + 1], go[i:i + 1], Kp)
        torch.cuda.synchronize()
        assert torch.equal(out[i:i + 1], o1), f"image {i}: output differs"
        assert torch.equal(gla[i:i + 1], gla1), f"image {i}: grad_loc_attn differs"
        assert bool(((gv[i:i + 1] - gv1).abs() <= 1e-5 + 1e-5 * gv1.abs()).all()), f"image {i}: grad_value differs"
    say(f"  {n} images: the split call agrees with the single-image calls")

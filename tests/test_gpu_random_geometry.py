"""Seeded random geometries against the oracle, through the C ABI.

Each case draws its batch, map size, channels per group, group count,
kernel (1, 3, 5 or 7 per axis), stride, padding, dilation, remove_center,
offset_scale, offset spread, storage dtype and the DCNv3 softmax mode from
one seeded generator, so the tile planner meets shapes that the named cases
do not: rectangular and 1-wide kernels, ragged tiles along both axes, maps
from 1 to 200 pixels a side, offsets far beyond the halo, and shapes the
tiled kernels decline (channel rows that are not a power of two of 16-byte
vectors, more than 25 points), which go to the general kernels.  Forward
and backward wherever the library takes the call; where it declines (the
general kernels have no softmax mode and no 16-bit backward) the call must
fail with UNSUPPORTED.  Tolerances as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_vision_amd import dcnv4
from dynamic_sparse_vision_amd.dcnv4 import Dcnv4Error
from dynamic_sparse_vision_amd.workloads import Workload
from tests.test_gpu_parity import check, device_inputs, say

pytestmark = pytest.mark.gpu


def _out_size(size, k, s, p, d):
    return (size + 2 * p - (d * (k - 1) + 1)) // s + 1


def _draw_cases(n_cases, seed=2024, size=(1, 25), batch=(1, 4), prefix="rnd", general=False):
    rng = np.random.RandomState(seed)
    cases = []
    while len(cases) < n_cases:
        dtype = ["fp32", "fp16", "bf16"][rng.randint(3)]
        if general and rng.rand() < 0.5:
            dtype = "fp32"   # the general backward is fp32 only
        kernels = [1, 3, 5]
        if not general:
            cg = int(rng.choice([4, 8, 16, 32] if dtype == "fp32" else [8, 16, 32]))
        elif rng.rand() < 0.5:
            # channel rows of 3, 5 or 6 vectors (not a power of two)
            cg = int(rng.choice([12, 20, 24] if dtype == "fp32" else [24, 40, 48]))
        else:
            # more than 25 points
            cg = int(rng.choice([4, 8, 16] if dtype == "fp32" else [8, 16]))
            kernels = [7]
        g = int(rng.randint(1, 5))
        kh, kw = int(rng.choice(kernels)), int(rng.choice(kernels if len(kernels) > 1 else [5, 7]))
        rc = bool(kh % 2 == 1 and kw % 2 == 1 and kh * kw > 1 and rng.rand() < 0.5)
        sh, sw = int(rng.randint(1, 3)), int(rng.randint(1, 3))
        dh, dw = int(rng.randint(1, 3)), int(rng.randint(1, 3))
        ph, pw = int(rng.randint(0, 3)), int(rng.randint(0, 3))
        H, W = int(rng.randint(*size)), int(rng.randint(*size))
        if _out_size(H, kh, sh, ph, dh) < 1 or _out_size(W, kw, sw, pw, dw) < 1:
            continue
        i = len(cases)
        softmax = bool(rng.rand() < 0.25)
        cases.append((Workload(
            f"{prefix}{i:02d}_{dtype}_{H}x{W}_g{g}c{cg}_k{kh}x{kw}{'rc' if rc else ''}"
            f"_s{sh}{sw}_p{ph}{pw}_d{dh}{dw}",
            N=int(rng.randint(*batch)), H=H, W=W, C=g * cg, G=g, dtype=dtype,
            seed=1000 + i, sigma_value=1.0, sigma_off=float(rng.choice([0.5, 2.0, 6.0, 12.0])),
            sigma_m=0.7, direction="fwd", remove_center=rc,
            integer_offsets=bool(rng.rand() < 0.2), kernel=(kh, kw), stride=(sh, sw),
            pad=(ph, pw), dilation=(dh, dw), offset_scale=float(rng.choice([0.5, 1.0, 1.5]))), softmax))
    return cases


CASES = _draw_cases(160)
# maps of 25 to 96 pixels a side: several output and cell tiles per image,
# ragged along both axes
CASES += _draw_cases(32, seed=2025, size=(25, 97), batch=(1, 3), prefix="big")
# maps of 128 to 200 pixels a side: the backward's cell tiles take a near
# radius of 9 to 11 there (7 below), with offsets far beyond it
CASES += _draw_cases(6, seed=2027, size=(128, 201), batch=(1, 2), prefix="wide")
# shapes the tiled kernels decline (channel rows that are not a power of two
# of 16-byte vectors, more than 25 points): the general kernels
CASES += _draw_cases(48, seed=2026, size=(1, 30), batch=(1, 3), prefix="gen", general=True)


def _tiled(w, backward):
    """The tiled kernels take K <= 25 points and channel rows of a power of
    two of 16-byte vectors; their backward 4 (fp32), 8, 16 or 32 channels
    per group."""
    es = 4 if w.dtype == "fp32" else 2
    nvp = w.Cg * es // 16
    ok = w.K <= 25 and (w.Cg * es) % 16 == 0 and nvp & (nvp - 1) == 0
    return ok and (not backward or w.Cg in (8, 16, 32) or (w.Cg == 4 and es == 4))


def _supported(w, softmax, backward):
    """Whether the library takes the call: the tiled kernels in every dtype
    and mode; else the general kernels, without the softmax mode: the forward
    for 16-byte channel rows, the backward in fp32 with lanes of 4, 8 or 16
    channels, a power of two of them per group."""
    if _tiled(w, backward):
        return True
    es = 4 if w.dtype == "fp32" else 2
    if softmax or (w.Cg * es) % 16 != 0:
        return False
    if not backward:
        return True
    return w.dtype == "fp32" and any(w.Cg % d == 0 and (w.Cg // d) & (w.Cg // d - 1) == 0 for d in (4, 8, 16))


@pytest.mark.parametrize("w,softmax", CASES, ids=lambda x: getattr(x, "name", None) or f"softmax={x}")
def test_random_geometry(w, softmax):
    say(f"[random] {w.name} N={w.N} sigma_off={w.sigma_off} scale={w.offset_scale} "
        f"int={w.integer_offsets} softmax={softmax}")
    d = device_inputs(w, with_grad=True)
    if not _supported(w, softmax, backward=False):
        with pytest.raises(Dcnv4Error, match="UNSUPPORTED"):
            dcnv4.forward(d["v"], d["om"], softmax=softmax, **w.kwargs())
        return
    out = dcnv4.forward(d["v"], d["om"], softmax=softmax, **w.kwargs())
    torch.cuda.synchronize()
    ref = oracle.forward(d["v_ref"], d["om_ref"], softmax=softmax, **w.kwargs())
    check(out.float().cpu().numpy(), ref, w.dtype, f"{w.name} output")
    if not _supported(w, softmax, backward=True):
        with pytest.raises(Dcnv4Error, match="UNSUPPORTED"):
            dcnv4.backward(d["v"], d["om"], d["g"], softmax=softmax, **w.kwargs())
        return
    gv, gom = dcnv4.backward(d["v"], d["om"], d["g"], softmax=softmax, **w.kwargs())
    torch.cuda.synchronize()
    rgv, rgom = oracle.backward(d["v_ref"], d["om_ref"], d["g_ref"], softmax=softmax, **w.kwargs())
    check(gv.cpu().numpy(), rgv, "fp32", f"{w.name} grad_value")
    gom32 = gom.float().cpu().numpy()
    check(gom32, rgom, w.dtype, f"{w.name} grad_offset_mask")
    assert np.all(gom32[..., 3 * w.G * w.K:] == 0), "padding gradient must be 0"

"""Non-finite, huge and far offsets through the DCNv4 kernels, against the
oracle (fp32 and bf16, forward and backward).

include/dcnv4.h: a sample whose location lies outside [-1,H) x [-1,W), or is
NaN, contributes nothing (zero-extended image; walkthrough "DCNv4论文解析",
section 1.2, bilinear sampling of the image).  Offsets here are NaN, +-inf,
+-1e30, +-50 px (outside the map), +-8 to 9 px (inside the map but beyond
the tiles' halo), and ordinary N(0, 2 px) ones, interleaved so that every
wave sees a mix; masks and values stay finite, as the contract requires.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_vision_amd import dcnv4, synth
from dynamic_sparse_vision_amd.workloads import Workload

from tests.test_gpu_parity import check, say

pytestmark = pytest.mark.gpu


def _inputs(dtype, N=2, H=12, W=13, C=32, G=2, kernel=(3, 3), pad=(1, 1), remove_center=False):
    w = Workload(f"edge_{dtype}", N, H, W, C, G, dtype, 91, 1.0, 2.0, 0.7, "bwd", kernel=kernel, pad=pad,
                 remove_center=remove_center)
    v, om, g = w.make_inputs(with_grad=True)
    K = w.K
    off = om[..., :3 * G * K].reshape(N, w.Ho, w.Wo, G, 3 * K)[..., :2 * K]   # view of the offsets
    big = 1e30 if dtype != "fp16" else 6.0e4
    specials = np.array([np.nan, np.inf, -np.inf, big, -big, 50.0, -50.0, 8.5, -8.25, 9.0, -9.0],
                        dtype=np.float32)
    flat = off.reshape(-1, 2 * K)
    rows = np.arange(flat.shape[0])
    for j in range(2 * K):
        pick = (rows * 7 + j * 3) % 5 == 0                  # about one offset in five
        flat[pick, j] = specials[(rows[pick] + j) % len(specials)]
    om[..., :3 * G * K] = np.concatenate(
        [flat.reshape(N, w.Ho, w.Wo, G, 2 * K), om[..., :3 * G * K].reshape(N, w.Ho, w.Wo, G, 3 * K)[..., 2 * K:]],
        axis=-1).reshape(N, w.Ho, w.Wo, 3 * G * K)
    assert np.isnan(om[..., :3 * G * K]).any() and np.isinf(om[..., :3 * G * K]).any()
    return w, v, om, g


# (id, kernel, C, G, remove_center): the 5x5 cases take the 25-point kernels,
# with 16 and 8 channels per group
GEOMETRIES = [("3x3_cg16", (3, 3), 32, 2, False), ("5x5rc_cg16", (5, 5), 32, 2, True),
              ("5x5rc_cg8", (5, 5), 16, 2, True)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("geo", GEOMETRIES, ids=[g[0] for g in GEOMETRIES])
def test_special_offsets_forward_backward(dtype, geo):
    name, kernel, C, G, rc = geo
    pad = (kernel[0] // 2, kernel[1] // 2)
    w, v, om, g = _inputs(dtype, C=C, G=G, kernel=kernel, pad=pad, remove_center=rc)
    say(f"[edge offsets] {dtype} {name}")
    vs, vr = synth.to_storage(v, dtype)
    oms, omr = synth.to_storage(om, dtype)
    gs, gr = synth.to_storage(g, dtype)
    vd, omd, gd = vs.cuda(), oms.cuda(), gs.cuda()
    y = dcnv4.forward(vd, omd, **w.kwargs())
    gv, gom = dcnv4.backward(vd, omd, gd, **w.kwargs())
    torch.cuda.synchronize()
    ref = oracle.forward(vr, omr, **w.kwargs())
    rgv, rgom = oracle.backward(vr, omr, gr, **w.kwargs())
    check(y.float().cpu().numpy(), ref, dtype, "forward")
    # grad_value is fp32 arithmetic on exactly upcast inputs for every dtype
    check(gv.cpu().numpy(), rgv, "fp32", "grad_value")
    gom32 = gom.float().cpu().numpy()
    check(gom32, rgom, dtype, "grad_offset_mask")
    assert np.all(gom32[..., 3 * w.G * w.K:] == 0), "padding gradient must be 0"

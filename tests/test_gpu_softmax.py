"""DCNv3 softmax mode (dcnv4_forward_ex / dcnv4_backward_ex with softmax=1)
against the oracle's softmax mode, element by element; same tolerances as
test_gpu_parity."""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_vision_amd import dcnv4
from dynamic_sparse_vision_amd.workloads import WORKLOADS
from tests.test_gpu_parity import COVERAGE, check, device_inputs, say

pytestmark = pytest.mark.gpu

FWD_CASES = [(WORKLOADS["c2_fwd_fp32_56x56_b64"], 4), (WORKLOADS["c3a_fwd_fp16_56x56x64_g4"], 4),
             (WORKLOADS["c3b_fwd_fp16_28x28x128_g8"], 4), (WORKLOADS["c4_fwd_bf16_270x480_k8"], None)]
FWD_CASES += [(w, None) for w in COVERAGE
              if w.name in ("k5x5_rc_fp32", "dil2_fp32", "stride2_fp16", "k1x1_fp32", "g8_c32_bf16",
                            "far_offsets_fp16", "g5_c16_fp16", "g3_c8_fp32")]

BWD_CASES = [(WORKLOADS["c5_bwd_fp32_56x56_b16"], 4), (WORKLOADS["c2_fwd_fp32_56x56_b64"], 2)]
BWD_CASES += [(w, None) for w in COVERAGE
              if w.name in ("g3_c8_fp32", "g1_c4_fp32", "g2_c32_fp32", "dil2_fp32", "k5x5_rc_fp32",
                            "k1x1_fp32", "int_offsets_fp32", "scale_half_fp32")]


@pytest.mark.parametrize("w,N", FWD_CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_softmax_forward(w, N):
    say(f"[softmax forward] {w.name} N={N or w.N}")
    d = device_inputs(w, N=N)
    out = dcnv4.forward(d["v"], d["om"], softmax=True, **w.kwargs())
    torch.cuda.synchronize()
    ref = oracle.forward(d["v_ref"], d["om_ref"], softmax=True, **w.kwargs())
    check(out.float().cpu().numpy(), ref, w.dtype, f"{w.name} softmax")


@pytest.mark.parametrize("w,N", BWD_CASES, ids=lambda x: getattr(x, "name", str(x)))
def test_softmax_backward(w, N):
    say(f"[softmax backward] {w.name} N={N or w.N}")
    d = device_inputs(w, N=N, with_grad=True)
    gv, gom = dcnv4.backward(d["v"], d["om"], d["g"], softmax=True, **w.kwargs())
    torch.cuda.synchronize()
    rgv, rgom = oracle.backward(d["v_ref"], d["om_ref"], d["g_ref"], softmax=True, **w.kwargs())
    check(gv.cpu().numpy(), rgv, "fp32", f"{w.name} softmax grad_value")
    check(gom.cpu().numpy(), rgom, "fp32", f"{w.name} softmax grad_offset_mask")
    gl = gom.cpu().numpy()[..., :3 * w.G * w.K].reshape(gom.shape[:3] + (w.G, 3 * w.K))[..., 2 * w.K:]
    assert np.abs(gl.sum(axis=-1)).max() < 1e-4, "logit gradients must sum to ~0 over K"

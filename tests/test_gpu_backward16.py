"""fp16 / bf16 backward against the oracle on the same rounded inputs,
element by element: grad_value is fp32 (fp32 arithmetic on exactly upcast
inputs: the fp32 tolerance of test_gpu_parity); grad_offset_mask is rounded
once into the storage dtype (the 16-bit tolerance, 2e-2 + one ulp)."""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_vision_amd import dcnv4
from dynamic_sparse_vision_amd.workloads import WORKLOADS
from tests.test_gpu_parity import COVERAGE, check, device_inputs, say

pytestmark = pytest.mark.gpu

CASES = [(WORKLOADS["c3a_fwd_fp16_56x56x64_g4"], 4, False),
         (WORKLOADS["c3b_fwd_fp16_28x28x128_g8"], 4, False),
         (WORKLOADS["c4_fwd_bf16_270x480_k9"], None, False),
         (WORKLOADS["c4_fwd_bf16_270x480_k8"], None, False),
         (WORKLOADS["c3a_fwd_fp16_56x56x64_g4"], 2, True)]
CASES += [(w, None, False) for w in COVERAGE
          if w.name in ("g5_c16_fp16", "g2_c8_bf16", "g8_c32_bf16", "stride2_fp16", "far_offsets_fp16",
                        "k3x5_s12_d21_bf16")]


@pytest.mark.parametrize("w,N,softmax", CASES,
                         ids=lambda x: getattr(x, "name", None) or str(x))
def test_backward_16bit(w, N, softmax):
    say(f"[backward {w.dtype}] {w.name} N={N or w.N} softmax={softmax}")
    d = device_inputs(w, N=N, with_grad=True)
    gv, gom = dcnv4.backward(d["v"], d["om"], d["g"], softmax=softmax, **w.kwargs())
    torch.cuda.synchronize()
    assert gv.dtype == torch.float32 and gom.dtype == d["om"].dtype
    rgv, rgom = oracle.backward(d["v_ref"], d["om_ref"], d["g_ref"], softmax=softmax, **w.kwargs())
    check(gv.cpu().numpy(), rgv, "fp32", f"{w.name} grad_value")
    gom32 = gom.float().cpu().numpy()
    check(gom32, rgom, w.dtype, f"{w.name} grad_offset_mask")
    assert np.all(gom32[..., 3 * w.G * w.K:] == 0), "padding gradient must be 0"

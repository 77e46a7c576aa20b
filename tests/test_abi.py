"""The C ABI of libdcnv4.so on the CPU: the library loads, exports every
symbol include/*.h declares, and rejects bad arguments before any HIP
call.  No call here reaches a kernel launch: each one fails validation (the
pointers are fake, 16-byte aligned addresses that are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from dynamic_sparse_vision_amd import dcnv4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]

OK, NULL, SHAPE, PARAM, DTYPE, ALIGN, UNSUP, OVERFLOW, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8

# fake device addresses: aligned, far apart, never dereferenced
A, B, Cp, D, E = (ctypes.c_void_p(x) for x in (0x100000000, 0x200000000, 0x300000000,
                                               0x400000000, 0x500000000))


def declared_symbols():
    names = set()
    for h in HEADERS:
        names |= set(re.findall(r"DCNV4_API\s+[\w\s\*]+?\b((?:dcnv4|flash_deform_attn)_\w+)\s*\(",
                                open(h).read()))
    return sorted(names)


def test_header_declares_the_abi():
    assert declared_symbols() == sorted([
        "dcnv4_abi_version", "dcnv4_status_string", "dcnv4_last_hip_error",
        "dcnv4_output_size", "dcnv4_om_channels", "dcnv4_forward", "dcnv4_backward",
        "dcnv4_forward_ex", "dcnv4_backward_ex",
        "flash_deform_attn_channels", "flash_deform_attn_forward", "flash_deform_attn_backward",
        "flash_deform_attn_backward_workspace", "flash_deform_attn_backward_noalloc"])


def test_library_exports_every_declared_symbol():
    lib = dcnv4.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dcnv4.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT ((?:dcnv4|flash_deform_attn)_\w+)", out))
    assert set(declared_symbols()) <= exported
    # nothing else with the prefix leaks out
    assert exported == set(declared_symbols())


def test_version_and_status_strings():
    lib = dcnv4.load()
    assert lib.dcnv4_abi_version() == 3
    for st in (OK, NULL, SHAPE, PARAM, DTYPE, ALIGN, UNSUP, OVERFLOW, HIP):
        assert lib.dcnv4_status_string(st)
    assert lib.dcnv4_status_string(12345) == b"unknown status"
    assert lib.dcnv4_last_hip_error() == b""


@pytest.mark.parametrize("args,expect", [
    ((56, 56, 3, 3, 1, 1, 1, 1, 1, 1), (OK, 56, 56)),
    ((14, 14, 3, 3, 2, 2, 1, 1, 1, 1), (OK, 7, 7)),
    ((9, 8, 5, 3, 1, 2, 4, 1, 2, 1), (OK, 9, 4)),
    ((7, 7, 5, 5, 1, 1, 0, 0, 2, 2), (SHAPE, None, None)),
    ((7, 7, 0, 3, 1, 1, 1, 1, 1, 1), (PARAM, None, None)),
    ((0, 7, 3, 3, 1, 1, 1, 1, 1, 1), (SHAPE, None, None)),
])
def test_output_size(args, expect):
    lib = dcnv4.load()
    ho, wo = ctypes.c_int(-1), ctypes.c_int(-1)
    st = lib.dcnv4_output_size(*args, ctypes.byref(ho), ctypes.byref(wo))
    assert st == expect[0]
    if st == OK:
        assert (ho.value, wo.value) == expect[1:]
    assert lib.dcnv4_output_size(*args, None, None) == NULL


def test_om_channels():
    lib = dcnv4.load()
    assert lib.dcnv4_om_channels(4, 3, 3, 0) == 112       # 108 -> 112
    assert lib.dcnv4_om_channels(16, 3, 3, 0) == 432
    assert lib.dcnv4_om_channels(16, 3, 3, 1) == 384
    assert lib.dcnv4_om_channels(32, 3, 3, 0) == 864
    assert lib.dcnv4_om_channels(1, 3, 3, 0) == 32        # 27 -> 32
    assert lib.dcnv4_om_channels(1, 2, 2, 1) == PARAM     # even kernel with remove_center
    assert lib.dcnv4_om_channels(0, 3, 3, 0) == PARAM


BASE = dict(N=2, H=8, W=8, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, G=4, Cg=16,
            scale=1.0, rc=0, P=112, dtype=0)


def fwd(ptrs=(A, B, Cp), **over):
    a = dict(BASE, **over)
    return dcnv4.load().dcnv4_forward(*ptrs, a["N"], a["H"], a["W"], a["kh"], a["kw"], a["sh"],
                                      a["sw"], a["ph"], a["pw"], a["dh"], a["dw"], a["G"], a["Cg"],
                                      a["scale"], a["rc"], a["P"], a["dtype"], None)


def bwd(ptrs=(A, B, Cp, D, E), **over):
    a = dict(BASE, **over)
    return dcnv4.load().dcnv4_backward(*ptrs, a["N"], a["H"], a["W"], a["kh"], a["kw"], a["sh"],
                                       a["sw"], a["ph"], a["pw"], a["dh"], a["dw"], a["G"],
                                       a["Cg"], a["scale"], a["rc"], a["P"], a["dtype"], None)


def fwd_ex(ptrs=(A, B, Cp), softmax=1, **over):
    a = dict(BASE, **over)
    return dcnv4.load().dcnv4_forward_ex(*ptrs, a["N"], a["H"], a["W"], a["kh"], a["kw"], a["sh"],
                                         a["sw"], a["ph"], a["pw"], a["dh"], a["dw"], a["G"],
                                         a["Cg"], a["scale"], a["rc"], a["P"], softmax, a["dtype"],
                                         None)


def bwd_ex(ptrs=(A, B, Cp, D, E), softmax=1, **over):
    a = dict(BASE, **over)
    return dcnv4.load().dcnv4_backward_ex(*ptrs, a["N"], a["H"], a["W"], a["kh"], a["kw"],
                                          a["sh"], a["sw"], a["ph"], a["pw"], a["dh"], a["dw"],
                                          a["G"], a["Cg"], a["scale"], a["rc"], a["P"], softmax,
                                          a["dtype"], None)


@pytest.mark.parametrize("call", [fwd, bwd, fwd_ex, bwd_ex],
                         ids=["forward", "backward", "forward_ex", "backward_ex"])
@pytest.mark.parametrize("over,expect", [
    (dict(dtype=3), DTYPE),
    (dict(dtype=-1), DTYPE),
    (dict(N=-1), SHAPE),
    (dict(H=0), SHAPE),
    (dict(W=-3), SHAPE),
    (dict(kh=0), PARAM),
    (dict(sw=0), PARAM),
    (dict(ph=-1), PARAM),
    (dict(dw=0), PARAM),
    (dict(G=0), PARAM),
    (dict(Cg=0), PARAM),
    (dict(rc=2), PARAM),
    (dict(rc=1, kh=2, P=112), PARAM),              # remove_center needs odd kernels
    (dict(rc=1, kh=1, kw=1, P=8), PARAM),          # ... and more than one point
    (dict(scale=float("nan")), PARAM),
    (dict(scale=float("inf")), PARAM),
    (dict(P=108), PARAM),                          # not a multiple of 8
    (dict(P=104), PARAM),                          # fewer than 3*G*K
    (dict(H=2, W=2, ph=0, pw=0), SHAPE),           # empty output
    (dict(Cg=2), UNSUP),                           # 8 bytes: not a 128-bit vector
    (dict(H=1 << 16, W=1 << 14, Cg=16, G=4), OVERFLOW),   # one image > 2^31 bytes
])
def test_rejected_before_any_device_work(call, over, expect):
    assert call(**over) == expect


def test_forward_pointer_and_layout_checks():
    assert fwd(ptrs=(None, B, Cp)) == NULL
    assert fwd(ptrs=(A, None, Cp)) == NULL
    assert fwd(ptrs=(A, B, None)) == NULL
    assert fwd(ptrs=(ctypes.c_void_p(0x100000008), B, Cp)) == ALIGN
    assert fwd(ptrs=(A, B, ctypes.c_void_p(0x100000010))) == PARAM      # output overlaps value
    assert fwd(ptrs=(A, B, ctypes.c_void_p(0x200000000 + 32))) == PARAM  # ... overlaps offset_mask
    assert fwd(dtype=1, Cg=4) == UNSUP                                    # 8 bytes of fp16
    assert fwd(N=0, ptrs=(None, None, None)) == OK                        # empty batch: no-op


def test_backward_pointer_and_dtype_checks():
    assert bwd(dtype=1, Cg=4) == UNSUP   # 8 bytes of fp16 per group pixel
    assert bwd(dtype=2, Cg=4) == UNSUP
    for i in range(5):
        ptrs = [A, B, Cp, D, E]
        ptrs[i] = None
        assert bwd(ptrs=tuple(ptrs)) == NULL
    assert bwd(ptrs=(A, B, Cp, ctypes.c_void_p(0x400000004), E)) == ALIGN
    assert bwd(ptrs=(A, B, Cp, ctypes.c_void_p(0x100000040), E)) == PARAM  # grad_value overlaps value
    assert bwd(ptrs=(A, B, Cp, D, ctypes.c_void_p(0x400000010))) == PARAM  # grad outputs overlap
    assert bwd(Cg=12) == UNSUP        # 3 lanes of 4 channels: not a power of two
    assert bwd(N=0, ptrs=(None,) * 5) == OK


def test_softmax_flag_checks():
    for call in (fwd_ex, bwd_ex):
        assert call(softmax=2) == PARAM
        assert call(softmax=-1) == PARAM
        assert call(softmax=1, N=0, ptrs=(None,) * (3 if call is fwd_ex else 5)) == OK
        # K = 49 > 25: only the general kernels could take it, and they have
        # no softmax mode
        assert call(softmax=1, kh=7, kw=7, ph=3, pw=3, P=592) == UNSUP
    assert bwd_ex(softmax=1, dtype=1, Cg=4) == UNSUP
    assert bwd_ex(softmax=0, dtype=2, kh=7, kw=7, ph=3, pw=3, P=592) == UNSUP   # 16-bit: tiled only


def test_binding_refuses_host_tensors():
    import torch

    v = torch.zeros(1, 4, 4, 64)
    om = torch.zeros(1, 4, 4, 112)
    with pytest.raises(ValueError):
        dcnv4.dcnv4_forward(v, om, torch.zeros_like(v), group=4, group_channels=16)


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="only meaningful where no GPU device exists")
def test_valid_call_without_a_device_reports_hip_error():
    # every argument is valid, so the library reaches the HIP runtime, which
    # has no device here: the call must fail with DCNV4_ERR_HIP, not crash
    st = fwd()
    assert st == HIP
    assert dcnv4.load().dcnv4_last_hip_error() != b""


def test_binding_checks_every_shape_before_a_launch():
    """Each tensor's full shape is compared with the geometry in the binding:
    the library sizes its buffer ranges from the geometry, so a wrongly
    shaped tensor must be refused before it is handed over.  (Meta tensors:
    shapes only; a correctly shaped call then stops at the device check.)"""
    import torch

    def t(*shape, dtype=torch.float32):
        return torch.empty(shape, dtype=dtype, device="meta")

    geo = dict(group=4, group_channels=16)
    v, om, out = t(2, 6, 5, 64), t(2, 6, 5, 112), t(2, 6, 5, 64)
    gv, gom = t(2, 6, 5, 64), t(2, 6, 5, 112)
    with pytest.raises(ValueError, match="device tensor"):
        dcnv4.dcnv4_forward(v, om, out, **geo)
    with pytest.raises(ValueError, match="device tensor"):
        dcnv4.dcnv4_backward(v, om, out, gv, gom, **geo)
    bad_fwd = [
        (t(2, 6, 5, 48), om, out, "channels"),          # C != G * C'
        (t(2, 6, 5), om, out, "4-D"),
        (v, t(2, 6, 4, 112), out, "offset_mask"),        # wrong Wo
        (v, t(1, 6, 5, 112), out, "offset_mask"),        # wrong N
        (v, om, t(2, 6, 5, 32), "output"),
        (v, om, t(2, 5, 5, 64), "output"),
    ]
    for vv, oo, yy, what in bad_fwd:
        with pytest.raises(ValueError, match=what):
            dcnv4.dcnv4_forward(vv, oo, yy, **geo)
        with pytest.raises(ValueError, match=what):
            dcnv4.dcnv4_forward_ex(vv, oo, yy, softmax=True, **geo)
    # stride 2: the output grid is 3 x 3
    s2 = dict(geo, stride_h=2, stride_w=2)
    with pytest.raises(ValueError, match="offset_mask"):
        dcnv4.dcnv4_forward(v, om, out, **s2)
    with pytest.raises(ValueError, match="device tensor"):
        dcnv4.dcnv4_forward(v, t(2, 3, 3, 112), t(2, 3, 3, 64), **s2)
    bad_bwd = [
        (out[:, :, :4], gv, gom, "grad_output"),
        (out, t(2, 6, 5, 32), gom, "grad_value"),
        (out, gv, t(2, 6, 5, 104), "grad_offset_mask"),
    ]
    for go, g1, g2, what in bad_bwd:
        with pytest.raises(ValueError, match=what):
            dcnv4.dcnv4_backward(v, om, go, g1, g2, **geo)

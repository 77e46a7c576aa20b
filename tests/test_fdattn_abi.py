"""The flash deformable attention entry points of libdcnv4.so on the CPU:
every rejected argument is refused before any HIP call (the pointers are
fake, 16-byte aligned addresses that are never dereferenced)."""
import ctypes
import os

import pytest

from dynamic_sparse_vision_amd import dcnv4
from dynamic_sparse_vision_amd import flash_deform_attn as fda

OK, NULL, SHAPE, PARAM, DTYPE, ALIGN, UNSUP, OVERFLOW, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8

A, B, Cp, D, E = (ctypes.c_void_p(x) for x in (0x100000000, 0x200000000, 0x300000000,
                                               0x400000000, 0x500000000))
SHAPES = [(8, 10), (4, 5)]   # S = 100


def shapes_arr(shapes):
    flat = [v for hw in shapes for v in hw]
    return (ctypes.c_int * max(1, len(flat)))(*flat), len(shapes)


def fwd(ptrs=(A, B, Cp), shapes=SHAPES, L=None, N=2, S=100, Q=7, M=2, Dh=32, K=4, P=24, dtype=0):
    arr, nl = shapes_arr(shapes)
    return dcnv4.load().flash_deform_attn_forward(ptrs[0], arr, nl if L is None else L, ptrs[1], ptrs[2],
                                                  N, S, Q, M, Dh, K, P, dtype, None)


F = ctypes.c_void_p(0x600000000)   # workspace


def bwd(ptrs=(A, B, Cp, D, E), shapes=SHAPES, L=None, N=2, S=100, Q=7, M=2, Dh=32, K=4, P=24, dtype=0,
        ws=None, ws_bytes=0):
    arr, nl = shapes_arr(shapes)
    return dcnv4.load().flash_deform_attn_backward(ptrs[0], arr, nl if L is None else L, ptrs[1], ptrs[2],
                                                   ptrs[3], ptrs[4], ws, ws_bytes, N, S, Q, M, Dh, K, P, dtype,
                                                   None)


def ws_bytes(shapes=SHAPES, N=2, S=100, Q=7, M=2, Dh=32, K=4, P=24, dtype=0):
    arr, nl = shapes_arr(shapes)
    out = ctypes.c_size_t()
    st = dcnv4.load().flash_deform_attn_backward_workspace(arr, nl, N, S, Q, M, Dh, K, P, dtype, ctypes.byref(out))
    return st, out.value


def test_channels():
    assert fda.flash_deform_attn_channels(4, 4) == 48
    assert fda.flash_deform_attn_channels(3, 3) == 32
    assert fda.flash_deform_attn_channels(1, 1) == 8
    assert dcnv4.load().flash_deform_attn_channels(0, 4) == PARAM
    assert dcnv4.load().flash_deform_attn_channels(16, 9) == PARAM   # L*K = 144 > 128


@pytest.mark.parametrize("call", [fwd, bwd], ids=["forward", "backward"])
@pytest.mark.parametrize("over,expect", [
    (dict(dtype=3), DTYPE),
    (dict(L=0), PARAM),
    (dict(shapes=[(2, 2)] * 17, S=68), PARAM),          # 17 levels
    (dict(K=0), SHAPE),
    (dict(M=0), SHAPE),
    (dict(Dh=0), SHAPE),
    (dict(N=-1), SHAPE),
    (dict(Q=-1), SHAPE),
    (dict(S=99), SHAPE),                                 # sum H_l*W_l = 100
    (dict(shapes=[(8, 10), (0, 5)]), SHAPE),
    (dict(K=65, P=392), PARAM),                          # L*K = 130 > 128
    (dict(P=16), PARAM),                                 # < 3LK = 24
    (dict(P=28), PARAM),                                 # not a multiple of 8
    (dict(Dh=12), UNSUP),
    (dict(Dh=24), UNSUP),                                # 3 lanes: not a power of two
    (dict(shapes=[(1 << 14, 1 << 14)], S=1 << 28, M=1, Dh=8), OVERFLOW),   # one image > 2^31 bytes
])
def test_rejected_before_any_device_work(call, over, expect):
    assert call(**over) == expect


def test_head_dim_limits():
    assert fwd(Dh=128, ptrs=(None, None, None)) == NULL      # 128 passes the shape rules of the forward
    assert bwd(Dh=128, ptrs=(None,) * 5) == UNSUP             # the backward stops at 64


def test_pointer_checks():
    assert fwd(ptrs=(None, B, Cp)) == NULL
    assert fwd(ptrs=(A, B, None)) == NULL
    assert fwd(ptrs=(ctypes.c_void_p(0x100000008), B, Cp)) == ALIGN
    assert fwd(ptrs=(A, B, ctypes.c_void_p(0x100000010))) == PARAM     # output overlaps value
    assert fwd(ptrs=(A, B, ctypes.c_void_p(0x200000000 + 64))) == PARAM  # ... overlaps loc_attn
    assert fwd(N=0, ptrs=(None, None, None)) == OK
    assert fwd(Q=0, ptrs=(None, None, None)) == OK
    for i in range(5):
        ptrs = [A, B, Cp, D, E]
        ptrs[i] = None
        assert bwd(ptrs=tuple(ptrs)) == NULL
    assert bwd(ptrs=(A, B, Cp, ctypes.c_void_p(0x400000004), E)) == ALIGN
    assert bwd(ptrs=(A, B, Cp, ctypes.c_void_p(0x100000040), E)) == PARAM   # grad_value overlaps value
    assert bwd(ptrs=(A, B, Cp, D, ctypes.c_void_p(0x400000010))) == PARAM   # grad outputs overlap
    assert bwd(N=0, ptrs=(None,) * 5) == OK


def test_null_shapes():
    lib = dcnv4.load()
    assert lib.flash_deform_attn_forward(A, None, 2, B, Cp, 2, 100, 7, 2, 32, 4, 24, 0, None) == NULL
    assert lib.flash_deform_attn_backward(A, None, 2, B, Cp, D, E, None, 0, 2, 100, 7, 2, 32, 4, 24, 0, None) == NULL
    out = ctypes.c_size_t()
    assert lib.flash_deform_attn_backward_workspace(None, 2, 2, 100, 7, 2, 32, 4, 24, 0, ctypes.byref(out)) == NULL
    arr, nl = shapes_arr(SHAPES)
    assert lib.flash_deform_attn_backward_workspace(arr, nl, 2, 100, 7, 2, 32, 4, 24, 0, None) == NULL


def test_workspace_size_and_checks():
    # bins: (8+1)*(10+1) + (4+1)*(5+1) = 129 per (image, head); 2 images x 2
    # heads -> 516, rounded up to 576 entries, twice (counts, starts); the
    # sort splits each slice over min(16, Q, ceil(256 / slices)) = 7 blocks,
    # each with its own offsets: 4 * 7 * 129 = 3612 -> 3648 entries; 4 bytes
    # each; per sample (2 * 2 * 7 * 2 * 4 = 224 -> 256 entries) a 4-byte key
    # and two 16-byte records (unsorted, sorted)
    st, n = ws_bytes()
    assert st == OK
    assert n == (2 * 576 + 3648 + 256) * 4 + 2 * 256 * 16
    assert ws_bytes(N=0) == (OK, 0)
    assert ws_bytes(Q=0) == (OK, 0)
    assert ws_bytes(Dh=12)[0] == UNSUP
    assert bwd(ws=F, ws_bytes=n - 1) == PARAM                              # too small
    assert bwd(ws=ctypes.c_void_p(0x600000008), ws_bytes=n) == ALIGN
    assert bwd(ws=ctypes.c_void_p(0x100000000 + 64), ws_bytes=n) == PARAM  # overlaps value
    assert bwd(ws=ctypes.c_void_p(0x400000000 + 64), ws_bytes=n) == PARAM  # overlaps grad_value


def test_binding_checks_every_shape_before_a_launch():
    """Every tensor's full shape is compared in the binding before the
    library is called (meta tensors: shapes only; a correctly shaped call
    stops at the device check)."""
    import torch

    from dynamic_sparse_vision_amd import flash_deform_attn as fda

    def t(*shape, dtype=torch.float32):
        return torch.empty(shape, dtype=dtype, device="meta")

    shapes = ((8, 10), (4, 5))                       # S = 100
    v, la, out = t(2, 100, 2, 32), t(2, 7, 2, 24), t(2, 7, 2, 32)
    gv, gla = t(2, 100, 2, 32), t(2, 7, 2, 24)
    with pytest.raises(ValueError, match="device tensor"):
        fda.flash_deform_attn_forward(v, shapes, la, out, num_points=4)
    with pytest.raises(ValueError, match="device tensor"):
        fda.flash_deform_attn_backward(v, shapes, la, out, gv, gla, num_points=4)
    for vv, ll, yy, what in [(t(2, 99, 2, 32), la, out, "rows"), (v, t(1, 7, 2, 24), out, "loc_attn"),
                             (v, t(2, 7, 3, 24), out, "loc_attn"), (v, la, t(2, 6, 2, 32), "output"),
                             (v, la, t(2, 7, 2, 16), "output")]:
        with pytest.raises(ValueError, match=what):
            fda.flash_deform_attn_forward(vv, shapes, ll, yy, num_points=4)
    for go, g1, g2, what in [(t(2, 7, 2, 16), gv, gla, "grad_output"), (out, t(2, 100, 2, 16), gla, "grad_value"),
                             (out, gv, t(2, 7, 2, 16), "grad_loc_attn")]:
        with pytest.raises(ValueError, match=what):
            fda.flash_deform_attn_backward(v, shapes, la, go, g1, g2, num_points=4)


def bwd_noalloc(ptrs=(A, B, Cp, D, E), shapes=SHAPES, L=None, N=2, S=100, Q=7, M=2, Dh=32, K=4, P=24, dtype=0):
    arr, nl = shapes_arr(shapes)
    return dcnv4.load().flash_deform_attn_backward_noalloc(ptrs[0], arr, nl if L is None else L, ptrs[1], ptrs[2],
                                                           ptrs[3], ptrs[4], N, S, Q, M, Dh, K, P, dtype, None)


def test_noalloc_argument_checks():
    """The no-allocation backward validates like the backward with a
    workspace, before any HIP call."""
    assert bwd_noalloc(dtype=7) == DTYPE
    assert bwd_noalloc(S=99) == SHAPE
    assert bwd_noalloc(P=20) == PARAM
    assert bwd_noalloc(Dh=128) == UNSUP            # the backward takes D <= 64
    assert bwd_noalloc(N=0, ptrs=(None,) * 5) == OK
    for i in range(5):
        ptrs = [A, B, Cp, D, E]
        ptrs[i] = None
        assert bwd_noalloc(ptrs=tuple(ptrs)) == NULL
    assert bwd_noalloc(ptrs=(A, B, Cp, ctypes.c_void_p(0x400000004), E)) == ALIGN
    assert bwd_noalloc(ptrs=(A, B, Cp, ctypes.c_void_p(0x100000040), E)) == PARAM   # grad_value overlaps value


def test_noalloc_refuses_images_larger_than_its_scratch():
    """One image whose sorted-path workspace exceeds the 128 MiB array is
    refused (UNSUPPORTED) before any HIP call; the size limit is the
    workspace the caller-workspace entry point reports for N = 1."""
    limit = 128 << 20
    # one 64x64 level, 8 heads, 4 points: 16 bytes x 2 per sample plus keys
    shapes = [(64, 64)]
    S = 64 * 64
    for Q, expect_fit in ((100_000, True), (300_000, False)):
        st, need = ws_bytes(shapes=shapes, N=1, S=S, Q=Q, M=8, Dh=32, K=4, P=16)
        assert st == OK and (need <= limit) == expect_fit, (Q, need)
    # only the refused call is made (a valid one would reach the runtime)
    assert bwd_noalloc(shapes=shapes, N=1, S=S, Q=300_000, M=8, Dh=32, K=4, P=16) == UNSUP
    assert bwd_noalloc(shapes=shapes, N=3, S=S, Q=300_000, M=8, Dh=32, K=4, P=16) == UNSUP


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="only meaningful where no GPU device exists")
def test_noalloc_valid_call_without_a_device_reports_hip_error():
    assert bwd_noalloc() == HIP
    assert dcnv4.load().dcnv4_last_hip_error() != b""

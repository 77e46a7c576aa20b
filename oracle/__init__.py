"""CPU oracle for the DCNv4 spatial-aggregation operator and for flash
deformable attention (multi-scale deformable attention).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and
by the CPU-baseline leg of the benchmark, never by the product library.  The
arithmetic lives in ``dcnv4_oracle.c`` (plain C, fp32 coordinates and weights,
double accumulation); this module only builds it with gcc and marshals numpy
arrays into it.  It shares no code with the HIP path.

Every function here follows the definition cited in ``dcnv4_oracle.c``
("Efficient Deformable ConvNets", DCNv3 recap equation with the softmax
removed, bilinear sampling with zero padding).  ``softmax=True`` selects the
DCNv3 form, with the masks of each (pixel, group) normalised by a softmax
over the K points.

``fdattn_forward`` / ``fdattn_backward`` wrap ``fdattn_oracle.c`` (the
multi-scale deformable attention definition cited there; its own library).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dcnv4_oracle.c")
_LIB = os.path.join(_HERE, "libdcnv4_oracle.so")
FDA_SRC = os.path.join(_HERE, "fdattn_oracle.c")
FDA_LIB = os.path.join(_HERE, "libfdattn_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = _SRC, out: str = _LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc (always; cheap)."""
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_all() -> None:
    """Compile both oracle libraries."""
    build()
    build(FDA_SRC, FDA_LIB)


_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load the oracle library; build it only if no built copy exists."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != _LIB:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    geo = [i] * 11 + [i, i, f, i, i, i]  # N H W kh kw sh sw ph pw dh dw | G Cg | scale | rc P nthreads
    geo_ex = geo[:-1] + [i, i]   # ... rc P softmax nthreads
    lib.dcnv4o_forward.argtypes = [p, p, p] + geo
    lib.dcnv4o_forward.restype = i
    lib.dcnv4o_backward.argtypes = [p, p, p, p, p] + geo
    lib.dcnv4o_backward.restype = i
    lib.dcnv4o_forward_ex.argtypes = [p, p, p] + geo_ex
    lib.dcnv4o_forward_ex.restype = i
    lib.dcnv4o_backward_ex.argtypes = [p, p, p, p, p] + geo_ex
    lib.dcnv4o_backward_ex.restype = i
    lib.dcnv4o_output_size.argtypes = [i, i, i, i, i]
    lib.dcnv4o_output_size.restype = i
    lib.dcnv4o_grid.argtypes = [i, i, i, p, p]
    lib.dcnv4o_grid.restype = i
    _lib_cache[path] = lib
    return lib


def output_size(H, W, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1,
                pad_h=1, pad_w=1, dilation_h=1, dilation_w=1, lib=None):
    lib = lib or load()
    return (lib.dcnv4o_output_size(H, kernel_h, stride_h, pad_h, dilation_h),
            lib.dcnv4o_output_size(W, kernel_w, stride_w, pad_w, dilation_w))


def grid(kernel_h=3, kernel_w=3, remove_center=False, lib=None):
    """Grid index pairs (i over kernel_w, j over kernel_h) in k order."""
    lib = lib or load()
    gi = np.zeros(kernel_h * kernel_w, np.int32)
    gj = np.zeros(kernel_h * kernel_w, np.int32)
    K = lib.dcnv4o_grid(kernel_h, kernel_w, int(bool(remove_center)),
                        gi.ctypes.data, gj.ctypes.data)
    return list(zip(gi[:K].tolist(), gj[:K].tolist()))


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _geom(value, offset_mask, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
          dilation_h, dilation_w, group, group_channels, offset_scale, remove_center):
    N, H, W, C = value.shape
    if C != group * group_channels:
        raise ValueError("value channels != group * group_channels")
    P = offset_mask.shape[-1]
    return (N, H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
            dilation_h, dilation_w, group, group_channels, float(offset_scale),
            int(bool(remove_center)), P)


def forward(value, offset_mask, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1,
            pad_h=1, pad_w=1, dilation_h=1, dilation_w=1, group=1, group_channels=None,
            offset_scale=1.0, remove_center=False, softmax=False, nthreads=0, lib=None):
    """y (N,Ho,Wo,C) float64 from value (N,H,W,C) and offset_mask (N,Ho,Wo,P).

    Inputs are converted to float32 (exact for fp16/bf16 storage values).
    """
    lib = lib or load()
    value = _f32(value)
    offset_mask = _f32(offset_mask)
    if group_channels is None:
        group_channels = value.shape[-1] // group
    g = _geom(value, offset_mask, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
              dilation_h, dilation_w, group, group_channels, offset_scale, remove_center)
    N, H, W = g[0], g[1], g[2]
    Ho = lib.dcnv4o_output_size(H, kernel_h, stride_h, pad_h, dilation_h)
    Wo = lib.dcnv4o_output_size(W, kernel_w, stride_w, pad_w, dilation_w)
    if offset_mask.shape[:3] != (N, Ho, Wo):
        raise ValueError(f"offset_mask shape {offset_mask.shape} != {(N, Ho, Wo)}+(P,)")
    out = np.zeros((N, Ho, Wo, group * group_channels), np.float64)
    K = lib.dcnv4o_forward_ex(value.ctypes.data, offset_mask.ctypes.data, out.ctypes.data,
                              *g, int(bool(softmax)), int(nthreads))
    if K < 0:
        raise ValueError("oracle rejected the geometry")
    return out


def backward(value, offset_mask, grad_output, kernel_h=3, kernel_w=3, stride_h=1,
             stride_w=1, pad_h=1, pad_w=1, dilation_h=1, dilation_w=1, group=1,
             group_channels=None, offset_scale=1.0, remove_center=False, softmax=False,
             nthreads=0, lib=None):
    """(grad_value (N,H,W,C), grad_offset_mask (N,Ho,Wo,P)), both float64."""
    lib = lib or load()
    value = _f32(value)
    offset_mask = _f32(offset_mask)
    grad_output = _f32(grad_output)
    if group_channels is None:
        group_channels = value.shape[-1] // group
    g = _geom(value, offset_mask, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
              dilation_h, dilation_w, group, group_channels, offset_scale, remove_center)
    N, H, W = g[0], g[1], g[2]
    Ho = lib.dcnv4o_output_size(H, kernel_h, stride_h, pad_h, dilation_h)
    Wo = lib.dcnv4o_output_size(W, kernel_w, stride_w, pad_w, dilation_w)
    if offset_mask.shape[:3] != (N, Ho, Wo) or grad_output.shape != (N, Ho, Wo, value.shape[-1]):
        raise ValueError("shape mismatch")
    gv = np.zeros(value.shape, np.float64)
    gom = np.zeros(offset_mask.shape, np.float64)
    K = lib.dcnv4o_backward_ex(value.ctypes.data, offset_mask.ctypes.data, grad_output.ctypes.data,
                               gv.ctypes.data, gom.ctypes.data, *g, int(bool(softmax)), int(nthreads))
    if K < 0:
        raise ValueError("oracle rejected the geometry")
    return gv, gom


# ------------------------------------------------- flash deformable attention --

def load_fdattn(path: str = FDA_LIB) -> ctypes.CDLL:
    """Load the flash deformable attention oracle; build it if missing."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        if path != FDA_LIB:
            raise FileNotFoundError(path)
        build(FDA_SRC, FDA_LIB)
    lib = ctypes.CDLL(path)
    i, p = ctypes.c_int, ctypes.c_void_p
    dims = [i] * 7  # N S Q M D K P
    lib.fdao_forward.argtypes = [p, p, i, p, p] + dims + [i]
    lib.fdao_forward.restype = i
    lib.fdao_backward.argtypes = [p, p, i, p, p, p, p] + dims + [i]
    lib.fdao_backward.restype = i
    _lib_cache[path] = lib
    return lib


def _fda_dims(value, shapes, loc_attn, points):
    shapes = np.ascontiguousarray(np.asarray(shapes, dtype=np.int32).reshape(-1, 2))
    N, S, M, D = value.shape
    if loc_attn.ndim != 4 or loc_attn.shape[0] != N or loc_attn.shape[2] != M:
        raise ValueError(f"loc_attn shape {loc_attn.shape} does not match value {value.shape}")
    Q, P = loc_attn.shape[1], loc_attn.shape[3]
    return shapes, (N, S, Q, M, D, int(points), P)


def fdattn_forward(value, spatial_shapes, loc_attn, points, nthreads=0, lib=None):
    """out (N,Q,M,D) float64 from value (N,S,M,D), the level shapes (L,2) =
    (H_l, W_l) and loc_attn (N,Q,M,P); inputs are upcast to float32."""
    lib = lib or load_fdattn()
    value = _f32(value)
    loc_attn = _f32(loc_attn)
    shapes, dims = _fda_dims(value, spatial_shapes, loc_attn, points)
    N, S, Q, M, D = dims[:5]
    out = np.zeros((N, Q, M, D), np.float64)
    rc = lib.fdao_forward(value.ctypes.data, shapes.ctypes.data, shapes.shape[0], loc_attn.ctypes.data,
                          out.ctypes.data, *dims, int(nthreads))
    if rc < 0:
        raise ValueError("oracle rejected the arguments")
    return out


def fdattn_backward(value, spatial_shapes, loc_attn, grad_output, points, nthreads=0, lib=None):
    """(grad_value (N,S,M,D), grad_loc_attn (N,Q,M,P)), both float64."""
    lib = lib or load_fdattn()
    value = _f32(value)
    loc_attn = _f32(loc_attn)
    grad_output = _f32(grad_output)
    shapes, dims = _fda_dims(value, spatial_shapes, loc_attn, points)
    N, S, Q, M, D = dims[:5]
    if grad_output.shape != (N, Q, M, D):
        raise ValueError(f"grad_output shape {grad_output.shape} != {(N, Q, M, D)}")
    gv = np.zeros(value.shape, np.float64)
    gla = np.zeros(loc_attn.shape, np.float64)
    rc = lib.fdao_backward(value.ctypes.data, shapes.ctypes.data, shapes.shape[0], loc_attn.ctypes.data,
                           grad_output.ctypes.data, gv.ctypes.data, gla.ctypes.data, *dims, int(nthreads))
    if rc < 0:
        raise ValueError("oracle rejected the arguments")
    return gv, gla

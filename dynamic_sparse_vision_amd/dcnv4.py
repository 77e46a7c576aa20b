"""ctypes binding of libdcnv4.so (argument marshalling only).

The names follow the C ABI in include/dcnv4.h.  ``dcnv4_forward`` and
``dcnv4_backward`` take torch tensors (device memory and the current stream
come from torch) and pass raw pointers and sizes to the library; every step
of the operator runs in the library's HIP kernels.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdcnv4.so")

DCNV4_OK = 0
STATUS = {0: "DCNV4_OK", -1: "DCNV4_ERR_NULL", -2: "DCNV4_ERR_SHAPE", -3: "DCNV4_ERR_PARAM",
          -4: "DCNV4_ERR_DTYPE", -5: "DCNV4_ERR_ALIGN", -6: "DCNV4_ERR_UNSUPPORTED",
          -7: "DCNV4_ERR_OVERFLOW", -8: "DCNV4_ERR_HIP"}
DTYPE_CODES = {"fp32": 0, "fp16": 1, "bf16": 2}

_lib = None


class Dcnv4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.dcnv4_status_string(status).decode()
        hip = lib.dcnv4_last_hip_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg}){' ' + hip if hip else ''}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libdcnv4.so from the package directory (built by
    ``python -m dynamic_sparse_vision_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m dynamic_sparse_vision_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i, f, p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    geo = [i] * 13 + [f, i, i, i, p]  # N H W kh kw sh sw ph pw dh dw G Cg | scale | rc P dtype | stream
    geo_ex = geo[:-2] + [i, i, p]  # ... rc P softmax dtype | stream
    lib.dcnv4_forward.argtypes = [p, p, p] + geo
    lib.dcnv4_forward.restype = i
    lib.dcnv4_backward.argtypes = [p, p, p, p, p] + geo
    lib.dcnv4_backward.restype = i
    lib.dcnv4_forward_ex.argtypes = [p, p, p] + geo_ex
    lib.dcnv4_forward_ex.restype = i
    lib.dcnv4_backward_ex.argtypes = [p, p, p, p, p] + geo_ex
    lib.dcnv4_backward_ex.restype = i
    lib.dcnv4_output_size.argtypes = [i] * 10 + [ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.dcnv4_output_size.restype = i
    lib.dcnv4_om_channels.argtypes = [i, i, i, i]
    lib.dcnv4_om_channels.restype = i
    lib.dcnv4_status_string.argtypes = [i]
    lib.dcnv4_status_string.restype = ctypes.c_char_p
    lib.dcnv4_last_hip_error.argtypes = []
    lib.dcnv4_last_hip_error.restype = ctypes.c_char_p
    lib.dcnv4_abi_version.argtypes = []
    lib.dcnv4_abi_version.restype = i
    # flash deformable attention (include/flash_deform_attn.h)
    ip = ctypes.POINTER(i)
    dims = [i] * 8 + [p]   # N S Q M D K P dtype | stream
    lib.flash_deform_attn_channels.argtypes = [i, i]
    lib.flash_deform_attn_channels.restype = i
    lib.flash_deform_attn_forward.argtypes = [p, ip, i, p, p] + dims
    lib.flash_deform_attn_forward.restype = i
    lib.flash_deform_attn_backward.argtypes = [p, ip, i, p, p, p, p, p, ctypes.c_size_t] + dims
    lib.flash_deform_attn_backward.restype = i
    lib.flash_deform_attn_backward_workspace.argtypes = [ip, i] + [i] * 8 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.flash_deform_attn_backward_workspace.restype = i
    lib.flash_deform_attn_backward_noalloc.argtypes = [p, ip, i, p, p, p, p] + dims
    lib.flash_deform_attn_backward_noalloc.restype = i
    _lib = lib
    return lib


def dcnv4_abi_version() -> int:
    return load().dcnv4_abi_version()


def dcnv4_status_string(status: int) -> str:
    return load().dcnv4_status_string(status).decode()


def dcnv4_last_hip_error() -> str:
    return load().dcnv4_last_hip_error().decode()


def dcnv4_output_size(H, W, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1,
                      dilation_h=1, dilation_w=1):
    ho, wo = ctypes.c_int(), ctypes.c_int()
    st = load().dcnv4_output_size(H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                                  dilation_h, dilation_w, ctypes.byref(ho), ctypes.byref(wo))
    if st != DCNV4_OK:
        raise Dcnv4Error(st, "dcnv4_output_size")
    return ho.value, wo.value


def dcnv4_om_channels(group, kernel_h=3, kernel_w=3, remove_center=False) -> int:
    st = load().dcnv4_om_channels(group, kernel_h, kernel_w, int(bool(remove_center)))
    if st < 0:
        raise Dcnv4Error(st, "dcnv4_om_channels")
    return st


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (channel-last, dense)")


def _expect_shape(t, name, want):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _check_geometry(value, offset_mask, outs, *, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                    dilation_h, dilation_w, group, group_channels, remove_center):
    """Every tensor's full shape against the call's geometry, before any
    launch (the library sizes its buffer ranges from the geometry, so a
    wrongly sized tensor would be read or written out of bounds).  ``outs``:
    (tensor, name, "pixel" | "value" | "offset_mask") triples: per output
    pixel (N,Ho,Wo,C), like value, or like offset_mask.  Invalid scalar
    parameters, and offset_mask's entry count P (passed to the library as
    om_channels), are left to the library, which reports their status code."""
    if value.dim() != 4:
        raise ValueError(f"value must be 4-D (N,H,W,C), got shape {tuple(value.shape)}")
    N, H, W, C = value.shape
    if C != group * group_channels:
        raise ValueError(f"value has C={C} channels, expected group*group_channels = "
                         f"{group}*{group_channels}")
    try:
        Ho, Wo = dcnv4_output_size(H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                                   dilation_h, dilation_w)
    except Dcnv4Error:
        return   # the library rejects the parameters with its own status
    if offset_mask.dim() != 4 or tuple(offset_mask.shape[:3]) != (N, Ho, Wo):
        raise ValueError(f"offset_mask has shape {tuple(offset_mask.shape)}, expected ({N}, {Ho}, {Wo}, P)")
    for t, name, kind in outs:
        want = {"pixel": (N, Ho, Wo, C), "value": tuple(value.shape),
                "offset_mask": tuple(offset_mask.shape)}[kind]
        _expect_shape(t, name, want)


def _stream_ptr(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dcnv4_forward(value, offset_mask, output, *, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1,
                  pad_h=1, pad_w=1, dilation_h=1, dilation_w=1, group, group_channels,
                  offset_scale=1.0, remove_center=False, stream=None) -> None:
    """value (N,H,W,C), offset_mask (N,Ho,Wo,P), output (N,Ho,Wo,C): device
    tensors of one dtype.  Enqueues the forward on ``stream`` (default: torch's
    current stream)."""
    dcnv4_forward_ex(value, offset_mask, output, kernel_h=kernel_h, kernel_w=kernel_w,
                     stride_h=stride_h, stride_w=stride_w, pad_h=pad_h, pad_w=pad_w,
                     dilation_h=dilation_h, dilation_w=dilation_w, group=group,
                     group_channels=group_channels, offset_scale=offset_scale,
                     remove_center=remove_center, softmax=False, stream=stream, _name="dcnv4_forward")


def dcnv4_forward_ex(value, offset_mask, output, *, kernel_h=3, kernel_w=3, stride_h=1, stride_w=1,
                     pad_h=1, pad_w=1, dilation_h=1, dilation_w=1, group, group_channels,
                     offset_scale=1.0, remove_center=False, softmax=False, stream=None,
                     _name="dcnv4_forward_ex") -> None:
    """dcnv4_forward with the DCNv3 softmax over the K masks when ``softmax``."""
    _check_geometry(value, offset_mask, [(output, "output", "pixel")], kernel_h=kernel_h, kernel_w=kernel_w,
                    stride_h=stride_h, stride_w=stride_w, pad_h=pad_h, pad_w=pad_w, dilation_h=dilation_h,
                    dilation_w=dilation_w, group=group, group_channels=group_channels,
                    remove_center=remove_center)
    for t, nm in ((value, "value"), (offset_mask, "offset_mask"), (output, "output")):
        _check(t, nm)
        if t.dtype != value.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} != value dtype {value.dtype}")
    N, H, W, C = value.shape
    lib = load()
    args = (ctypes.c_void_p(value.data_ptr()), ctypes.c_void_p(offset_mask.data_ptr()),
            ctypes.c_void_p(output.data_ptr()), N, H, W, kernel_h, kernel_w, stride_h, stride_w,
            pad_h, pad_w, dilation_h, dilation_w, group, group_channels, float(offset_scale),
            int(bool(remove_center)), offset_mask.shape[-1])
    if _name == "dcnv4_forward":
        st = lib.dcnv4_forward(*args, _dtype_code(value), _stream_ptr(stream))
    else:
        st = lib.dcnv4_forward_ex(*args, int(bool(softmax)), _dtype_code(value), _stream_ptr(stream))
    if st != DCNV4_OK:
        raise Dcnv4Error(st, _name)


def dcnv4_backward(value, offset_mask, grad_output, grad_value, grad_offset_mask, *, kernel_h=3,
                   kernel_w=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1, dilation_h=1,
                   dilation_w=1, group, group_channels, offset_scale=1.0, remove_center=False,
                   stream=None) -> None:
    """Backward into caller-allocated grad_value (N,H,W,C) float32 and
    grad_offset_mask (N,Ho,Wo,P) in the inputs' dtype (both overwritten)."""
    dcnv4_backward_ex(value, offset_mask, grad_output, grad_value, grad_offset_mask,
                      kernel_h=kernel_h, kernel_w=kernel_w, stride_h=stride_h, stride_w=stride_w,
                      pad_h=pad_h, pad_w=pad_w, dilation_h=dilation_h, dilation_w=dilation_w,
                      group=group, group_channels=group_channels, offset_scale=offset_scale,
                      remove_center=remove_center, softmax=False, stream=stream,
                      _name="dcnv4_backward")


def dcnv4_backward_ex(value, offset_mask, grad_output, grad_value, grad_offset_mask, *, kernel_h=3,
                      kernel_w=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1, dilation_h=1,
                      dilation_w=1, group, group_channels, offset_scale=1.0, remove_center=False,
                      softmax=False, stream=None, _name="dcnv4_backward_ex") -> None:
    """dcnv4_backward with the DCNv3 softmax over the K masks when ``softmax``
    (the mask gradient is then taken with respect to the logits)."""
    import torch

    _check_geometry(value, offset_mask, [(grad_output, "grad_output", "pixel"), (grad_value, "grad_value", "value"),
                                         (grad_offset_mask, "grad_offset_mask", "offset_mask")],
                    kernel_h=kernel_h, kernel_w=kernel_w, stride_h=stride_h, stride_w=stride_w, pad_h=pad_h,
                    pad_w=pad_w, dilation_h=dilation_h, dilation_w=dilation_w, group=group,
                    group_channels=group_channels, remove_center=remove_center)
    for t, nm in ((value, "value"), (offset_mask, "offset_mask"), (grad_output, "grad_output"),
                  (grad_value, "grad_value"), (grad_offset_mask, "grad_offset_mask")):
        _check(t, nm)
        want = torch.float32 if nm == "grad_value" else value.dtype
        if t.dtype != want:
            raise TypeError(f"{nm} dtype {t.dtype} != {want}")
    N, H, W, C = value.shape
    lib = load()
    args = (ctypes.c_void_p(value.data_ptr()), ctypes.c_void_p(offset_mask.data_ptr()),
            ctypes.c_void_p(grad_output.data_ptr()), ctypes.c_void_p(grad_value.data_ptr()),
            ctypes.c_void_p(grad_offset_mask.data_ptr()), N, H, W, kernel_h, kernel_w, stride_h,
            stride_w, pad_h, pad_w, dilation_h, dilation_w, group, group_channels,
            float(offset_scale), int(bool(remove_center)), offset_mask.shape[-1])
    if _name == "dcnv4_backward":
        st = lib.dcnv4_backward(*args, _dtype_code(value), _stream_ptr(stream))
    else:
        st = lib.dcnv4_backward_ex(*args, int(bool(softmax)), _dtype_code(value), _stream_ptr(stream))
    if st != DCNV4_OK:
        raise Dcnv4Error(st, _name)


def forward(value, offset_mask, **params):
    """Allocate the output with torch and call dcnv4_forward (dcnv4_forward_ex
    when ``softmax=True`` is among the parameters)."""
    import torch

    N, H, W, C = value.shape
    Ho, Wo = dcnv4_output_size(H, W, params.get("kernel_h", 3), params.get("kernel_w", 3),
                               params.get("stride_h", 1), params.get("stride_w", 1),
                               params.get("pad_h", 1), params.get("pad_w", 1),
                               params.get("dilation_h", 1), params.get("dilation_w", 1))
    out = torch.empty((N, Ho, Wo, C), dtype=value.dtype, device=value.device)
    if params.get("softmax"):
        dcnv4_forward_ex(value, offset_mask, out, **params)
    else:
        params.pop("softmax", None)
        dcnv4_forward(value, offset_mask, out, **params)
    return out


def backward(value, offset_mask, grad_output, **params):
    """Allocate grad_value / grad_offset_mask with torch and call dcnv4_backward
    (dcnv4_backward_ex when ``softmax=True`` is among the parameters)."""
    import torch

    gv = torch.empty(value.shape, dtype=torch.float32, device=value.device)
    gom = torch.empty_like(offset_mask)
    if params.get("softmax"):
        dcnv4_backward_ex(value, offset_mask, grad_output, gv, gom, **params)
    else:
        params.pop("softmax", None)
        dcnv4_backward(value, offset_mask, grad_output, gv, gom, **params)
    return gv, gom

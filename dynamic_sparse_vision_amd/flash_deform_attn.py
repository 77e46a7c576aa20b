"""ctypes binding of the flash deformable attention entry points of
libdcnv4.so (argument marshalling only; include/flash_deform_attn.h).

Tensors are torch device tensors (memory and the current stream come from
torch); ``spatial_shapes`` is a host sequence of (H_l, W_l) pairs.  Every
step of the operator runs in the library's HIP kernels; a missing library
or a failing call raises.
"""
from __future__ import annotations

import ctypes

from .dcnv4 import DCNV4_OK, Dcnv4Error, _check, _dtype_code, _stream_ptr, load


def _shapes_arg(spatial_shapes):
    flat = [int(v) for hw in spatial_shapes for v in hw]
    if len(flat) % 2:
        raise ValueError("spatial_shapes must be (H, W) pairs")
    arr = (ctypes.c_int * max(1, len(flat)))(*flat)
    return arr, len(flat) // 2


def _check_shapes(value, spatial_shapes, loc_attn, outs):
    """Every tensor's full shape, before any launch: value (N,S,M,D) with
    S = sum of H_l*W_l; loc_attn (N,Q,M,P) (P, passed as loc_attn_channels,
    is checked by the library); ``outs``: (tensor, name, "query" | "value" |
    "loc_attn") triples, shaped (N,Q,M,D), like value, or like loc_attn."""
    if value.dim() != 4:
        raise ValueError(f"value must be 4-D (N,S,M,D), got shape {tuple(value.shape)}")
    N, S, M, D = value.shape
    want_s = sum(int(h) * int(w) for h, w in spatial_shapes)
    if S != want_s:
        raise ValueError(f"value has S={S} rows, the levels hold {want_s} pixels")
    if loc_attn.dim() != 4 or loc_attn.shape[0] != N or loc_attn.shape[2] != M:
        raise ValueError(f"loc_attn has shape {tuple(loc_attn.shape)}, expected ({N}, Q, {M}, P)")
    Q = loc_attn.shape[1]
    for t, name, kind in outs:
        want = {"query": (N, Q, M, D), "value": tuple(value.shape), "loc_attn": tuple(loc_attn.shape)}[kind]
        if tuple(t.shape) != want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")


def flash_deform_attn_channels(num_levels: int, num_points: int) -> int:
    st = load().flash_deform_attn_channels(num_levels, num_points)
    if st < 0:
        raise Dcnv4Error(st, "flash_deform_attn_channels")
    return st


def flash_deform_attn_forward(value, spatial_shapes, loc_attn, output, *, num_points, stream=None) -> None:
    """value (N,S,M,D), loc_attn (N,Q,M,P), output (N,Q,M,D): device tensors
    of one dtype.  Enqueues the forward on ``stream`` (default: torch's
    current stream)."""
    _check_shapes(value, spatial_shapes, loc_attn, [(output, "output", "query")])
    for t, nm in ((value, "value"), (loc_attn, "loc_attn"), (output, "output")):
        _check(t, nm)
        if t.dtype != value.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} != value dtype {value.dtype}")
    N, S, M, D = value.shape
    Q, P = loc_attn.shape[1], loc_attn.shape[3]
    arr, L = _shapes_arg(spatial_shapes)
    st = load().flash_deform_attn_forward(
        ctypes.c_void_p(value.data_ptr()), arr, L, ctypes.c_void_p(loc_attn.data_ptr()),
        ctypes.c_void_p(output.data_ptr()), N, S, Q, M, D, int(num_points), P, _dtype_code(value),
        _stream_ptr(stream))
    if st != DCNV4_OK:
        raise Dcnv4Error(st, "flash_deform_attn_forward")


def flash_deform_attn_backward_workspace(value, spatial_shapes, loc_attn, *, num_points) -> int:
    """Workspace bytes the sorted grad_value path needs for these tensors."""
    N, S, M, D = value.shape
    Q, P = loc_attn.shape[1], loc_attn.shape[3]
    arr, L = _shapes_arg(spatial_shapes)
    nbytes = ctypes.c_size_t()
    st = load().flash_deform_attn_backward_workspace(arr, L, N, S, Q, M, D, int(num_points), P,
                                                     _dtype_code(value), ctypes.byref(nbytes))
    if st != DCNV4_OK:
        raise Dcnv4Error(st, "flash_deform_attn_backward_workspace")
    return nbytes.value


def flash_deform_attn_backward(value, spatial_shapes, loc_attn, grad_output, grad_value, grad_loc_attn, *,
                               num_points, workspace=None, stream=None) -> None:
    """Backward into caller-allocated grad_value (N,S,M,D) float32 and
    grad_loc_attn (N,Q,M,P) in the inputs' dtype (both overwritten).

    ``workspace``: a device tensor of at least
    ``flash_deform_attn_backward_workspace`` bytes selects the sorted
    (gather) grad_value path; None selects the device-atomic path."""
    import torch

    _check_shapes(value, spatial_shapes, loc_attn, [(grad_output, "grad_output", "query"),
                                                    (grad_value, "grad_value", "value"),
                                                    (grad_loc_attn, "grad_loc_attn", "loc_attn")])
    for t, nm in ((value, "value"), (loc_attn, "loc_attn"), (grad_output, "grad_output"),
                  (grad_value, "grad_value"), (grad_loc_attn, "grad_loc_attn")):
        _check(t, nm)
        want = torch.float32 if nm == "grad_value" else value.dtype
        if t.dtype != want:
            raise TypeError(f"{nm} dtype {t.dtype} != {want}")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _check(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    N, S, M, D = value.shape
    Q, P = loc_attn.shape[1], loc_attn.shape[3]
    arr, L = _shapes_arg(spatial_shapes)
    st = load().flash_deform_attn_backward(
        ctypes.c_void_p(value.data_ptr()), arr, L, ctypes.c_void_p(loc_attn.data_ptr()),
        ctypes.c_void_p(grad_output.data_ptr()), ctypes.c_void_p(grad_value.data_ptr()),
        ctypes.c_void_p(grad_loc_attn.data_ptr()), ctypes.c_void_p(ws_ptr), ws_bytes, N, S, Q, M, D,
        int(num_points), P, _dtype_code(value), _stream_ptr(stream))
    if st != DCNV4_OK:
        raise Dcnv4Error(st, "flash_deform_attn_backward")


def flash_deform_attn_backward_noalloc(value, spatial_shapes, loc_attn, grad_output, grad_value, grad_loc_attn, *,
                                       num_points, stream=None) -> None:
    """flash_deform_attn_backward without a workspace argument and without
    any allocation: the library's own per-device scratch array stands in for
    the workspace.  Calls that overlap on one device race (they share the
    array); calls ordered on one stream do not."""
    import torch

    _check_shapes(value, spatial_shapes, loc_attn, [(grad_output, "grad_output", "query"),
                                                    (grad_value, "grad_value", "value"),
                                                    (grad_loc_attn, "grad_loc_attn", "loc_attn")])
    for t, nm in ((value, "value"), (loc_attn, "loc_attn"), (grad_output, "grad_output"),
                  (grad_value, "grad_value"), (grad_loc_attn, "grad_loc_attn")):
        _check(t, nm)
        want = torch.float32 if nm == "grad_value" else value.dtype
        if t.dtype != want:
            raise TypeError(f"{nm} dtype {t.dtype} != {want}")
    N, S, M, D = value.shape
    Q, P = loc_attn.shape[1], loc_attn.shape[3]
    arr, L = _shapes_arg(spatial_shapes)
    st = load().flash_deform_attn_backward_noalloc(
        ctypes.c_void_p(value.data_ptr()), arr, L, ctypes.c_void_p(loc_attn.data_ptr()),
        ctypes.c_void_p(grad_output.data_ptr()), ctypes.c_void_p(grad_value.data_ptr()),
        ctypes.c_void_p(grad_loc_attn.data_ptr()), N, S, Q, M, D, int(num_points), P, _dtype_code(value),
        _stream_ptr(stream))
    if st != DCNV4_OK:
        raise Dcnv4Error(st, "flash_deform_attn_backward_noalloc")


def forward(value, spatial_shapes, loc_attn, num_points):
    """Allocate the output (N,Q,M,D) with torch and call the forward."""
    import torch

    N, S, M, D = value.shape
    out = torch.empty((N, loc_attn.shape[1], M, D), dtype=value.dtype, device=value.device)
    flash_deform_attn_forward(value, spatial_shapes, loc_attn, out, num_points=num_points)
    return out


def workspace_for(value, spatial_shapes, loc_attn, num_points):
    """A torch-allocated workspace for the sorted backward (None if empty)."""
    import torch

    nbytes = flash_deform_attn_backward_workspace(value, spatial_shapes, loc_attn, num_points=num_points)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=value.device)


def backward(value, spatial_shapes, loc_attn, grad_output, num_points, sorted_grad_value=True):
    """Allocate grad_value (fp32), grad_loc_attn and (for the sorted path)
    the workspace with torch and call the backward."""
    import torch

    gv = torch.empty(value.shape, dtype=torch.float32, device=value.device)
    gla = torch.empty_like(loc_attn)
    ws = workspace_for(value, spatial_shapes, loc_attn, num_points) if sorted_grad_value else None
    flash_deform_attn_backward(value, spatial_shapes, loc_attn, grad_output, gv, gla, num_points=num_points,
                               workspace=ws)
    return gv, gla

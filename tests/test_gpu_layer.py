"""The DCNv4 layer (projections + operator, dynamic_sparse_vision_amd.layer)
on the GPU against a float64 CPU composition around the oracle, forward and
backward (torch autograd on the GPU; hand-written chain rule around
oracle.backward on the CPU).

Inputs and weights are dyadic (few significant bits), so every projection
result is exact in fp32 on both sides and the offsets reach the operator
bit-identical (floor() of a sampling coordinate never differs between the
two paths).  Tolerances are the operator's fp32 bound (1e-5 + 1e-5*|ref|)
carried through the projections that follow it:
|err(A @ W)| <= err(A) @ |W| + 2^-22 * (|A| @ |W|)  (fp32 sums of <= 256 terms).
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_vision_amd import layer

pytestmark = pytest.mark.gpu

CFGS = [
    ("base", layer.LayerConfig(channels=64, group=4), 4, 20, 20),
    ("dw_softmax_rc", layer.LayerConfig(channels=64, group=4, dw_kernel_size=3, softmax=True,
                                        remove_center=True, output_bias=False), 2, 13, 17),
    ("g8_c128", layer.LayerConfig(channels=128, group=8), 2, 14, 14),
    ("no_pointwise_stride2", layer.LayerConfig(channels=32, group=2, stride=2, without_pointwise=True),
     2, 15, 12),
]


def dyadic(t, bits):
    return torch.round(t * 2.0 ** bits) / 2.0 ** bits


def op_tol(ref):
    return 1e-5 + 1e-5 * np.abs(ref)


def mm_bound(err_a, a, w):
    """Error bound of a @ w given the elementwise error bound of a."""
    return err_a @ np.abs(w) + 2.0 ** -22 * (np.abs(a) @ np.abs(w))


def close(gpu, ref, bound, what):
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    print(f"  {what}: max|err| {err.max():.3e}  max bound {np.max(bound):.3e}", flush=True)
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} of {err.size} out of bound"


@pytest.mark.parametrize("name,cfg,N,H,W", CFGS, ids=[c[0] for c in CFGS])
def test_layer_forward_backward(name, cfg, N, H, W):
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.backends.cudnn.allow_tf32 = False
    print(f"[layer] {name} N={N} {H}x{W} C={cfg.channels} G={cfg.group}", flush=True)
    g = torch.Generator().manual_seed(5)
    C = cfg.channels
    x64 = dyadic(torch.randn(N, H, W, C, generator=g, dtype=torch.float64), 4)
    # 7 fractional bits for the linear weights, 3 for the depthwise kernel:
    # every projection stays within fp32's 24 significant bits
    w = {k: dyadic(v.double().cpu(), 3 if k.endswith("_dw") else 7)
         for k, v in layer.init_weights(cfg, "cpu", torch.float64, seed=3).items()}
    # device copies (exact in fp32)
    xd = x64.float().cuda().requires_grad_(True)
    wd = {k: v.float().cuda().requires_grad_(True) for k, v in w.items()}
    out = layer.layer_forward(xd, wd, cfg)
    d_out = dyadic(torch.randn(out.shape, generator=g, dtype=torch.float64), 4)
    out.backward(d_out.float().cuda())
    torch.cuda.synchronize()

    # CPU reference: float64 projections, the oracle on fp32 copies
    x = x64.numpy()
    prm = cfg.op_params()
    okw = {k: v for k, v in prm.items()}
    value = x if cfg.without_pointwise else x @ w["w_v"].numpy() + w["b_v"].numpy()
    xo_t = x64.clone().requires_grad_(True)
    if cfg.dw_kernel_size:
        xc = torch.nn.functional.conv2d(xo_t.permute(0, 3, 1, 2), w["w_dw"], w["b_dw"],
                                        padding=(cfg.dw_kernel_size - 1) // 2, groups=C)
        xo_t2 = xc.permute(0, 2, 3, 1)
    else:
        xo_t2 = xo_t
    xo_t2 = layer.centre_features(xo_t2, cfg)
    xo = xo_t2.detach().numpy()
    om = xo @ w["w_om"].numpy() + w["b_om"].numpy()
    v32, om32 = value.astype(np.float32), om.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), value) and np.array_equal(om32.astype(np.float64), om), \
        "projections must be exact in fp32 (dyadic inputs)"
    y = oracle.forward(v32, om32, **okw)
    dy_full = d_out.numpy()
    if cfg.without_pointwise:
        ref_out, dy, y_tol = y, dy_full, op_tol(y)
        out_bound = y_tol
    else:
        wo = w["w_o"].numpy()
        ref_out = y @ wo + (w["b_o"].numpy() if "b_o" in w else 0.0)
        y_tol = op_tol(y)
        out_bound = mm_bound(y_tol, y, wo)
        dy = dy_full @ wo.T        # exact: dyadic d_out and weights
    close(out.detach().cpu().numpy(), ref_out, out_bound, f"{name} out")

    gv, gom = oracle.backward(v32, om32, dy.astype(np.float32), **okw)
    gv_tol, gom_tol = op_tol(gv), op_tol(gom)
    # grads of the projections
    if not cfg.without_pointwise:
        wv = w["w_v"].numpy()
        yf = y.reshape(-1, C)
        close(wd["w_o"].grad.cpu().numpy(), yf.T @ dy_full.reshape(-1, C),
              mm_bound(y_tol.reshape(-1, C).T, yf.T, dy_full.reshape(-1, C)), f"{name} dW_o")
        close(wd["w_v"].grad.cpu().numpy(), x.reshape(-1, C).T @ gv.reshape(-1, C),
              mm_bound(gv_tol.reshape(-1, C).T, gv.reshape(-1, C).T, x.reshape(-1, C)).T, f"{name} dW_v")
        close(wd["b_v"].grad.cpu().numpy(), gv.reshape(-1, C).sum(0),
              gv_tol.reshape(-1, C).sum(0) + 2.0 ** -22 * np.abs(gv).reshape(-1, C).sum(0), f"{name} db_v")
        dx_v = gv @ wv.T
        dx_v_bound = mm_bound(gv_tol, gv, wv.T)
    else:
        dx_v, dx_v_bound = gv, gv_tol
    wom = w["w_om"].numpy()
    P = om.shape[-1]
    close(wd["w_om"].grad.cpu().numpy(), xo.reshape(-1, C).T @ gom.reshape(-1, P),
          mm_bound(gom_tol.reshape(-1, P).T, gom.reshape(-1, P).T, xo.reshape(-1, C)).T, f"{name} dW_om")
    dxo = gom @ wom.T
    dxo_bound = mm_bound(gom_tol, gom, wom.T)
    if cfg.dw_kernel_size or cfg.stride > 1:
        (dx_o,) = torch.autograd.grad(xo_t2, xo_t, torch.from_numpy(dxo))
        dx_o = dx_o.numpy()
        # the bound carried through the depthwise convolution's backward with
        # |kernel| (plus its own fp32 rounding)
        xb = torch.zeros_like(x64, requires_grad=True)
        cb = xb
        if cfg.dw_kernel_size:
            cb = torch.nn.functional.conv2d(xb.permute(0, 3, 1, 2), w["w_dw"].abs(), None,
                                            padding=(cfg.dw_kernel_size - 1) // 2, groups=C).permute(0, 2, 3, 1)
        cb = layer.centre_features(cb, cfg)
        (dx_o_bound,) = torch.autograd.grad(cb, xb, torch.from_numpy(dxo_bound + 2.0 ** -21 * np.abs(dxo)))
        dx_o_bound = dx_o_bound.numpy()
    else:
        dx_o, dx_o_bound = dxo, dxo_bound
    close(xd.grad.cpu().numpy(), dx_v + dx_o, dx_v_bound + dx_o_bound, f"{name} dx")

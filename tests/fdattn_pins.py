"""Pins that tie the flash deformable attention oracle to something other
than itself.

Each ``pin_*`` function takes a loaded oracle library (ctypes handle, see
``oracle.load_fdattn``) and raises AssertionError when the oracle disagrees
with an independent fact of multi-scale deformable attention (Zhu et al.,
"Deformable DETR", equation 3, with the locations and logits of a (query,
head) in one row and the softmax applied inside the operator):

* a library routine: ``torch.nn.functional.grid_sample`` (bilinear, zeros,
  align_corners=False: pixel centres at (c + 1/2) / W in normalised units)
  and ``torch.softmax``, with autograd, all in float64;
* closed forms: exact gathers at pixel centres, constant maps (the weights
  sum to 1), affine maps (bilinear sampling reproduces them, so the
  location gradient is the slope times the map size);
* algebra: invariance of every output to a common shift of the logits, the
  zero sum of the logit gradients, the adjoint identity of grad_value
  (the output is linear in the value), finite differences for the locations
  (exact inside a cell) and the logits;
* explicit boundary samples at -1, at size - 1 and just below size.

The row layout (L*K (u, v) pairs, level-major, then L*K logits, then
padding) is encoded here independently of the oracle's source.  The same
functions run against oracle builds with planted mistakes
(tests/test_fdattn_mutants.py).
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def P_of(L, K):
    return (3 * L * K + 7) // 8 * 8


def pack(loc, logits, P=None, pad=np.nan):
    """loc (N,Q,M,L,K,2) and logits (N,Q,M,L,K) -> (N,Q,M,P) rows."""
    N, Q, M, L, K = logits.shape
    P = P or P_of(L, K)
    row = np.full((N, Q, M, P), pad, np.float32)
    row[..., :2 * L * K] = loc.reshape(N, Q, M, 2 * L * K)
    row[..., 2 * L * K:3 * L * K] = logits.reshape(N, Q, M, L * K)
    return row


class Case:
    """A random problem; locations are multiples of 2**-bits so that every
    sampling coordinate and bilinear weight is exact in fp32."""

    def __init__(self, seed=0, N=2, Q=5, M=2, D=3, K=3, shapes=((4, 8), (2, 4), (5, 3)),
                 bits=10, lo=-0.2, hi=1.2, logit_sigma=1.0):
        rng = np.random.default_rng(seed)
        self.shapes = [tuple(s) for s in shapes]
        self.N, self.Q, self.M, self.D, self.K, self.L = N, Q, M, D, K, len(shapes)
        self.S = sum(h * w for h, w in self.shapes)
        self.value = rng.standard_normal((N, self.S, M, D)).astype(np.float32)
        self.loc = (np.round(rng.uniform(lo, hi, (N, Q, M, self.L, K, 2)) * 2 ** bits) / 2 ** bits).astype(np.float32)
        self.logits = (np.round(rng.standard_normal((N, Q, M, self.L, K)) * logit_sigma * 256) / 256).astype(np.float32)
        self.grad = rng.standard_normal((N, Q, M, D)).astype(np.float32)

    def rows(self, pad=np.nan):
        return pack(self.loc, self.logits, pad=pad)

    def fwd(self, lib, value=None, loc=None, logits=None):
        rows = pack(self.loc if loc is None else loc, self.logits if logits is None else logits)
        return oracle.fdattn_forward(self.value if value is None else value, self.shapes, rows, self.K, lib=lib)

    def bwd(self, lib):
        return oracle.fdattn_backward(self.value, self.shapes, self.rows(), self.grad, self.K, lib=lib)


def torch_reference(value, shapes, loc, logits):
    """Multi-scale deformable attention from grid_sample + softmax (float64
    torch tensors; loc (N,Q,M,L,K,2) with u first, logits (N,Q,M,L,K))."""
    N, S, M, D = value.shape
    _, Q, _, L, K, _ = loc.shape
    a = torch.softmax(logits.reshape(N, Q, M, L * K), dim=-1).reshape(N, Q, M, L, K)
    out = torch.zeros(N, Q, M, D, dtype=value.dtype)
    s0 = 0
    for l, (H, W) in enumerate(shapes):
        vl = value[:, s0:s0 + H * W].reshape(N, H, W, M, D).permute(0, 3, 4, 1, 2).reshape(N * M, D, H, W)
        grid = (2.0 * loc[:, :, :, l] - 1.0).permute(0, 2, 1, 3, 4).reshape(N * M, Q, K, 2)
        smp = F.grid_sample(vl, grid, mode="bilinear", padding_mode="zeros", align_corners=False)
        smp = smp.reshape(N, M, D, Q, K).permute(0, 3, 1, 4, 2)     # N Q M K D
        out = out + (a[:, :, :, l, :, None] * smp).sum(3)
        s0 += H * W
    return out


def _close(got, ref, tol, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    bound = tol * (1.0 + np.abs(ref))
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e} (tol {tol})"


# -------------------------------------------------------------------- pins --

def pin_grid_sample_forward(lib):
    for seed, kw in ((0, {}), (1, dict(K=1, shapes=((3, 5),))), (2, dict(M=3, D=5, K=4))):
        c = Case(seed=seed, **kw)
        ref = torch_reference(torch.from_numpy(c.value).double(), c.shapes,
                              torch.from_numpy(c.loc).double(), torch.from_numpy(c.logits).double())
        _close(c.fwd(lib), ref.numpy(), 1e-6, f"forward vs grid_sample (seed {seed})")


def pin_grid_sample_backward(lib):
    for seed, kw in ((3, {}), (4, dict(M=1, D=4, K=2, shapes=((6, 4), (3, 2))))):
        c = Case(seed=seed, **kw)
        v = torch.from_numpy(c.value).double().requires_grad_(True)
        loc = torch.from_numpy(c.loc).double().requires_grad_(True)
        lg = torch.from_numpy(c.logits).double().requires_grad_(True)
        out = torch_reference(v, c.shapes, loc, lg)
        out.backward(torch.from_numpy(c.grad).double())
        gv, grow = c.bwd(lib)
        L, K = c.L, c.K
        _close(gv, v.grad.numpy(), 1e-6, "grad_value vs grid_sample autograd")
        N, Q, M = c.N, c.Q, c.M
        _close(grow[..., :2 * L * K], loc.grad.numpy().reshape(N, Q, M, 2 * L * K), 1e-5,
               "grad of locations vs grid_sample autograd")
        _close(grow[..., 2 * L * K:3 * L * K], lg.grad.numpy().reshape(N, Q, M, L * K), 1e-6,
               "grad of logits vs softmax autograd")
        assert np.all(grow[..., 3 * L * K:] == 0.0), "padding of grad_loc_attn must be 0"


def pin_boundary_samples(lib):
    """Samples exactly at -1, at size-1 and just inside/outside each border:
    values and derivatives against grid_sample (right derivative at
    integers, as grid_sample's backward takes the cell chosen by floor)."""
    H, W = 4, 8
    xs = np.array([-1.0, -1.0 + 2 ** -6, W - 1.0, W - 2 ** -6, W - 0.5, -1.5, 0.0, W, 2.0]) + 0.0
    ys = np.array([1.25, H - 1.0, -1.0, 0.5, H - 2 ** -6, 2.0, -1.0 + 2 ** -6, 1.0, H - 1.0])
    n = len(xs)
    loc = np.zeros((1, n, 1, 1, 1, 2), np.float32)
    loc[0, :, 0, 0, 0, 0] = (xs + 0.5) / W
    loc[0, :, 0, 0, 0, 1] = (ys + 0.5) / H
    logits = np.zeros((1, n, 1, 1, 1), np.float32)
    rng = np.random.default_rng(7)
    value = rng.standard_normal((1, H * W, 1, 3)).astype(np.float32)
    grad = rng.standard_normal((1, n, 1, 3)).astype(np.float32)
    rows = pack(loc, logits)
    out = oracle.fdattn_forward(value, [(H, W)], rows, 1, lib=lib)
    gv, grow = oracle.fdattn_backward(value, [(H, W)], rows, grad, 1, lib=lib)
    tv = torch.from_numpy(value).double().requires_grad_(True)
    tl = torch.from_numpy(loc).double().requires_grad_(True)
    ref = torch_reference(tv, [(H, W)], tl, torch.from_numpy(logits).double())
    ref.backward(torch.from_numpy(grad).double())
    _close(out, ref.detach().numpy(), 1e-6, "boundary forward")
    _close(gv, tv.grad.numpy(), 1e-6, "boundary grad_value")
    _close(grow[..., :2], tl.grad.numpy().reshape(1, n, 1, 2), 1e-6, "boundary location grads")


def pin_pixel_centres(lib):
    """Locations at pixel centres of power-of-two maps gather the pixel
    exactly; with one point per head the softmax weight is exactly 1, with
    equal logits it is 1/(L*K)."""
    rng = np.random.default_rng(11)
    shapes = [(4, 8), (2, 4)]
    S = 32 + 8
    value = rng.standard_normal((1, S, 2, 4)).astype(np.float32)
    Q, M = 6, 2
    r = rng.integers(0, 4, (1, Q, M, 1, 1))
    c = rng.integers(0, 8, (1, Q, M, 1, 1))
    loc = np.stack([(c + 0.5) / 8, (r + 0.5) / 4], -1).astype(np.float32)
    logits = rng.standard_normal((1, Q, M, 1, 1)).astype(np.float32)
    out = oracle.fdattn_forward(value[:, :32], [(4, 8)], pack(loc, logits), 1, lib=lib)
    for q in range(Q):
        for m in range(M):
            pix = r[0, q, m, 0, 0] * 8 + c[0, q, m, 0, 0]
            assert np.array_equal(out[0, q, m], value[0, pix, m].astype(np.float64)), "pixel-centre gather"
    # two levels, two points each, equal logits: the mean of the gathered pixels
    K = 2
    rr = rng.integers(0, 2, (1, Q, M, 2, K))
    cc = rng.integers(0, 4, (1, Q, M, 2, K))
    hw = np.array([[4, 8], [2, 4]])
    u = (cc + 0.5) / hw[None, None, None, :, None, 1]
    v = (rr + 0.5) / hw[None, None, None, :, None, 0]
    loc2 = np.stack([u, v], -1).astype(np.float32)
    out = oracle.fdattn_forward(value, shapes, pack(loc2, np.full((1, Q, M, 2, K), 0.75, np.float32)), K, lib=lib)
    for q in range(Q):
        for m in range(M):
            acc = 0.0
            for l in range(2):
                for k in range(K):
                    start = 0 if l == 0 else 32
                    pix = start + rr[0, q, m, l, k] * hw[l, 1] + cc[0, q, m, l, k]
                    acc = acc + value[0, pix, m].astype(np.float64) / (2 * K)
            assert np.allclose(out[0, q, m], acc, rtol=0, atol=1e-14), "equal-logit mean of pixels"


def pin_constant_and_affine_maps(lib):
    """Interior samples of affine maps f(x, y) = alpha*x + beta*y + gamma
    (per channel, x and y in the sampled level's pixel coordinates) with
    equal logits: out = mean_i f(x_i, y_i); d out / d u_i = W_l * alpha / (LK),
    d out / d v_i = H_l * beta / (LK); a constant map gives gamma."""
    rng = np.random.default_rng(12)
    shapes = [(8, 16), (4, 2)]      # powers of two: (x + 1/2) / W is exact in fp32
    L, K, M, D, Q = 2, 3, 2, 3, 7
    alpha = rng.integers(-4, 5, D).astype(np.float64)
    beta = rng.integers(-4, 5, D).astype(np.float64)
    gamma = rng.integers(-4, 5, D).astype(np.float64)
    S = 128 + 8
    value = np.zeros((1, S, M, D), np.float32)
    s0 = 0
    for H, W in shapes:
        r, c = np.divmod(np.arange(H * W), W)
        value[0, s0:s0 + H * W] = (alpha[None, None, :] * c[:, None, None] + beta[None, None, :] * r[:, None, None]
                                   + gamma[None, None, :]).astype(np.float32)
        s0 += H * W
    # interior coordinates x in [0, W-1), y in [0, H-1), multiples of 1/64
    hw = np.array(shapes, np.float64)
    x = np.floor(rng.uniform(0, 1, (1, Q, M, L, K)) * (hw[None, None, None, :, None, 1] - 1) * 64) / 64
    y = np.floor(rng.uniform(0, 1, (1, Q, M, L, K)) * (hw[None, None, None, :, None, 0] - 1) * 64) / 64
    loc = np.stack([(x + 0.5) / hw[None, None, None, :, None, 1], (y + 0.5) / hw[None, None, None, :, None, 0]],
                   -1).astype(np.float32)
    assert np.array_equal(loc[..., 0].astype(np.float64) * hw[None, None, None, :, None, 1] - 0.5, x)
    assert np.array_equal(loc[..., 1].astype(np.float64) * hw[None, None, None, :, None, 0] - 0.5, y)
    logits = np.full((1, Q, M, L, K), -1.5, np.float32)
    rows = pack(loc, logits)
    out = oracle.fdattn_forward(value, shapes, rows, K, lib=lib)
    expect = (alpha * x[..., None] + beta * y[..., None] + gamma).mean(axis=(3, 4))
    _close(out, expect, 1e-12, "affine maps")
    grad = rng.standard_normal((1, Q, M, D)).astype(np.float32)
    gv, grow = oracle.fdattn_backward(value, shapes, rows, grad, K, lib=lib)
    LK = L * K
    g_alpha = (grad.astype(np.float64) * alpha).sum(-1)
    g_beta = (grad.astype(np.float64) * beta).sum(-1)
    gu = g_alpha[..., None, None] * hw[None, None, None, :, None, 1] / LK
    gvv = g_beta[..., None, None] * hw[None, None, None, :, None, 0] / LK
    got = grow[..., :2 * LK].reshape(1, Q, M, L, K, 2)
    _close(got[..., 0], gu, 1e-12, "affine d/du")
    _close(got[..., 1], gvv, 1e-12, "affine d/dv")
    # constant maps: alpha = beta = 0
    value_c = np.broadcast_to(gamma.astype(np.float32), (1, S, M, D)).copy()
    logits_r = (np.round(rng.standard_normal((1, Q, M, L, K)) * 64) / 64).astype(np.float32)
    out = oracle.fdattn_forward(value_c, shapes, pack(loc, logits_r), K, lib=lib)
    _close(out, np.broadcast_to(gamma, out.shape), 1e-12, "constant maps")


def pin_logit_shift(lib):
    """A common shift of the logits of a (query, head) changes nothing; the
    logit gradients of a (query, head) sum to zero."""
    c = Case(seed=21, M=3, D=4, K=2)
    base = c.fwd(lib)
    shifted = c.fwd(lib, logits=(c.logits + np.float32(3.0)).astype(np.float32))
    _close(shifted, base, 1e-12, "logit shift")
    _, grow = c.bwd(lib)
    LK = c.L * c.K
    s = grow[..., 2 * LK:3 * LK].sum(-1)
    scale = np.abs(grow[..., 2 * LK:3 * LK]).sum(-1)
    assert np.all(np.abs(s) <= 1e-12 * (1 + scale)), "logit gradients must sum to zero"
    assert scale.max() > 1e-3, "degenerate logit gradients"


def pin_adjoint_grad_value(lib):
    """out is linear in the value: <grad_value, dv> = <g, out(dv)>."""
    c = Case(seed=31, M=2, D=3, K=3)
    gv, _ = c.bwd(lib)
    rng = np.random.default_rng(32)
    for _ in range(3):
        dv = rng.standard_normal(c.value.shape).astype(np.float32)
        lhs = float((gv * dv.astype(np.float64)).sum())
        rhs = float((c.grad.astype(np.float64) * c.fwd(lib, value=dv)).sum())
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(rhs)), f"adjoint {lhs} vs {rhs}"


def pin_finite_differences(lib):
    """Central differences: locations (exact inside a cell: the sample is
    linear along each axis there) and logits (O(h^2))."""
    c = Case(seed=41, N=1, Q=3, M=2, D=3, K=2, bits=8, lo=0.05, hi=0.95)
    _, grow = c.bwd(lib)
    L, K, LK = c.L, c.K, c.L * c.K
    g64 = c.grad.astype(np.float64)
    h = 2.0 ** -16
    rng = np.random.default_rng(42)
    checked = 0
    for _ in range(24):
        q, m, l, k, ax = (int(rng.integers(0, c.Q)), int(rng.integers(0, c.M)), int(rng.integers(0, L)),
                          int(rng.integers(0, K)), int(rng.integers(0, 2)))
        size = c.shapes[l][1 - ax]
        coord = float(c.loc[0, q, m, l, k, ax]) * size - 0.5
        if np.floor(coord - h * size) != np.floor(coord + h * size) or np.floor(coord) != np.floor(coord - h * size):
            continue
        lp = c.loc.copy()
        lm = c.loc.copy()
        lp[0, q, m, l, k, ax] += np.float32(h)
        lm[0, q, m, l, k, ax] -= np.float32(h)
        fd = ((c.fwd(lib, loc=lp)[0, q, m] - c.fwd(lib, loc=lm)[0, q, m]) * g64[0, q, m]).sum() / (2 * h)
        got = grow[0, q, m, 2 * (l * K + k) + ax]
        assert abs(fd - got) <= 1e-9 * (1 + abs(got)), f"location FD {fd} vs {got}"
        checked += 1
    assert checked >= 8
    hz = 2.0 ** -10
    for i in range(LK):
        l, k = divmod(i, K)
        zp = c.logits.copy()
        zm = c.logits.copy()
        zp[0, :, :, l, k] += np.float32(hz)
        zm[0, :, :, l, k] -= np.float32(hz)
        fd = ((c.fwd(lib, logits=zp) - c.fwd(lib, logits=zm)) * g64).sum(-1) / (2 * hz)
        got = grow[..., 2 * LK + i]
        assert np.all(np.abs(fd - got) <= 1e-5 * (1 + np.abs(got))), "logit FD"


PINS = [pin_grid_sample_forward, pin_grid_sample_backward, pin_boundary_samples, pin_pixel_centres,
        pin_constant_and_affine_maps, pin_logit_shift, pin_adjoint_grad_value, pin_finite_differences]

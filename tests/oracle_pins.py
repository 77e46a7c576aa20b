"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes a loaded oracle library (ctypes handle) and
raises AssertionError when the oracle disagrees with an independent fact:

* closed forms fixed by the definition of the operator ("Efficient Deformable
  ConvNets", DCNv3 recap equation with the softmax removed): identity and
  stride-2 subsampling with a one-hot centre mask, the grouped depthwise
  convolution that zero offsets reduce to (it is "as in regular
  convolution"), exact gathers at integer offsets, exact averages at
  half-integer offsets, the affine-image closed form;
* library routines: ``torch.nn.functional.conv2d`` (groups = C) and
  ``torch.nn.functional.grid_sample`` (bilinear, zeros, align_corners=True)
  with its autograd, all in float64;
* algebra: linearity in x and in m, adjoint identities for grad_value and
  grad_mask, finite differences for grad_offset (central inside a cell,
  forward one-sided at integers, including -1 and size-1);
* brute force: a vectorised zero-padded formulation written independently
  here, and the transposed dense Jacobian on tiny inputs.

The offset/mask channel layout (per group: K (dx, dy) pairs then K masks,
padding at the end of the pixel row) and the grid order (x index outer, y
index inner) are encoded here independently of the oracle's source.

The same functions are run against oracle builds with planted mistakes
(tests/test_oracle_mutants.py) to show that each mistake is caught.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle


# ----------------------------------------------------------------- helpers --

def grid_pairs(kh, kw, rc):
    return [(i, j) for i in range(kw) for j in range(kh)
            if not (rc and i == (kw - 1) // 2 and j == (kh - 1) // 2)]


def P_of(G, K):
    return (3 * G * K + 7) // 8 * 8


def out_hw(H, W, kh, kw, sh, sw, ph, pw, dh, dw):
    return ((H + 2 * ph - (dh * (kh - 1) + 1)) // sh + 1,
            (W + 2 * pw - (dw * (kw - 1) + 1)) // sw + 1)


def make_om(dx, dy, m, P=None, pad=np.nan):
    """Pack (N,Ho,Wo,G,K) dx, dy, m into the fused (N,Ho,Wo,P) tensor."""
    N, Ho, Wo, G, K = m.shape
    P = P or P_of(G, K)
    body = np.empty((N, Ho, Wo, G, 3 * K), np.float32)
    body[..., 0:2 * K:2] = dx
    body[..., 1:2 * K:2] = dy
    body[..., 2 * K:] = m
    om = np.full((N, Ho, Wo, P), pad, np.float32)
    om[..., :3 * G * K] = body.reshape(N, Ho, Wo, 3 * G * K)
    return om


def unpack_om(om, G, K):
    N, Ho, Wo, _ = om.shape
    body = om[..., :3 * G * K].reshape(N, Ho, Wo, G, 3 * K)
    return body[..., 0:2 * K:2], body[..., 1:2 * K:2], body[..., 2 * K:]


class Case:
    """A random problem with explicit geometry."""

    def __init__(self, seed=0, N=1, H=6, W=7, G=2, Cg=3, kh=3, kw=3, sh=1, sw=1,
                 ph=1, pw=1, dh=1, dw=1, rc=False, scale=1.0, off_sigma=1.5,
                 off_kind="normal", pad=np.nan):
        rng = np.random.default_rng(seed)
        self.__dict__.update(N=N, H=H, W=W, G=G, Cg=Cg, kh=kh, kw=kw, sh=sh, sw=sw,
                             ph=ph, pw=pw, dh=dh, dw=dw, rc=rc, scale=scale)
        self.pairs = grid_pairs(kh, kw, rc)
        self.K = len(self.pairs)
        self.Ho, self.Wo = out_hw(H, W, kh, kw, sh, sw, ph, pw, dh, dw)
        shp = (N, self.Ho, self.Wo, G, self.K)
        self.x = rng.standard_normal((N, H, W, G * Cg)).astype(np.float32)
        if off_kind == "normal":
            self.dx = (rng.standard_normal(shp) * off_sigma).astype(np.float32)
            self.dy = (rng.standard_normal(shp) * off_sigma).astype(np.float32)
        elif off_kind == "dyadic":  # multiples of 2^-12 kept >= 0.05 px from integers
            def dy_(s):
                v = rng.uniform(-off_sigma, off_sigma, s)
                fr = v - np.floor(v)
                fr = np.clip(fr, 0.05, 0.95)
                v = np.floor(v) + fr
                return (np.round(v * 4096) / 4096).astype(np.float32)
            self.dx, self.dy = dy_(shp), dy_(shp)
        elif off_kind == "integer":
            self.dx = rng.integers(-3, 4, shp).astype(np.float32)
            self.dy = rng.integers(-3, 4, shp).astype(np.float32)
        elif off_kind == "half":
            self.dx = (rng.integers(-4, 4, shp) + 0.5).astype(np.float32)
            self.dy = (rng.integers(-4, 4, shp) + 0.5).astype(np.float32)
        elif off_kind == "zero":
            self.dx = np.zeros(shp, np.float32)
            self.dy = np.zeros(shp, np.float32)
        else:
            raise ValueError(off_kind)
        self.m = (rng.standard_normal(shp)).astype(np.float32)
        self.g = rng.standard_normal((N, self.Ho, self.Wo, G * Cg)).astype(np.float32)
        self.pad = pad

    @property
    def om(self):
        return make_om(self.dx, self.dy, self.m, pad=self.pad)

    def kw_(self):
        return dict(kernel_h=self.kh, kernel_w=self.kw, stride_h=self.sh, stride_w=self.sw,
                    pad_h=self.ph, pad_w=self.pw, dilation_h=self.dh, dilation_w=self.dw,
                    group=self.G, group_channels=self.Cg, offset_scale=self.scale,
                    remove_center=self.rc)

    def fwd(self, lib, x=None, om=None):
        return oracle.forward(self.x if x is None else x, self.om if om is None else om,
                              lib=lib, **self.kw_())

    def bwd(self, lib, g=None):
        return oracle.backward(self.x, self.om, self.g if g is None else g, lib=lib, **self.kw_())

    def locs(self):
        """fp32 sampling coordinates (loc_h, loc_w), shape (N,Ho,Wo,G,K).

        The scales used by the pins are powers of two, so scale*d is exact in
        fp32 and one fp32 addition reproduces the single rounding of an fma.
        """
        ho = np.arange(self.Ho)[None, :, None, None, None]
        wo = np.arange(self.Wo)[None, None, :, None, None]
        ii = np.array([p[0] for p in self.pairs])[None, None, None, None, :]
        jj = np.array([p[1] for p in self.pairs])[None, None, None, None, :]
        bh = (ho * self.sh - self.ph + jj * self.dh).astype(np.float32)
        bw = (wo * self.sw - self.pw + ii * self.dw).astype(np.float32)
        s = np.float32(self.scale)
        return (bh + s * self.dy).astype(np.float32), (bw + s * self.dx).astype(np.float32)


def padded_bilinear_forward(case, x=None, m=None):
    """Independent zero-padded formulation (double weights, no bounds logic):
    the image is embedded in a zero frame wider than any sample reaches."""
    x = case.x if x is None else x
    m = case.m if m is None else m
    lh, lw = case.locs()
    lh = lh.astype(np.float64)
    lw = lw.astype(np.float64)
    M = int(np.nanmax(np.abs(np.concatenate([lh.ravel(), lw.ravel()])))) + 3
    N, H, W, C = x.shape
    xp = np.zeros((N, H + 2 * M, W + 2 * M, C))
    xp[:, M:M + H, M:M + W] = x
    ok = np.isfinite(lh) & np.isfinite(lw)
    lh = np.where(ok, lh, -M + 1.5)  # NaN samples land in the zero frame
    lw = np.where(ok, lw, -M + 1.5)
    h0 = np.floor(lh).astype(np.int64)
    w0 = np.floor(lw).astype(np.int64)
    fh = lh - h0
    fw = lw - w0
    y = np.zeros((N, case.Ho, case.Wo, C))
    n_ = np.arange(N)[:, None, None, None, None]
    for g in range(case.G):
        sl = slice(g * case.Cg, (g + 1) * case.Cg)
        a, b = h0[..., g, :] + M, w0[..., g, :] + M
        nn = np.broadcast_to(n_[..., 0, :], a.shape)
        v00 = xp[nn, a, b][..., sl]
        v01 = xp[nn, a, b + 1][..., sl]
        v10 = xp[nn, a + 1, b][..., sl]
        v11 = xp[nn, a + 1, b + 1][..., sl]
        th, tw = fh[..., g, :, None], fw[..., g, :, None]
        s = ((1 - th) * (1 - tw) * v00 + (1 - th) * tw * v01
             + th * (1 - tw) * v10 + th * tw * v11)
        y[..., sl] = np.sum(m[..., g, :, None].astype(np.float64) * s, axis=-2)
    return y


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b)
    bad = err > atol + rtol * np.abs(b)
    assert not bad.any(), f"{what}: max err {err.max():.3e} at {np.argwhere(bad)[0]}"


# -------------------------------------------------------------------- pins --

def pin_identity(lib):
    """Zero offsets, m one-hot at the grid centre, stride 1, pad = dil*(k-1)/2:
    the output is the input, bit for bit."""
    for kh, kw, dh, dw in [(3, 3, 1, 1), (5, 5, 1, 1), (3, 3, 2, 2), (3, 5, 1, 2)]:
        c = Case(seed=kh * 10 + dw, N=2, H=7, W=6, kh=kh, kw=kw, dh=dh, dw=dw,
                 ph=dh * (kh - 1) // 2, pw=dw * (kw - 1) // 2, off_kind="zero")
        kc = c.pairs.index(((kw - 1) // 2, (kh - 1) // 2))
        c.m[:] = 0
        c.m[..., kc] = 1
        y = c.fwd(lib)
        assert np.array_equal(y, c.x.astype(np.float64)), (kh, kw, dh, dw)


def pin_stride2(lib):
    """Same one-hot centre mask with stride 2: y = x[::2, ::2]."""
    c = Case(seed=3, N=1, H=9, W=8, sh=2, sw=2, off_kind="zero")
    kc = c.pairs.index((1, 1))
    c.m[:] = 0
    c.m[..., kc] = 1
    y = c.fwd(lib)
    assert np.array_equal(y, c.x[:, ::2, ::2].astype(np.float64))


def pin_depthwise_conv(lib):
    """Zero offsets and spatially constant m_gk: a grouped depthwise
    convolution (zero padding) with weight[c][ky][kx] = m_{g(c), k(kx,ky)},
    compared with torch conv2d (groups = C) in float64."""
    cases = [
        dict(kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, rc=False),
        dict(kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, rc=True),
        dict(kh=3, kw=5, sh=1, sw=2, ph=1, pw=2, dh=1, dw=1, rc=False),
        dict(kh=5, kw=5, sh=2, sw=1, ph=4, pw=2, dh=2, dw=1, rc=True),
        dict(kh=3, kw=3, sh=1, sw=1, ph=0, pw=2, dh=2, dw=2, rc=False),
    ]
    for t, cfg in enumerate(cases):
        c = Case(seed=100 + t, N=2, H=9, W=8, G=2, Cg=3, off_kind="zero", **cfg)
        mg = np.random.default_rng(t).standard_normal((c.G, c.K)).astype(np.float32)
        c.m[:] = mg[None, None, None]
        y = c.fwd(lib)
        C = c.G * c.Cg
        wt = np.zeros((C, 1, c.kh, c.kw))
        for ch in range(C):
            for k, (i, j) in enumerate(c.pairs):
                wt[ch, 0, j, i] = mg[ch // c.Cg, k]
        ref = F.conv2d(torch.from_numpy(c.x.astype(np.float64)).permute(0, 3, 1, 2),
                       torch.from_numpy(wt), stride=(c.sh, c.sw), padding=(c.ph, c.pw),
                       dilation=(c.dh, c.dw), groups=C).permute(0, 2, 3, 1).numpy()
        _close(y, ref, 1e-12, 1e-12, f"depthwise {cfg}")


def pin_integer_gather(lib):
    """Integer offsets: every sample is one pixel of the zero-extended image."""
    c = Case(seed=7, N=2, H=6, W=5, G=2, Cg=4, off_kind="integer")
    y = c.fwd(lib)
    M = 8
    xp = np.zeros((c.N, c.H + 2 * M, c.W + 2 * M, c.G * c.Cg))
    xp[:, M:M + c.H, M:M + c.W] = c.x
    ref = np.zeros_like(y)
    for n in range(c.N):
        for ho in range(c.Ho):
            for wo in range(c.Wo):
                for g in range(c.G):
                    for k, (i, j) in enumerate(c.pairs):
                        r = ho - c.ph + j + int(c.dy[n, ho, wo, g, k]) + M
                        q = wo - c.pw + i + int(c.dx[n, ho, wo, g, k]) + M
                        sl = slice(g * c.Cg, (g + 1) * c.Cg)
                        ref[n, ho, wo, sl] += float(c.m[n, ho, wo, g, k]) * xp[n, r, q, sl]
    _close(y, ref, 1e-12, 1e-12, "integer gather")


def pin_half_integer(lib):
    """Half-integer offsets: weights are exactly 1/4 (or 1/2 on an integer
    axis), so samples are exact means of neighbours (zero outside)."""
    c = Case(seed=8, N=1, H=6, W=6, G=2, Cg=4, off_kind="half")
    c.dy[..., ::2] = np.round(c.dy[..., ::2] - 0.5)  # mix integer and half rows
    y = c.fwd(lib)
    ref = padded_bilinear_forward(c)
    _close(y, ref, 1e-13, 1e-13, "half-integer")


def pin_padded_bruteforce(lib):
    """Arbitrary offsets (many out of bounds, NaNs, huge values) against the
    independent zero-padded formulation."""
    for t, kw_ in enumerate([dict(), dict(rc=True), dict(kh=5, kw=3, ph=2, pw=1, dh=1, dw=2),
                             dict(sh=2, sw=2, scale=0.5), dict(H=1, W=4)]):
        c = Case(seed=20 + t, N=2, G=2, Cg=3, off_sigma=2.5, **kw_)
        c.dx.flat[::17] = np.nan
        c.dy.flat[::23] = 1e30
        c.dx.flat[::29] = -1e30
        y = c.fwd(lib)
        c2 = Case(seed=20 + t, N=2, G=2, Cg=3, off_sigma=2.5, **kw_)
        c2.dx, c2.dy = c.dx.copy(), c.dy.copy()
        far = ~np.isfinite(c2.dx) | ~np.isfinite(c2.dy) | (np.abs(c2.dx) > 1e6) | (np.abs(c2.dy) > 1e6)
        c2.dx[far] = np.nan
        c2.dy[far] = np.nan
        ref = padded_bilinear_forward(c2)
        _close(y, ref, 1e-6, 1e-6, f"padded brute force {kw_}")


def pin_affine_image(lib):
    """x[h][w][c] = a_c*h + b_c*w + d_c: a bilinear sample of an affine image
    inside [0,H-1]x[0,W-1] is exact, so y = sum_k m (a*loc_h + b*loc_w + d);
    and inside a cell d y / d loc_w = m*b, d y / d loc_h = m*a."""
    c = Case(seed=9, N=1, H=9, W=10, G=2, Cg=3, off_kind="dyadic", off_sigma=1.0, scale=0.5)
    rng = np.random.default_rng(90)
    # dyadic coefficients: every pixel value is exact in fp32
    a = rng.integers(64, 128, c.G * c.Cg) / 64.0
    b = -rng.integers(192, 256, c.G * c.Cg) / 64.0
    d = rng.integers(-64, 64, c.G * c.Cg) / 64.0
    hh = np.arange(c.H)[:, None, None]
    ww = np.arange(c.W)[None, :, None]
    c.x = (a * hh + b * ww + d)[None].astype(np.float32)
    assert np.array_equal(c.x[0].astype(np.float64), a * hh + b * ww + d)
    # keep only samples strictly inside the image
    lh, lw = c.locs()
    inside = (lh > 0) & (lh < c.H - 1) & (lw > 0) & (lw < c.W - 1)
    c.m = np.where(inside, c.m, 0).astype(np.float32)
    y = c.fwd(lib)
    lh64, lw64 = lh.astype(np.float64), lw.astype(np.float64)
    ref = np.zeros_like(y)
    for g in range(c.G):
        sl = slice(g * c.Cg, (g + 1) * c.Cg)
        val = a[sl] * lh64[..., g, :, None] + b[sl] * lw64[..., g, :, None] + d[sl]
        ref[..., sl] = np.sum(c.m[..., g, :, None] * val, axis=-2)
    _close(y, ref, 2e-6, 2e-5, "affine forward")
    gv, gom = c.bwd(lib)
    gdx, gdy, gm = unpack_om(gom, c.G, c.K)
    for g in range(c.G):
        sl = slice(g * c.Cg, (g + 1) * c.Cg)
        gs = c.g[..., sl].astype(np.float64)
        mm = c.m[..., g, :].astype(np.float64)
        ex_dx = c.scale * mm * (gs @ b[sl])[..., None]
        ex_dy = c.scale * mm * (gs @ a[sl])[..., None]
        val = (a[sl] * lh64[..., g, :, None] + b[sl] * lw64[..., g, :, None] + d[sl])
        ex_m = np.sum(gs[..., None, :] * val, axis=-1)
        ins = inside[..., g, :]
        _close(gdx[..., g, :], ex_dx, 2e-5, 2e-5, "affine grad dx")
        _close(gdy[..., g, :], ex_dy, 2e-5, 2e-5, "affine grad dy")
        _close(gm[..., g, :][ins], ex_m[ins], 2e-5, 2e-5, "affine grad m")


def _grid_sample_terms(c, x, dx, dy, m):
    """sum_k m * grid_sample(x_g, loc_k) per group, differentiable (float64)."""
    N, H, W, C = x.shape
    ho = torch.arange(c.Ho, dtype=torch.float64)[None, :, None, None, None]
    wo = torch.arange(c.Wo, dtype=torch.float64)[None, None, :, None, None]
    ii = torch.tensor([p[0] for p in c.pairs], dtype=torch.float64)
    jj = torch.tensor([p[1] for p in c.pairs], dtype=torch.float64)
    loc_h = ho * c.sh - c.ph + jj * c.dh + c.scale * dy
    loc_w = wo * c.sw - c.pw + ii * c.dw + c.scale * dx
    gx = 2 * loc_w / (W - 1) - 1
    gy = 2 * loc_h / (H - 1) - 1
    outs = []
    for g in range(c.G):
        xg = x[..., g * c.Cg:(g + 1) * c.Cg].permute(0, 3, 1, 2)
        grid = torch.stack([gx[..., g, :], gy[..., g, :]], -1).reshape(N, c.Ho, c.Wo * c.K, 2)
        s = F.grid_sample(xg, grid, mode="bilinear", padding_mode="zeros", align_corners=True)
        s = s.reshape(N, c.Cg, c.Ho, c.Wo, c.K).permute(0, 2, 3, 4, 1)
        outs.append(torch.sum(m[..., g, :, None] * s, dim=-2))
    return torch.cat(outs, -1)


def pin_grid_sample(lib):
    """Forward and all gradients against torch grid_sample (bilinear, zeros,
    align_corners=True) and its autograd, float64, at coordinates away from
    integers (where the bilinear sample is differentiable)."""
    for t, kw_ in enumerate([dict(), dict(rc=True, G=3, Cg=2),
                             dict(sh=2, sw=1, dh=2, ph=2, scale=0.5)]):
        c = Case(seed=40 + t, N=2, H=6, W=7, off_kind="dyadic", off_sigma=3.0, **kw_)
        y = c.fwd(lib)
        x = torch.from_numpy(c.x.astype(np.float64)).requires_grad_()
        dx = torch.from_numpy(c.dx.astype(np.float64)).requires_grad_()
        dy = torch.from_numpy(c.dy.astype(np.float64)).requires_grad_()
        m = torch.from_numpy(c.m.astype(np.float64)).requires_grad_()
        ref = _grid_sample_terms(c, x, dx, dy, m)
        _close(y, ref.detach().numpy(), 1e-6, 1e-6, f"grid_sample fwd {kw_}")
        (ref * torch.from_numpy(c.g.astype(np.float64))).sum().backward()
        gv, gom = c.bwd(lib)
        gdx, gdy, gm = unpack_om(gom, c.G, c.K)
        _close(gv, x.grad.numpy(), 1e-6, 1e-6, "grid_sample grad_value")
        _close(gdx, dx.grad.numpy(), 1e-5, 1e-5, "grid_sample grad dx")
        _close(gdy, dy.grad.numpy(), 1e-5, 1e-5, "grid_sample grad dy")
        _close(gm, m.grad.numpy(), 1e-6, 1e-6, "grid_sample grad m")


def pin_linearity(lib):
    """f(a*x1 + b*x2, m) = a f(x1, m) + b f(x2, m); likewise in m."""
    c = Case(seed=11, N=1, H=6, W=6, G=2, Cg=4)
    rng = np.random.default_rng(110)
    x2 = rng.standard_normal(c.x.shape).astype(np.float32)
    a, b = np.float32(0.75), np.float32(-1.25)
    y1, y2 = c.fwd(lib), c.fwd(lib, x=x2)
    y12 = c.fwd(lib, x=(a * c.x + b * x2).astype(np.float32))
    _close(y12, a * y1 + b * y2, 1e-6, 1e-6, "linear in x")
    m2 = rng.standard_normal(c.m.shape).astype(np.float32)
    om1, om2 = c.om, make_om(c.dx, c.dy, m2)
    om12 = make_om(c.dx, c.dy, (a * c.m + b * m2).astype(np.float32))
    _close(c.fwd(lib, om=om12), a * c.fwd(lib, om=om1) + b * c.fwd(lib, om=om2),
           1e-6, 1e-6, "linear in m")


def pin_adjoint(lib):
    """<f(x), g> = <x, grad_value(g)> and <f(m), g> = <m, grad_m(g)>, with
    offsets mixing integers (-1 and size-1 included) and fractions."""
    for t, kw_ in enumerate([dict(), dict(rc=True, sh=2, sw=2), dict(kh=5, kw=3, ph=2, dh=1, dw=2, pw=2)]):
        c = Case(seed=12 + t, N=2, H=6, W=5, G=2, Cg=4, **kw_)
        c.dx[..., ::3] = np.round(c.dx[..., ::3])
        c.dy[..., ::2] = np.round(c.dy[..., ::2])
        y = c.fwd(lib)
        gv, gom = c.bwd(lib)
        lhs = float(np.sum(y * c.g))
        _close(np.sum(c.x.astype(np.float64) * gv), lhs, 1e-10, 1e-10, "adjoint value")
        _, _, gm = unpack_om(gom, c.G, c.K)
        _close(np.sum(c.m.astype(np.float64) * gm), lhs, 1e-10, 1e-10, "adjoint mask")
        assert np.all(gom[..., 3 * c.G * c.K:] == 0), "padding gradient must be 0"


def _objective(c, lib, dx, dy):
    om = make_om(dx, dy, c.m)
    return float(np.sum(oracle.forward(c.x, om, lib=lib, **c.kw_()) * c.g))


def pin_finite_differences(lib):
    """grad_offset against finite differences of <f, g>.  Offsets are dyadic
    (multiples of 2^-12) and the step is 2^-10, so coordinates, steps and
    fp32 weights are exact and the difference quotient is exact inside a
    cell.  Central differences >= 0.05 px from integers; forward one-sided
    differences at integers (the right derivative), including -1 and
    size-1."""
    c = Case(seed=13, N=1, H=5, W=6, G=2, Cg=3, off_kind="dyadic", off_sigma=2.5, scale=1.0)
    rng = np.random.default_rng(130)
    # samples placed exactly on integer coordinates: -1 and size-1 on each
    # axis, and interior integers (target loc_w, loc_h; None keeps the offset)
    specials = [((0, 0, 0), 0, 0, -1, 2), ((0, 0, 1), 1, 4, 3, -1),
                ((0, 2, 3), 0, 5, c.W - 1, None), ((0, 1, 2), 1, 7, None, c.H - 1),
                ((0, 3, 3), 0, 2, 2, 3), ((0, 4, 5), 1, 1, 0, 0)]
    for (n, ho, wo), g, k, tw, th in specials:
        i, j = c.pairs[k]
        if tw is not None:
            c.dx[n, ho, wo, g, k] = tw - (wo * c.sw - c.pw + i * c.dw)
        if th is not None:
            c.dy[n, ho, wo, g, k] = th - (ho * c.sh - c.ph + j * c.dh)
    gv, gom = c.bwd(lib)
    gdx, gdy, _ = unpack_om(gom, c.G, c.K)
    h = np.float32(2.0 ** -10)
    idx = [tuple(int(v) for v in i) for i in np.argwhere(np.ones(c.dx.shape, bool))]
    picks = [idx[i] for i in rng.choice(len(idx), 40, replace=False)]
    picks += [(n, ho, wo, g, k) for (n, ho, wo), g, k, _, _ in specials]
    for p in picks:
        for comp, grad in (("x", gdx), ("y", gdy)):
            base = c.dx if comp == "x" else c.dy
            v = base[p]
            integer = float(v) == np.floor(v)
            plus = base.copy()
            plus[p] = v + h
            if integer:
                f0 = _objective(c, lib, c.dx, c.dy)
                f1 = _objective(c, lib, plus if comp == "x" else c.dx, plus if comp == "y" else c.dy)
                fd = (f1 - f0) / float(h)
            else:
                minus = base.copy()
                minus[p] = v - h
                fp_ = _objective(c, lib, plus if comp == "x" else c.dx, plus if comp == "y" else c.dy)
                fm_ = _objective(c, lib, minus if comp == "x" else c.dx, minus if comp == "y" else c.dy)
                fd = (fp_ - fm_) / (2 * float(h))
            _close(grad[p], fd, 1e-9, 1e-9, f"FD d{comp} at {p} (integer={integer})")
    # the right derivatives at -1 are not zero (zero-extended image)
    assert abs(gdx[0, 0, 0, 0, 0]) > 1e-6 and abs(gdy[0, 0, 1, 1, 4]) > 1e-6


def pin_dense_jacobian(lib):
    """Tiny inputs: grad_value = J_x^T g and grad_m = J_m^T g with the
    Jacobians built column by column from the zero-padded formulation."""
    c = Case(seed=14, N=1, H=4, W=3, G=2, Cg=2, off_sigma=1.5)
    gv, gom = c.bwd(lib)
    _, _, gm = unpack_om(gom, c.G, c.K)
    ex = np.zeros(c.x.size)
    base = np.zeros(c.x.shape, np.float32)
    for q in range(c.x.size):
        e = base.copy()
        e.flat[q] = 1
        ex[q] = np.sum(padded_bilinear_forward(c, x=e) * c.g)
    _close(gv.ravel(), ex, 1e-6, 1e-6, "dense J_x^T g")
    em = np.zeros(c.m.size)
    zm = np.zeros(c.m.shape, np.float32)
    for q in range(c.m.size):
        e = zm.copy()
        e.flat[q] = 1
        em[q] = np.sum(padded_bilinear_forward(c, m=e) * c.g)
    _close(gm.ravel(), em, 1e-6, 1e-6, "dense J_m^T g")


def pin_padding_and_nan(lib):
    """Padding channels are never read (NaN padding gives the same bits as
    zero padding); a NaN offset contributes nothing; far offsets give 0."""
    c = Case(seed=15, N=1, H=5, W=5, G=3, Cg=2)  # 3*3*9 = 81 -> P = 88
    y_nan = oracle.forward(c.x, make_om(c.dx, c.dy, c.m, pad=np.nan), lib=lib, **c.kw_())
    y_zero = oracle.forward(c.x, make_om(c.dx, c.dy, c.m, pad=0.0), lib=lib, **c.kw_())
    assert np.array_equal(y_nan, y_zero) and np.isfinite(y_nan).all()
    P = P_of(c.G, c.K) + 8
    y_wide = oracle.forward(c.x, make_om(c.dx, c.dy, c.m, P=P, pad=np.nan), lib=lib, **c.kw_())
    assert np.array_equal(y_wide, y_zero)
    dx = c.dx.copy()
    dx[..., 0] = np.nan
    m0 = c.m.copy()
    m0[..., 0] = 0
    assert np.array_equal(oracle.forward(c.x, make_om(dx, c.dy, c.m), lib=lib, **c.kw_()),
                          oracle.forward(c.x, make_om(c.dx, c.dy, m0), lib=lib, **c.kw_()))
    far = np.full_like(c.dx, 50.0)
    assert np.all(oracle.forward(c.x, make_om(far, c.dy, c.m), lib=lib, **c.kw_()) == 0)
    gv, gom = oracle.backward(c.x, make_om(dx, c.dy, c.m), c.g, lib=lib, **c.kw_())
    gdx, gdy, gm = unpack_om(gom, c.G, c.K)
    assert np.all(gdx[..., 0] == 0) and np.all(gdy[..., 0] == 0) and np.all(gm[..., 0] == 0)


def pin_remove_center(lib):
    """remove_center with K = 8 equals the full 3x3 grid with a zero centre
    mask (the remaining points keep their order)."""
    c8 = Case(seed=16, N=1, H=6, W=6, G=2, Cg=3, rc=True)
    c9 = Case(seed=16, N=1, H=6, W=6, G=2, Cg=3, rc=False)
    kc = c9.pairs.index((1, 1))
    keep = [k for k in range(9) if k != kc]
    for arr9, arr8 in ((c9.dx, c8.dx), (c9.dy, c8.dy), (c9.m, c8.m)):
        arr9[..., keep] = arr8
    c9.m[..., kc] = 0
    c9.x = c8.x
    _close(c8.fwd(lib), c9.fwd(lib), 1e-12, 1e-12, "remove_center forward")


# ---- DCNv3 softmax mode ------------------------------------------------------


def _dyadic(a, bits=10):
    return (np.round(a * 2.0 ** bits) / 2.0 ** bits).astype(np.float32)


def pin_softmax_plain_reduction(lib):
    """softmax mode = the plain operator with masks replaced by
    scipy.special.softmax over the K points (a library routine), forward and
    backward; its mask gradient is the softmax Jacobian applied to the plain
    mask gradient."""
    from scipy.special import softmax as sp_softmax

    c = Case(seed=21, N=2, H=6, W=7, G=2, Cg=3, off_sigma=2.0)
    p = sp_softmax(c.m.astype(np.float64), axis=-1)
    om_l = c.om
    om_p = make_om(c.dx, c.dy, p.astype(np.float32))
    kw = c.kw_()
    _close(oracle.forward(c.x, om_l, softmax=True, lib=lib, **kw),
           oracle.forward(c.x, om_p, lib=lib, **kw), 1e-6, 1e-6, "softmax forward")
    gv_s, gom_s = oracle.backward(c.x, om_l, c.g, softmax=True, lib=lib, **kw)
    gv_p, gom_p = oracle.backward(c.x, om_p, c.g, lib=lib, **kw)
    _close(gv_s, gv_p, 1e-6, 1e-6, "softmax grad_value")
    dx_s, dy_s, gl = unpack_om(gom_s, c.G, c.K)
    dx_p, dy_p, gp = unpack_om(gom_p, c.G, c.K)
    _close(dx_s, dx_p, 1e-6, 1e-6, "softmax grad dx")
    _close(dy_s, dy_p, 1e-6, 1e-6, "softmax grad dy")
    # chain rule through the softmax, written with the Jacobian matrix
    jac = np.einsum("...k,kj->...kj", p, np.eye(c.K)) - np.einsum("...k,...j->...kj", p, p)
    _close(gl, np.einsum("...kj,...k->...j", jac, gp), 1e-6, 1e-6, "softmax Jacobian")


def pin_softmax_invariants(lib):
    """Shifting all K logits of a (pixel, group) by one constant changes
    nothing; the logit gradients sum to 0 over K; a dominant centre logit
    with zero offsets reproduces the input (identity)."""
    c = Case(seed=22, N=1, H=5, W=6, G=2, Cg=3, off_sigma=1.5)
    c.m = _dyadic(c.m)
    kw = c.kw_()
    shift = np.random.default_rng(220).integers(-3, 4, c.m.shape[:-1] + (1,)).astype(np.float32)
    om_shift = make_om(c.dx, c.dy, (c.m + shift).astype(np.float32))
    y0 = oracle.forward(c.x, c.om, softmax=True, lib=lib, **kw)
    y1 = oracle.forward(c.x, om_shift, softmax=True, lib=lib, **kw)
    _close(y1, y0, 1e-12, 1e-12, "softmax shift invariance")
    gv, gom = oracle.backward(c.x, c.om, c.g, softmax=True, lib=lib, **kw)
    _, _, gl = unpack_om(gom, c.G, c.K)
    assert np.abs(gl.sum(axis=-1)).max() < 1e-12, "logit gradients must sum to 0"
    ci = Case(seed=23, N=1, H=5, W=6, G=2, Cg=3, off_kind="zero")
    kc = ci.pairs.index((1, 1))
    ci.m[:] = 0
    ci.m[..., kc] = 100.0
    _close(oracle.forward(ci.x, ci.om, softmax=True, lib=lib, **ci.kw_()), ci.x, 1e-12, 1e-12,
           "dominant centre logit = identity")


def pin_softmax_finite_differences(lib):
    """Logit gradients against central differences of <f, g> (the softmax is
    smooth; dyadic logits and a 2^-12 step are exact in fp32)."""
    c = Case(seed=24, N=1, H=4, W=5, G=2, Cg=2, off_sigma=1.5)
    c.m = _dyadic(c.m)
    kw = c.kw_()
    _, gom = oracle.backward(c.x, c.om, c.g, softmax=True, lib=lib, **kw)
    _, _, gl = unpack_om(gom, c.G, c.K)
    h = np.float32(2.0 ** -12)
    rng = np.random.default_rng(240)
    idx = [tuple(int(v) for v in i) for i in np.argwhere(np.ones(c.m.shape, bool))]
    for p in [idx[i] for i in rng.choice(len(idx), 30, replace=False)]:
        mp, mm = c.m.copy(), c.m.copy()
        mp[p] += h
        mm[p] -= h
        fp_ = float(np.sum(oracle.forward(c.x, make_om(c.dx, c.dy, mp), softmax=True, lib=lib, **kw) * c.g))
        fm_ = float(np.sum(oracle.forward(c.x, make_om(c.dx, c.dy, mm), softmax=True, lib=lib, **kw) * c.g))
        _close(gl[p], (fp_ - fm_) / (2 * float(h)), 1e-6, 1e-6, f"FD logit at {p}")


PINS = [pin_identity, pin_stride2, pin_depthwise_conv, pin_integer_gather, pin_half_integer,
        pin_padded_bruteforce, pin_affine_image, pin_grid_sample, pin_linearity, pin_adjoint,
        pin_finite_differences, pin_dense_jacobian, pin_padding_and_nan, pin_remove_center,
        pin_softmax_plain_reduction, pin_softmax_invariants, pin_softmax_finite_differences]

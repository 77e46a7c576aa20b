"""Flash deformable attention: HIP path against the CPU oracle, element by
element, through the C ABI.

Tolerances (elementwise; ref = oracle in double on the same rounded inputs):
  fp32   output, grad_value, logit gradients: |gpu - ref| <= 1e-5 + 1e-5 |ref|
         location gradients: |gpu - ref| <= 1e-5 (max(1, a W_l) + |ref|) for u
         (H_l for v): the kernel sums grad_out_d * d sample_d / dx over the D
         channels in fp32 and only then multiplies by a * W_l, so its rounding
         error carries that factor.
  16-bit |gpu - ref| <= 2e-2 + ulp_dtype(|ref|) for the output and
         grad_loc_attn (rounded to the storage dtype; the location gradients
         with the same a * size factor); grad_value is fp32 for every dtype and
         is held to the fp32 bound.
"""
import numpy as np
import pytest
import torch

import oracle
from dynamic_sparse_vision_amd import flash_deform_attn as fda
from dynamic_sparse_vision_amd import synth
from dynamic_sparse_vision_amd.workloads import FDA_WORKLOADS, FdaWorkload

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def ulp(ref, dtype):
    a = np.abs(ref)
    if dtype == "fp16":
        return np.spacing(a.astype(np.float16)).astype(np.float64)
    if dtype == "bf16":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
        return 2.0 ** (e - 7)
    return np.zeros_like(a)


def check(gpu, ref, dtype, what, scale=None):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    s = np.ones_like(ref) if scale is None else np.maximum(1.0, scale)
    if dtype == "fp32":
        bound = 1e-5 * (s + np.abs(ref))
    else:
        bound = 2e-2 * s + ulp(ref, dtype)
    bad = err > bound
    say(f"  {what}: max|err| {err.max():.3e}  n>bound {int(bad.sum())} of {err.size}")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance, first at {np.argwhere(bad)[0]}"


def location_scale(la_ref, shapes, K):
    """a_i * W_l (u entries) and a_i * H_l (v entries) per row, for the
    location-gradient tolerance."""
    L = len(shapes)
    LK = L * K
    z = la_ref[..., 2 * LK:3 * LK].astype(np.float64)
    a = np.exp(z - z.max(-1, keepdims=True))
    a /= a.sum(-1, keepdims=True)
    size = np.array([[w, h] for h, w in shapes for _ in range(K)], np.float64)   # (LK, 2)
    return (a[..., :, None] * size).reshape(*la_ref.shape[:-1], 2 * LK)


def to_dev(arrs, dtype):
    out = []
    for a in arrs:
        st, ref = synth.to_storage(a, dtype)
        out.append((st.cuda(), ref))
    return out


def run_case(w: FdaWorkload, N=None, backward=True, la_override=None, sorted_grad_value=True):
    v32, la32, g32 = w.make_inputs(N=N)
    if la_override is not None:
        la32 = la_override(la32)
    (v, vr), (la, lar), (g, gr) = to_dev((v32, la32, g32), w.dtype)
    out = fda.forward(v, w.shapes, la, w.K)
    torch.cuda.synchronize()
    ref = oracle.fdattn_forward(vr, w.shapes, lar, w.K)
    check(out.float().cpu().numpy(), ref, w.dtype, f"{w.name} output")
    if not backward:
        return
    gv, gla = fda.backward(v, w.shapes, la, g, w.K, sorted_grad_value=sorted_grad_value)
    torch.cuda.synchronize()
    rgv, rgla = oracle.fdattn_backward(vr, w.shapes, lar, gr, w.K)
    LK = w.L * w.K
    # grad_value is fp32 for every dtype, summed from the same rounded inputs
    check(gv.cpu().numpy(), rgv, "fp32", f"{w.name} grad_value")
    gla = gla.float().cpu().numpy()
    check(gla[..., :2 * LK], rgla[..., :2 * LK], w.dtype, f"{w.name} grad locations",
          scale=location_scale(lar, w.shapes, w.K))
    check(gla[..., 2 * LK:3 * LK], rgla[..., 2 * LK:3 * LK], w.dtype, f"{w.name} grad logits")
    assert np.all(gla[..., 3 * LK:] == 0.0), "padding of grad_loc_attn must be 0"


def _w(name, dtype="fp32", N=2, shapes=((8, 10), (4, 5), (2, 3)), M=2, D=32, K=4, Q=37, **kw):
    return FdaWorkload(name, N, tuple(shapes), M, D, K, dtype, seed=90 + len(name), Q=Q, **kw)


CASES = [
    # several blocks with a ragged tail, random reference points, three levels
    _w("d32_fp32"),
    # other head widths: one lane (D = 8), two, eight; the forward also at 128
    _w("d8_fp32", D=8, M=3, Q=53),
    _w("d16_fp32", D=16, M=5, Q=29),
    _w("d64_fp32", D=64, M=1, Q=61, K=3),
    # wide spread: many samples leave their level's map
    _w("spread_fp32", sigma_px=12.0, shapes=((6, 7), (3, 9)), K=5),
    # one level, one point: the softmax weight is exactly 1
    _w("l1k1_fp32", shapes=((11, 13),), K=1, Q=40),
    # the largest point count: 16 levels x 8 points
    _w("l16k8_fp32", shapes=tuple((2 + l % 3, 3 + l % 4) for l in range(16)), K=8, M=2, Q=9),
    # the same with one lane per query (D = 8): 256 queries per block, whose
    # attention weights and lane sums take 128 KB of LDS
    _w("l16k8_d8_fp32", shapes=tuple((2 + l % 3, 3 + l % 4) for l in range(16)), K=8, M=1, D=8, Q=300),
    # encoder queries over four levels
    FDA_WORKLOADS["fda_small_fp32"],
    # 16-bit storage
    _w("d32_fp16", dtype="fp16"),
    _w("d16_bf16", dtype="bf16", D=16, M=3),
    _w("d64_bf16", dtype="bf16", D=64, M=2, K=2),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_parity(w):
    say(f"[fdattn] {w.name} N={w.N} levels={w.shapes} Q={w.queries} M={w.M} D={w.D} K={w.K} {w.dtype}")
    run_case(w)


# Encoder-ordered queries (Q = S, query q is pixel q of the concatenated
# levels) with 32-channel heads, the benchmark's layout at small sizes: odd
# level sizes, one-pixel levels, several images and heads, a wide spread
# (many samples off their level's map), and 16-bit storage.
ENCODER_CASES = [
    _w("enc_odd_fp32", N=2, M=3, Q=0, shapes=((13, 19), (7, 10), (4, 5), (1, 1))),
    _w("enc_spread_fp32", N=1, M=2, Q=0, shapes=((24, 40), (12, 20), (6, 10)), sigma_px=14.0),
    _w("enc_fp16", dtype="fp16", N=2, M=2, Q=0, shapes=((16, 24), (8, 12), (4, 6), (2, 3))),
    _w("enc_bf16", dtype="bf16", N=1, M=4, Q=0, shapes=((9, 17), (5, 9), (3, 5))),
]


@pytest.mark.parametrize("w", ENCODER_CASES, ids=[c.name for c in ENCODER_CASES])
def test_parity_encoder_windows(w):
    say(f"[fdattn] {w.name} N={w.N} levels={w.shapes} encoder queries M={w.M} D={w.D} K={w.K} {w.dtype}")
    run_case(w)


ATOMIC_CASES = [c for c in CASES if c.name in ("d32_fp32", "spread_fp32", "l16k8_fp32", "l16k8_d8_fp32", "d16_bf16")]


@pytest.mark.parametrize("w", ATOMIC_CASES, ids=[c.name for c in ATOMIC_CASES])
def test_parity_atomic_grad_value(w):
    """The backward without a workspace (grad_value by device atomics)."""
    say(f"[fdattn] {w.name} atomic grad_value path")
    run_case(w, sorted_grad_value=False)


EDGE_CASES = [
    # one query, one image, degenerate maps: 1x1, a single row and a single column
    _w("tiny_maps_fp32", N=1, Q=1, M=1, D=8, K=3, shapes=((1, 1), (1, 7), (5, 1))),
    _w("tiny_maps_many_q_fp32", N=1, Q=19, M=3, D=16, K=2, shapes=((1, 1), (2, 1), (1, 2))),
    # a level whose corner bins (201 x 201) do not fit the per-slice sort in
    # LDS: the backward takes the device-atomic path even with a workspace
    _w("big_level_fp32", N=1, Q=50, M=1, D=8, K=2, shapes=((200, 200),), sigma_px=3.0),
    # odd sizes everywhere
    _w("odd_sizes_bf16", dtype="bf16", N=3, Q=23, M=3, D=16, K=5, shapes=((9, 13), (5, 7), (3, 3))),
]


@pytest.mark.parametrize("w", EDGE_CASES, ids=[c.name for c in EDGE_CASES])
def test_parity_edge_cases(w):
    say(f"[fdattn] {w.name} N={w.N} levels={w.shapes} Q={w.queries} M={w.M} D={w.D} K={w.K} {w.dtype}")
    if w.name == "big_level_fp32":
        v = torch.zeros((w.N, w.S, w.M, w.D), device="cuda")
        la = torch.zeros((w.N, w.queries, w.M, w.P), device="cuda")
        assert fda.flash_deform_attn_backward_workspace(v, w.shapes, la, num_points=w.K) == 0, \
            "a slice of 40401 bins should not fit the LDS sort"
    run_case(w)


def test_forward_head_dim_128():
    w = _w("d128_fp32", D=128, M=2, Q=21)
    say(f"[fdattn] {w.name} forward only (the backward takes D <= 64)")
    run_case(w, backward=False)


def test_boundary_and_non_finite_locations():
    """Locations exactly on the borders (-1, size-1), outside every map and
    NaN: the GPU follows the oracle (NaN samples are skipped but keep their
    softmax share)."""
    w = _w("borders_fp32", shapes=((8, 16), (4, 8)), K=3, Q=24, M=2, D=32)
    rng = np.random.default_rng(5)

    def override(la):
        la = la.copy()
        L, K = w.L, w.K
        pairs = la[..., :2 * L * K].reshape(*la.shape[:-1], L, K, 2)
        for l, (H, W) in enumerate(w.shapes):
            xs = np.array([-1.0, W - 1.0, -1.5, W + 0.0, 0.0, W - 0.5])
            ys = np.array([H - 1.0, -1.0, 0.25, 1.0, H + 3.0, -1.0])
            sel = rng.integers(0, len(xs), pairs.shape[:-3] + (K,))
            pairs[..., l, :, 0] = np.where(rng.random(sel.shape) < 0.5, (xs[sel] + 0.5) / W, pairs[..., l, :, 0])
            pairs[..., l, :, 1] = np.where(rng.random(sel.shape) < 0.5, (ys[sel] + 0.5) / H, pairs[..., l, :, 1])
        pairs[0, 3, 1, 0, 1, 0] = np.nan
        pairs[1, 5, 0, 1, 2, 1] = np.nan
        la[..., :2 * L * K] = pairs.reshape(*la.shape[:-1], 2 * L * K)
        return la

    say(f"[fdattn] {w.name}: border, out-of-map and NaN locations")
    run_case(w, la_override=override)
    rng = np.random.default_rng(5)
    say(f"[fdattn] {w.name}: the same, atomic grad_value path")
    run_case(w, la_override=override, sorted_grad_value=False)


def test_empty_query_set_zeroes_grad_value():
    w = _w("q0_fp32")
    v32, _, _ = w.make_inputs()
    v = torch.from_numpy(v32).cuda()
    la = torch.empty((w.N, 0, w.M, w.P), device="cuda")
    g = torch.empty((w.N, 0, w.M, w.D), device="cuda")
    gv = torch.full(v.shape, 7.0, device="cuda")
    gla = torch.empty_like(la)
    fda.flash_deform_attn_backward(v, w.shapes, la, g, gv, gla, num_points=w.K)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gv).item() == 0


@pytest.mark.parametrize("name", ["fda_enc_800x1280_b4_fp32", "fda_enc_800x1280_b4_fp16"])
def test_benchmark_workload_elementwise(name):
    """The benchmark workload at its full size and in the launch
    configuration the benchmark times (four images, four levels of an
    800x1280 input, 21260 encoder queries, 8 heads of 32 channels): output,
    every grad_value element, and every location and logit gradient against
    the oracle, in fp32 and fp16 storage."""
    w = FDA_WORKLOADS[name]
    say(f"[fdattn] {w.name}, all {w.N} images, every element")
    run_case(w)


def test_benchmark_workload_sampled():
    """The benchmark call at full size (N=4, four levels of an 800x1280
    input, encoder queries): the forward and the location / logit gradients
    are compared on sampled queries (the oracle computes those rows alone);
    grad_value is checked through the adjoint identity
    <grad_value, dv> = <grad_out, forward(dv)> with the GPU forward, which
    holds at any size."""
    w = FDA_WORKLOADS["fda_enc_800x1280_b4_fp32"]
    say(f"[fdattn] {w.name} full size, sampled rows")
    v32, la32, g32 = w.make_inputs()
    v, la, g = (torch.from_numpy(a).cuda() for a in (v32, la32, g32))
    out = fda.forward(v, w.shapes, la, w.K)
    gv, gla = fda.backward(v, w.shapes, la, g, w.K)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    qs = np.sort(rng.choice(w.queries, 300, replace=False))
    ref = oracle.fdattn_forward(v32, w.shapes, la32[:, qs], w.K)
    check(out.cpu().numpy()[:, qs], ref, "fp32", "sampled output")
    _, rgla = oracle.fdattn_backward(v32, w.shapes, la32[:, qs], g32[:, qs], w.K)
    LK = w.L * w.K
    glq = gla.cpu().numpy()[:, qs]
    check(glq[..., :2 * LK], rgla[..., :2 * LK], "fp32", "sampled grad locations",
          scale=location_scale(la32[:, qs], w.shapes, w.K))
    check(glq[..., 2 * LK:3 * LK], rgla[..., 2 * LK:3 * LK], "fp32", "sampled grad logits")
    del out
    for seed in (1, 2):
        dv = torch.from_numpy(np.random.default_rng(seed).standard_normal(v32.shape).astype(np.float32)).cuda()
        fdv = fda.forward(dv, w.shapes, la, w.K)
        torch.cuda.synchronize()
        lhs = float((gv.double() * dv.double()).sum())
        rhs = float((g.double() * fdv.double()).sum())
        scale = float((gv.double().abs() * dv.double().abs()).sum())
        say(f"  adjoint: {lhs:.6e} vs {rhs:.6e} (scale {scale:.3e})")
        assert abs(lhs - rhs) <= 1e-5 * scale

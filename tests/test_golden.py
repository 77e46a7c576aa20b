"""Stored values from the pages (cited in each fixture) and hand-worked
examples, checked against the oracle and the byte accounting (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from dynamic_sparse_vision_amd.workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


HAND = _load("hand_examples.json")


@pytest.mark.parametrize("ex", HAND["examples"], ids=lambda e: e["name"])
def test_hand_example(ex, oracle_lib):
    img = np.array(HAND["image"], np.float32)[None, :, :, None]   # (1,3,3,1)
    rc = ex["remove_center"]
    K = 8 if rc else 9
    P = (3 * K + 7) // 8 * 8
    om = np.zeros((1, 3, 3, P), np.float32)
    om[..., 3 * K:] = np.nan                                       # padding is never read
    ho, wo = ex["pixel"]
    for pt in ex["points"]:
        k = pt["k"]
        om[0, ho, wo, 2 * k] = pt["dx"]
        om[0, ho, wo, 2 * k + 1] = pt["dy"]
        om[0, ho, wo, 2 * K + k] = pt["m"]
    kw = dict(group=1, group_channels=1, remove_center=rc, lib=oracle_lib)
    y = oracle.forward(img, om, **kw)
    expect = np.zeros_like(y)
    expect[0, ho, wo, 0] = ex["y"]
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-12)
    g = np.zeros((1, 3, 3, 1), np.float32)
    g[0, ho, wo, 0] = 1.0
    _, gom = oracle.backward(img, np.nan_to_num(om, nan=0.0), g, **kw)
    gr = ex["grad"]
    k = gr["k"]
    got = (gom[0, ho, wo, 2 * k], gom[0, ho, wo, 2 * k + 1], gom[0, ho, wo, 2 * K + k])
    np.testing.assert_allclose(got, (gr["dx"], gr["dy"], gr["m"]), rtol=0, atol=1e-12)


def test_ideal_mac_matches_byte_accounting():
    """The compulsory bytes the benchmark divides by are the pages' ideal MAC
    (2HWC + 27HWG elements for a 3x3 grid) plus the pad-to-8 channels."""
    mac = _load("ideal_mac.json")
    a, b = mac["mac_coeff_hwc"], mac["mac_coeff_hwg"]
    # the pages' rounded figures follow from the coefficients at C' = 16
    assert round(a + b / 16, 1) == mac["mac_over_hwc_at_group_dim_16"]
    assert round(mac["nocache_over_hwc"] / (a + b / 16)) == mac["nocache_over_ideal"]
    for w in WORKLOADS.values():
        if w.K != 9 or w.direction != "fwd":
            continue
        assert (w.Ho, w.Wo) == (w.H, w.W)
        hw = w.N * w.H * w.W
        ideal = a * hw * w.C + b * hw * w.G
        padding = hw * (w.P - 27 * w.G)
        assert w.fwd_bytes() == w.elem_bytes * (ideal + padding), w.name
        # sampled points = 9 per output element; 4 FLOP-ish per bilinear sample
        assert 4 * w.points == mac["flops_over_hwc"] * hw * w.C

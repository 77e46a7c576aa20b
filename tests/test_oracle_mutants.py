"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle/dcnv4_oracle.c with one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, another boundary
reading), compiled with gcc into a temporary library.  The pins of
tests/oracle_pins.py are run against it; the mutant is caught when any pin
fails.  All mutants keep the oracle's memory bounds checks intact.  CPU only.
"""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dcnv4_oracle.c")

MUTANTS = {
    "dx_dy_swapped": [("float dx = omg[2 * k];", "float dx = omg[2 * k + 1];"),
                      ("float dy = omg[2 * k + 1];", "float dy = omg[2 * k];")],
    "mask_interleaved_layout": [("(double)omg[2 * K + k];", "(double)omg[3 * k + 2];")],
    "grid_transposed": [("gi[K] = i;\n            gj[K] = j;", "gi[K] = j;\n            gj[K] = i;")],
    "offset_scale_dropped": [("fmaf(offset_scale, dx,", "fmaf(1.0f, dx,"),
                             ("fmaf(offset_scale, dy,", "fmaf(1.0f, dy,")],
    "offset_sign": [("fmaf(offset_scale, dx,", "fmaf(-offset_scale, dx,")],
    "pad_sign": [("wo * stride_w - pad_w", "wo * stride_w + pad_w")],
    "dilation_dropped": [("gi[k] * dil_w", "gi[k]")],
    "stride_dropped": [("ho * stride_h - pad_h", "ho - pad_h")],
    "trunc_not_floor": [("floorf(loc_h)", "truncf(loc_h)"), ("floorf(loc_w)", "truncf(loc_w)")],
    "skip_at_minus_one": [("loc_h >= -1.0f", "loc_h > -1.0f"), ("loc_w >= -1.0f", "loc_w > -1.0f")],
    "upper_bound_off_by_one": [("loc_w < (float)W", "loc_w < (float)(W - 1)")],
    "weights_w01_w10_swapped": [("f.wt[1] = f.hh * f.lw;", "f.wt[1] = f.lh * f.hw;"),
                                ("f.wt[2] = f.lh * f.hw;", "f.wt[2] = f.hh * f.lw;")],
    "corner_swapped_in_forward": [("(double)f.wt[1] * xval(value, n, f.h0, f.w0 + 1, ch, H, W, C)",
                                   "(double)f.wt[1] * xval(value, n, f.h0 + 1, f.w0, ch, H, W, C)")],
    "output_channels_interleaved": [("y[g * Cg + c] = acc[c];", "y[c * G + g] = acc[c];")],
    "mask_not_applied": [("acc[c] += m * s;", "acc[c] += s;")],
    "grad_w_sign": [("(double)f.hh * (v[1] - v[0])", "(double)f.hh * (v[0] - v[1])")],
    "grad_h_wrong_weight": [("(double)f.hw * (v[2] - v[0])", "(double)f.hh * (v[2] - v[0])")],
    "grad_offset_missing_m": [("(double)offset_scale * m * gw", "(double)offset_scale * gw")],
    "grad_offset_missing_scale": [("(double)offset_scale * m * gh", "m * gh")],
    "grad_value_missing_m": [("+= m * (double)f.wt[q] * go;", "+= (double)f.wt[q] * go;")],
    "grad_mask_corner_only": [("gm += go * s;", "gm += go * v[0];")],
    "grad_dx_dy_slots_swapped": [("gomg[2 * k] = (double)offset_scale * m * gw;",
                                  "gomg[2 * k] = (double)offset_scale * m * gh;"),
                                 ("gomg[2 * k + 1] = (double)offset_scale * m * gh;",
                                  "gomg[2 * k + 1] = (double)offset_scale * m * gw;")],
    "grad_value_wrong_corner": [("int cc[4] = {f.w0, f.w0 + 1, f.w0, f.w0 + 1};",
                                 "int cc[4] = {f.w0, f.w0, f.w0 + 1, f.w0 + 1};")],
    # DCNv3 softmax mode
    "softmax_not_normalised": [("p[k] /= sum;", "p[k] /= 1.0;")],
    "softmax_jacobian_missing_sum": [("gomg[2 * K + k] = pk[k] * (gomg[2 * K + k] - s);",
                                      "gomg[2 * K + k] = pk[k] * gomg[2 * K + k];")],
    "softmax_jacobian_missing_p": [("gomg[2 * K + k] = pk[k] * (gomg[2 * K + k] - s);",
                                    "gomg[2 * K + k] = gomg[2 * K + k] - s;")],
    "softmax_backward_slice_off_by_one": [("                        softmax_masks(omg + 2 * K, K, pk);",
                                           "                        softmax_masks(omg + 2 * K - 1, K, pk);")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) >= 1, f"mutation site not found: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / f"mutant_{name}.c"
    path.write_text(src)
    lib_path = str(tmp_path / f"libmutant_{name}.so")
    oracle.build(src=str(path), out=lib_path)
    lib = oracle.load(lib_path)
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

"""Planted mistakes in the flash deformable attention oracle must each fail
at least one pin of tests/fdattn_pins.py.

Each mutant is a copy of oracle/fdattn_oracle.c with one plausible mistake
(a swapped coordinate, a dropped term, a wrong index or sign, another
boundary reading), compiled with gcc into a temporary library.  All mutants
keep the oracle's memory bounds checks intact.  CPU only.
"""
import os

import pytest

import oracle
from tests import fdattn_pins

SRC = oracle.FDA_SRC

MUTANTS = {
    "uv_swapped": [("fmaf(row[2 * i], (float)W, -0.5f)", "fmaf(row[2 * i + 1], (float)W, -0.5f)"),
                   ("fmaf(row[2 * i + 1], (float)H, -0.5f)", "fmaf(row[2 * i], (float)H, -0.5f)")],
    "coord_plus_half": [("fmaf(row[2 * i], (float)W, -0.5f)", "fmaf(row[2 * i], (float)W, 0.5f)")],
    "coord_no_half_shift": [("fmaf(row[2 * i + 1], (float)H, -0.5f)", "fmaf(row[2 * i + 1], (float)H, 0.0f)")],
    "coord_sizes_swapped": [("fmaf(row[2 * i], (float)W, -0.5f)", "fmaf(row[2 * i], (float)H, -0.5f)"),
                            ("fmaf(row[2 * i + 1], (float)H, -0.5f)", "fmaf(row[2 * i + 1], (float)W, -0.5f)")],
    "point_index_level_minor": [("int i = l * K + k;", "int i = k * L + l;")],
    "logits_slot_off_by_one": [("fdao_softmax(row + 2 * LK, LK, a);", "fdao_softmax(row + 2 * LK - 1, LK, a);")],
    "softmax_not_normalised": [("a[i] /= sum;", "a[i] /= 1.0;")],
    "softmax_max_not_subtracted_sign": [("a[i] = exp((double)z[i] - mx);", "a[i] = exp(mx - (double)z[i]);")],
    "level_start_ignored": [("long s = start + (long)r * W + c;", "long s = (long)r * W + c;")],
    "level_row_stride_height": [("long s = start + (long)r * W + c;", "long s = start + (long)r * H + c;")],
    "weights_w01_w10_swapped": [("f.wt[1] = f.hy * f.lx;", "f.wt[1] = f.ly * f.hx;"),
                                ("f.wt[2] = f.ly * f.hx;", "f.wt[2] = f.hy * f.lx;")],
    "skip_at_minus_one": [("y >= -1.0f && y < (float)H && x >= -1.0f", "y > -1.0f && y < (float)H && x > -1.0f")],
    "upper_bound_off_by_one": [("x < (float)W))", "x < (float)(W - 1)))")],
    "trunc_not_floor": [("floorf(y)", "truncf(y)"), ("floorf(x)", "truncf(x)")],
    "attention_not_applied": [("y[d] += a[i] * s;", "y[d] += s;")],
    "grad_u_missing_size": [("grow[2 * i] = a[i] * (double)W * gx;", "grow[2 * i] = a[i] * gx;")],
    "grad_v_uses_width": [("grow[2 * i + 1] = a[i] * (double)H * gy;", "grow[2 * i + 1] = a[i] * (double)W * gy;")],
    "grad_u_sign": [("(double)f.hy * (v[1] - v[0])", "(double)f.hy * (v[0] - v[1])")],
    "grad_v_wrong_weight": [("(double)f.hx * (v[2] - v[0])", "(double)f.hy * (v[2] - v[0])")],
    "grad_uv_slots_swapped": [("grow[2 * i] = a[i] * (double)W * gx;", "grow[2 * i + 1] = a[i] * (double)W * gx;"),
                              ("grow[2 * i + 1] = a[i] * (double)H * gy;", "grow[2 * i] = a[i] * (double)H * gy;")],
    "grad_value_missing_attention": [("+= a[i] * (double)f.wt[c] * go;", "+= (double)f.wt[c] * go;")],
    "grad_value_wrong_corner": [("int cc[4] = {f.c0, f.c0 + 1, f.c0, f.c0 + 1};",
                                 "int cc[4] = {f.c0, f.c0, f.c0 + 1, f.c0 + 1};")],
    "grad_attention_corner_only": [("gs += go * s;", "gs += go * v[0];")],
    "softmax_jacobian_missing_sum": [("grow[2 * LK + i] = a[i] * (ga[i] - dot);", "grow[2 * LK + i] = a[i] * ga[i];")],
    "softmax_jacobian_missing_a": [("grow[2 * LK + i] = a[i] * (ga[i] - dot);", "grow[2 * LK + i] = ga[i] - dot;")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) >= 1, f"mutation site not found: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / f"fdattn_mutant_{name}.c"
    path.write_text(src)
    lib_path = str(tmp_path / f"libfdattn_mutant_{name}.so")
    oracle.build(src=str(path), out=lib_path)
    lib = oracle.load_fdattn(lib_path)
    failed = []
    for pin in fdattn_pins.PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"

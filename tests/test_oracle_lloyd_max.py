"""Pins of the oracle's Lloyd-Max N(0, 1) tables.

PolyKV explainer, section 2.B: rotated V coordinates are mapped to
precomputed Lloyd-Max centroids for N(0, 1).  The pages print no values, so
the table is pinned by (i) the fixed-point conditions themselves in double,
(ii) the published table of J. Max (1960) to its printed precision,
(iii) the 1-bit closed form +-sqrt(2/pi), (iv) the MSE against numerical
integration, and (v) the frozen fp32 table written by tests/golden/make_golden.py.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm as normal

from oracle import lloyd_max

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_fixed_point_conditions_hold_in_double(bits):
    c, t = lloyd_max.lloyd_max_normal(bits)
    assert c.shape == (2 ** bits,) and t.shape == (2 ** bits - 1,)
    assert lloyd_max.fixed_point_residual(c, t) < 1e-13
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    assert np.all((t > c[:-1]) & (t < c[1:]))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_symmetry_and_zero_middle_threshold(bits):
    c, t = lloyd_max.table_f32(bits)
    assert np.array_equal(c, -c[::-1])
    assert np.array_equal(t, -t[::-1])
    assert t[len(t) // 2] == 0.0


def test_one_bit_closed_form():
    c, t = lloyd_max.lloyd_max_normal(1)
    assert abs(c[1] - math.sqrt(2.0 / math.pi)) < 1e-15 and c[0] == -c[1] and t[0] == 0.0


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_matches_max_1960_table(bits):
    ref = json.load(open(os.path.join(GOLD, "max1960.json")))
    lv = ref["levels"][str(2 ** bits)]
    c, t = lloyd_max.lloyd_max_normal(bits)
    half = 2 ** (bits - 1)
    assert np.allclose(c[half:], lv["outputs"], atol=ref["tolerance"], rtol=0)
    assert np.allclose(t[half - 1:], lv["thresholds"], atol=ref["tolerance"], rtol=0)
    mse = lloyd_max.mse_closed_form(c, t)
    assert abs(mse - lv["mse"]) / lv["mse"] < 2e-3


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_mse_closed_form_matches_integration(bits):
    c, t = lloyd_max.lloyd_max_normal(bits)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    tot = 0.0
    for j in range(len(c)):
        val, _ = integrate.quad(lambda x, cj=c[j]: (x - cj) ** 2 * normal.pdf(x), edges[j], edges[j + 1],
                                epsabs=1e-14, epsrel=1e-12)
        tot += val
    assert abs(tot - lloyd_max.mse_closed_form(c, t)) < 1e-10


@pytest.mark.parametrize("bits", [2, 3])
def test_local_optimality(bits):
    # moving any centroid (with thresholds re-centred) raises the distortion
    c, t = lloyd_max.lloyd_max_normal(bits)
    d0 = lloyd_max.mse_closed_form(c, t)
    for j in range(len(c)):
        for eps in (-1e-3, 1e-3):
            c2 = c.copy()
            c2[j] += eps
            t2 = 0.5 * (c2[:-1] + c2[1:])
            assert lloyd_max.mse_closed_form(c2, t2) > d0


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fp32_table_is_frozen_and_unambiguous(bits):
    gold = json.load(open(os.path.join(GOLD, "lloyd_max_fp32.json")))["tables"][str(bits)]
    c32, t32 = lloyd_max.table_f32(bits)
    assert [format(int(x), "08x") for x in c32.view(np.uint32)] == gold["centroids_hex"]
    assert [format(int(x), "08x") for x in t32.view(np.uint32)] == gold["thresholds_hex"]
    # every double value is far from an fp32 rounding midpoint, so any correct
    # double solver rounds to the same fp32 table
    c, t = lloyd_max.lloyd_max_normal(bits)
    for x in np.concatenate([c, t]):
        if x == 0.0:
            continue
        f = np.float32(x)
        ulp = float(np.spacing(np.float32(abs(f))))
        frac = abs(x - float(f)) / ulp
        assert frac < 0.5 - 1e-3

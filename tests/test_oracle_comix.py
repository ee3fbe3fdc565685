"""Pins of the oracle's CoMixKV controller (sensitivity and bit allocation).

CoMixKV news article (abstract, method): sensitivity from recent Q/K/V as a
local attention-error bound; 2 to 4 bits allocated jointly over agents and
layers under one byte budget.  The article prints no formula or example, so the
oracle is pinned by closed forms and special cases of its own definition
(single-token window, uniform attention, a dominant score, permutation and
scale behaviour), by the bound actually holding for the oracle codec's
errors, by the published Lloyd-Max distortions (Max 1960), and by brute force
over every allocation on small instances where the greedy rule is provably
optimal (equal byte cost per added bit and convex error factors).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import codec, comixkv

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_distortion_matches_max_1960():
    gold = json.load(open(os.path.join(GOLD, "max1960.json")))
    for bits, levels in ((2, "4"), (3, "8"), (4, "16")):
        want = gold["levels"][levels]["mse"]
        assert abs(comixkv.distortion(bits) - want) <= 5e-4 * want + 1e-6


def test_error_factors_decrease_and_are_convex():
    e = comixkv.error_factors()
    assert e[0] > e[1] > e[2] > 0
    assert e[0] - e[1] > e[1] - e[2]  # the greedy rule is exact for unit costs only if so


def _window(rng, A, L, Hkv, cap, d):
    k = rng.standard_normal((A, L, Hkv, cap, d))
    v = rng.standard_normal((A, L, Hkv, cap, d)) * rng.lognormal(0.0, 0.5, (A, L, Hkv, 1, d))
    return k, v


def test_single_token_window_gives_its_norm():
    rng = np.random.default_rng(1)
    k, v = _window(rng, 2, 3, 2, 4, 64)
    q = rng.standard_normal((2, 2, 3, 4, 64))
    s = comixkv.sensitivity(q, k, v, [1, 1], 2)
    want = np.linalg.norm(v[:, :, :, 0], axis=-1).mean(axis=-1)  # mean over kv heads (equal row counts)
    np.testing.assert_allclose(s, want, rtol=1e-12)


def test_zero_queries_give_mean_norm_and_empty_window_gives_zero():
    rng = np.random.default_rng(2)
    k, v = _window(rng, 2, 2, 2, 16, 64)
    q = np.zeros((3, 2, 2, 4, 64))
    s = comixkv.sensitivity(q, k, v, [16, 0], 2)
    want = np.linalg.norm(v[0, :, :, :16], axis=-1).mean(axis=(-1, -2))
    np.testing.assert_allclose(s[0], want, rtol=1e-12)
    assert np.all(s[1] == 0.0)


def test_dominant_score_selects_that_token():
    rng = np.random.default_rng(3)
    d, n = 64, 12
    k, v = _window(rng, 1, 1, 1, n, d)
    q = np.zeros((1, 1, 1, 1, d))
    q[..., 0] = 1.0
    k[0, 0, 0, :, 0] = 0.0
    k[0, 0, 0, 5, 0] = 4000.0  # score 500 above every other token
    s = comixkv.sensitivity(q, k, v, [n], 1)
    assert abs(s[0, 0] - np.linalg.norm(v[0, 0, 0, 5])) < 1e-9


def test_permutation_and_scale():
    rng = np.random.default_rng(4)
    k, v = _window(rng, 1, 2, 2, 20, 128)
    q = rng.standard_normal((2, 1, 2, 8, 128))
    s = comixkv.sensitivity(q, k, v, [20], 2)
    perm = rng.permutation(20)
    s_p = comixkv.sensitivity(q, k[:, :, :, perm], v[:, :, :, perm], [20], 2)
    np.testing.assert_allclose(s_p, s, rtol=1e-12)
    np.testing.assert_allclose(comixkv.sensitivity(q, k, 3.0 * v, [20], 2), 3.0 * s, rtol=1e-12)
    # only the first win_len tokens count
    v2 = v.copy()
    v2[:, :, :, 15:] *= 100.0
    np.testing.assert_allclose(comixkv.sensitivity(q, k, v2, [15], 2), comixkv.sensitivity(q, k, v, [15], 2),
                               rtol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_bound_holds_for_the_codec(bits):
    """Mean attention-output error of V quantised by the codec <= sqrt(D_b) * s (the stated bound)."""
    rng = np.random.default_rng(10 + bits)
    d, n, R, Hq = 128, 48, 4, 4
    errs, bounds = [], []
    for trial in range(6):
        k, v = _window(rng, 1, 1, 1, n, d)
        q = rng.standard_normal((R, 1, 1, Hq, d))
        s = comixkv.sensitivity(q, k, v, [n], 1)[0, 0]
        nrm, codes = codec.v_encode(v[0, 0, 0].astype(np.float32), bits)
        vhat = codec.v_decode(nrm, codes, bits)
        vq = v[0, 0, 0].astype(np.float32).astype(np.float64)
        e = 0.0
        for r in range(R):
            for h in range(Hq):
                sc = (k[0, 0, 0] @ q[r, 0, 0, h]) / math.sqrt(d)
                p = np.exp(sc - sc.max())
                p /= p.sum()
                e += np.linalg.norm(p @ (vq - vhat))
        errs.append(e / (R * Hq))
        bounds.append(math.sqrt(comixkv.distortion(bits)) * s)
    assert np.mean(errs) <= np.mean(bounds)
    # and the bound is not vacuous: the triangle inequality over ~n tokens loses at most ~sqrt(n)
    assert np.mean(errs) >= np.mean(bounds) / (2.0 * math.sqrt(n))


def _brute(sens, cost, err, budget):
    best, arg = math.inf, None
    for bits in itertools.product((2, 3, 4), repeat=len(sens)):
        c = sum(int(cost[i][b - 2]) for i, b in enumerate(bits))
        if c <= budget:
            o = comixkv.objective(sens, err, bits)
            if o < best:
                best, arg = o, bits
    return best, arg


@pytest.mark.parametrize("seed", range(8))
def test_greedy_is_optimal_with_equal_step_costs(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 7))
    sens = rng.lognormal(0.0, 1.0, n).astype(np.float32)
    unit = int(rng.integers(100, 1000))
    base = int(rng.integers(1000, 5000))
    cost = np.array([[base + 2 * unit, base + 3 * unit, base + 4 * unit]] * n, dtype=np.uint64)
    err = comixkv.error_factors()
    for extra in range(0, 2 * n + 1):
        budget = int(cost[:, 0].sum()) + extra * unit + int(rng.integers(0, unit))
        bits = comixkv.allocate(sens, cost, err, budget)
        assert int(cost[np.arange(n), bits - 2].sum()) <= budget
        best, _ = _brute(sens, cost, err, budget)
        assert comixkv.objective(sens, err, bits) == pytest.approx(best, rel=1e-12, abs=0)


@pytest.mark.parametrize("seed", range(6))
def test_greedy_with_real_costs_is_feasible_and_near_optimal(seed):
    rng = np.random.default_rng(200 + seed)
    n = 5
    sens = rng.lognormal(0.0, 1.0, n).astype(np.float32)
    cost = np.stack([comixkv.block_cost(int(t), 8, 128) for t in rng.integers(16, 512, n)])
    err = comixkv.error_factors()
    lo, hi = int(cost[:, 0].sum()), int(cost[:, 2].sum())
    for budget in np.linspace(lo, hi, 7).astype(np.int64):
        bits = comixkv.allocate(sens, cost, err, int(budget))
        assert int(cost[np.arange(n), bits - 2].sum()) <= budget
        best, _ = _brute(sens, cost, err, int(budget))
        assert comixkv.objective(sens, err, bits) >= best - 1e-12
        assert comixkv.objective(sens, err, bits) <= 1.25 * best  # stated rule, not global optimum


def test_budget_edges_and_ties():
    err = comixkv.error_factors()
    cost = np.array([[200, 300, 400]] * 4, dtype=np.uint64)
    assert comixkv.allocate([1, 1, 1, 1], cost, err, 799) is None
    assert list(comixkv.allocate([1, 1, 1, 1], cost, err, 800)) == [2, 2, 2, 2]
    assert list(comixkv.allocate([1, 1, 1, 1], cost, err, 1600)) == [4, 4, 4, 4]
    # equal sensitivities: widths differ by at most one, lower indices first
    assert list(comixkv.allocate([1, 1, 1, 1], cost, err, 1000)) == [3, 3, 2, 2]
    assert list(comixkv.allocate([1, 1, 1, 1], cost, err, 1300)) == [4, 3, 3, 3]
    # a much more sensitive item gets the bits first
    assert list(comixkv.allocate([1, 50, 1, 1], cost, err, 1000)) == [2, 4, 2, 2]


def test_block_cost_matches_pool_layout_bytes_per_token():
    # 180 B per (token, kv head) at d 128 and 3 bits, plus 4 B of K scale per token
    assert list(comixkv.block_cost(1, 1, 128)) == [128 + 32 + 4 + 4, 128 + 48 + 4 + 4, 128 + 64 + 4 + 4]
    assert comixkv.block_cost(4096, 8, 128)[1] == 4096 * (8 * 180 + 4)

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


# ---------------------------------------------------------------- refresh cycle
def _widths(w):
    return {a: [int(x) for x in b] for a, b in w.items()}


def test_refresh_cycle_hand_worked():
    """A start -> refresh -> commit -> exit -> refresh sequence worked by hand.

    Two layers, one kv head, d = 64: a token of one layer takes 64 + 64 b / 8 + 4 + 4 bytes,
    88 / 96 / 104 at 2 / 3 / 4 bits.  Two agents of 16 tokens capacity each, budget 5988.
    Error decreases per unit of sensitivity: e2 - e3 = 0.15689, e3 - e4 = 0.08840.
    """
    rc = comixkv.RefreshCycle(5988, 2, 1, 64)
    rc.start(0, 16)
    rc.start(1, 16)
    sens = {0: [4.0, 1.0], 1: [2.0, 3.0]}
    # 16 remaining tokens per item: 1408 / 1536 / 1664, upgrades of 128.  2 bits everywhere:
    # 5632 of 5988, 356 spare.  Gains: (0,0) 2->3 0.628, (1,1) 2->3 0.471 fit (100 left);
    # (0,0) 3->4 0.354 and every later one need 128: frozen.
    w = rc.refresh(sens)
    assert _widths(w) == {0: [3, 2], 1: [2, 3]}
    rc.commit(w, 8)  # the first 8-token blocks: 768 + 704 bytes each
    assert rc.stored_bytes() == 2944 and rc.remaining(0) == rc.remaining(1) == 8
    # 8 remaining tokens per item: 704 / 768 / 832, upgrades of 64; 3044 free, 2816 at 2 bits,
    # 228 spare: (0,0) 0.628 -> 164, (1,1) 0.471 -> 100, (0,0) 3->4 0.354 -> 36; (1,0) 0.314 frozen
    assert _widths(rc.refresh(sens)) == {0: [4, 2], 1: [2, 3]}
    # agent 1 exits: its block and its remaining capacity go; agent 0 alone has 1408 at 2 bits
    # against 4516 free: every upgrade fits
    assert rc.exit(1) == 1472
    assert rc.stored_bytes() == 1472
    w = rc.refresh(sens)
    assert _widths(w) == {0: [4, 4]}
    rc.commit(w, 8)
    assert [(n, list(b)) for n, b in rc.blocks[0]] == [(8, [3, 2]), (8, [4, 4])]
    assert rc.stored_bytes() == 1472 + 1664 and rc.remaining(0) == 0
    # a full agent has no items; a new one of 32 tokens needs 5632 at 2 bits against 2852 free
    assert rc.refresh(sens) == {}
    rc.start(2, 32)
    assert rc.refresh(sens) is None
    assert rc.exit(0) == 3136
    # zero sensitivity: every gain is 0 and ties; the rule still takes an upgrade that fits,
    # lowest index first: 5632 at 2 bits, 356 spare, upgrades of 256 -> one
    assert _widths(rc.refresh({})) == {2: [3, 2]}


def test_refresh_cycle_orders_items_by_agent_id():
    """One upgrade fits and every gain ties: it goes to the lowest agent id's first layer,
    whatever order the agents started in."""
    rc = comixkv.RefreshCycle(2816 + 64 + 10, 2, 1, 64)
    rc.start(5, 8)
    rc.start(3, 8)
    w = rc.refresh({5: [1.0, 1.0], 3: [1.0, 1.0]})
    assert _widths(w) == {3: [3, 2], 5: [2, 2]}


def test_refresh_cycle_stored_blocks_keep_their_widths():
    """Refreshes and commits never change a stored block; an exit frees exactly its blocks;
    stored bytes never exceed the budget."""
    rng = np.random.default_rng(3)
    L = 4
    rc = comixkv.RefreshCycle(5 * L * 640 * (8 * (128 + 48 + 4) + 4), L, 8, 128)  # 3 bits on average
    for a in range(5):
        rc.start(a, 640)
    history = []
    for step in range(6):
        w = rc.refresh({a: rng.lognormal(0, 1, L) for a in rc.blocks})
        assert w is not None
        rc.commit(w, 64)
        assert rc.stored_bytes() <= rc.budget
        history.append({a: [(n, b.copy()) for n, b in bl] for a, bl in rc.blocks.items()})
        for past in history:
            for a, bl in past.items():
                if a in rc.blocks:
                    assert all(n == m and np.array_equal(x, y) for (n, x), (m, y) in zip(bl, rc.blocks[a]))
        if step == 2:
            want = sum(rc.block_bytes(n, b) for n, b in rc.blocks[1])
            before = rc.stored_bytes()
            assert rc.exit(1) == want and rc.stored_bytes() == before - want

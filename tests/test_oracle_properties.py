"""Property-based checks of the oracle on random small shapes and values (hypothesis).

Each property follows from the definitions the oracle writes out, not from the
oracle itself:

* V codec (PolyKV explainer, section 2.B): the code of each rotated, normalised
  coordinate is the index of the nearest Lloyd-Max centroid (the thresholds are
  the midpoints), except exactly on a threshold; pack and unpack are inverse;
  a signed rotation changes no norm.
* K codec (section 2.B, per-tensor int8): |k - s q| <= s / 2 up to one
  rounding of the quotient, the largest |k| maps to +-127, and q(-k) = -q(k).
* Attention: the rotated-domain form (one inverse transform per output) equals
  decoding every token and then attending, for any pool and window sizes and
  bit widths, with or without signs.
* Allocation (CoMixKV article): the budget holds, and with equal byte steps
  more budget never raises the predicted error.
"""
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import attention, codec, comixkv, hadamard, lloyd_max

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def v_batch(draw):
    d = draw(st.sampled_from([64, 128]))
    bits = draw(st.sampled_from([2, 3, 4]))
    n = draw(st.integers(1, 12))
    seed = draw(st.integers(0, 2**31 - 1))
    scale = draw(st.sampled_from([1e-3, 1.0, 37.0]))
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((n, d)) * scale).astype(np.float32)
    if draw(st.booleans()):
        v[rng.integers(0, n)] = 0.0  # a zero vector
    signed = draw(st.booleans())
    signs = np.where(rng.random(d) < 0.5, -1.0, 1.0) if signed else None
    return v, bits, signs


@SETTINGS
@given(v_batch())
def test_v_code_is_the_nearest_centroid(case):
    v, bits, signs = case
    n, codes = codec.v_encode(v, bits, signs)
    cent, thr = lloyd_max.table_f32(bits)
    x = v if signs is None else (v * signs.astype(np.float32))
    y = hadamard.fwht_f32(x) * np.where(n > 0, np.float32(1) / np.where(n > 0, n, 1), 0).astype(np.float32)[:, None]
    near = np.argmin(np.abs(y[..., None].astype(np.float64) - cent.astype(np.float64)), axis=-1)
    tie = np.isin(y, thr)
    live = (n > 0)[:, None] & ~tie
    assert np.array_equal(codes[live], near[live])
    assert np.all(codes[n == 0] == 0)
    # norms do not see the signs
    n_plain, _ = codec.v_encode(v, bits)
    assert np.array_equal(n, n_plain)


@SETTINGS
@given(st.sampled_from([64, 128]), st.sampled_from([2, 3, 4]), st.integers(1, 4), st.integers(0, 2**31 - 1))
def test_pack_unpack_round_trip(d, bits, groups, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 1 << bits, (groups * 8, d)).astype(np.uint8)
    p = codec.pack_codes(c, bits)
    assert p.shape == (groups, d * bits)
    assert np.array_equal(codec.unpack_codes(p, d, bits), c)


@SETTINGS
@given(st.integers(1, 6), st.integers(1, 40), st.sampled_from([64, 128]), st.integers(0, 2**31 - 1),
       st.sampled_from([1e-4, 1.0, 300.0]))
def test_k_codec_error_bound_and_symmetry(h, t, d, seed, scale):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((h, t, d)) * scale).astype(np.float32)
    s, q = codec.k_quantize(k)
    amax = np.max(np.abs(k))
    assert s == np.float32(amax / np.float32(127.0))
    err = np.abs(k.astype(np.float64) - float(s) * q.astype(np.float64))
    assert np.all(err <= float(s) * (0.5 + 1e-5) + 1e-30)
    assert np.max(np.abs(q.astype(int))) == 127
    s2, q2 = codec.k_quantize(-k)
    assert s2 == s and np.array_equal(q2.astype(int), -q.astype(int))


@SETTINGS
@given(st.sampled_from([64, 128]), st.sampled_from([2, 3, 4]), st.integers(1, 70), st.integers(0, 9),
       st.integers(0, 2**31 - 1), st.booleans())
def test_rotated_form_equals_decode_then_attend(d, bits, t, s_len, seed, signed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((t, d)).astype(np.float32)
    v = rng.standard_normal((t, d)).astype(np.float32)
    q = rng.standard_normal((3, d))
    signs = np.where(rng.random(d) < 0.5, -1.0, 1.0) if signed else None
    ks, kq = codec.k_quantize(k)
    n, c = codec.v_encode(v, bits, signs)
    ksf = rng.standard_normal((s_len, d))
    vsf = rng.standard_normal((s_len, d))
    khat = codec.k_dequantize(ks, kq)
    vhat = codec.v_decode(n, c, bits, signs)
    want = attention.attend_pool_and_suffix(q, khat, vhat, ksf, vsf)
    # the rotated form accumulates before one inverse transform; signs apply after it
    got = attention.rotated_form(q, np.full(t, ks), kq, n, c, bits, ksf, vsf) if signs is None else None
    if signs is None:
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-10 * max(1.0, float(np.max(np.abs(want)))))
    else:
        # with signs: rotated form of the unsigned accumulation, then the signs on the pool part
        sigma = 1.0 / math.sqrt(d)
        sc = np.concatenate([sigma * q @ khat.T, sigma * q @ ksf.T], axis=1)
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        l = p.sum(axis=1, keepdims=True)
        cent, _ = lloyd_max.table_f32(bits)
        acc = (p[:, :t] * n.astype(np.float64)) @ cent.astype(np.float64)[c.astype(int)]
        o = signs * ((acc @ hadamard.hadamard_matrix(d).astype(np.float64)) / d) + p[:, t:] @ vsf
        np.testing.assert_allclose(o / l, want, rtol=0, atol=1e-10 * max(1.0, float(np.max(np.abs(want)))))


@SETTINGS
@given(st.integers(1, 12), st.integers(0, 2**31 - 1))
def test_allocation_budget_and_monotonicity(n, seed):
    rng = np.random.default_rng(seed)
    sens = rng.lognormal(0.0, 1.5, n).astype(np.float32)
    unit, base = int(rng.integers(50, 500)), int(rng.integers(500, 5000))
    cost = np.array([[base + 2 * unit, base + 3 * unit, base + 4 * unit]] * n, dtype=np.uint64)
    err = comixkv.error_factors()
    lo = int(cost[:, 0].sum())
    prev = math.inf
    for extra in range(0, 2 * n + 2):
        budget = lo + extra * unit
        bits = comixkv.allocate(sens, cost, err, budget)
        assert int(cost[np.arange(n), bits - 2].sum()) <= budget
        obj = comixkv.objective(sens, err, bits)
        assert obj <= prev + 1e-12
        prev = obj
    assert comixkv.allocate(sens, cost, err, lo - 1) is None

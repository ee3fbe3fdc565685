"""Pins of the oracle's K and V codecs and of the code-group packing.

PolyKV explainer, section 2.B: K to int8 under a per-tensor linear scale;
V by FWHT rotation, Lloyd-Max N(0, 1) codes and dequantisation by centroid
lookup plus inverse FWHT.  CoMixKV news article: 2/3/4-bit V per layer.
"""
import json
import os

import numpy as np
import pytest

from oracle import codec, hadamard, lloyd_max

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- K
def test_k_worked_example_scale_one():
    # amax = 127 gives scale exactly 1, so codes are rint(k) with ties to even
    k = np.array([127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -127.0, 0.49], dtype=np.float32)
    s, q = codec.k_quantize(k)
    assert s == np.float32(1.0)
    assert q.tolist() == [127, 2, 4, -2, 0, 0, 2, -127, 0]


def test_k_worked_example_scale_two():
    k = np.array([254.0, 5.0, 7.0, -3.0], dtype=np.float32)  # s = 2: 2.5 -> 2, 3.5 -> 4, -1.5 -> -2
    s, q = codec.k_quantize(k)
    assert s == np.float32(2.0) and q.tolist() == [127, 2, 4, -2]


def test_k_bounds_symmetry_and_error():
    rng = np.random.default_rng(4)
    k = (rng.standard_normal((8, 300, 128)) * rng.lognormal(0, 0.5, 128)).astype(np.float32)
    s, q = codec.k_quantize(k)
    amax = np.max(np.abs(k))
    assert s == np.float32(amax / np.float32(127.0))
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    i = np.unravel_index(np.argmax(np.abs(k)), k.shape)
    assert abs(int(q[i])) == 127
    err = np.abs(k.astype(np.float64) - float(s) * q.astype(np.float64))
    assert np.all(err <= 0.5 * float(s) * (1 + 1e-6) + 1e-30)
    s2, q2 = codec.k_quantize(-k)
    assert s2 == s and np.array_equal(q2, -q)


def test_k_zero_tensor():
    s, q = codec.k_quantize(np.zeros((2, 3, 64), dtype=np.float32))
    assert s == 0.0 and not q.any()


# ---------------------------------------------------------------- V
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_v_codes_are_nearest_centroid(bits, d):
    # Lloyd-Max thresholds are centroid midpoints, so the threshold count equals the
    # nearest centroid of the rotated, normalised coordinate (computed here in fp64)
    rng = np.random.default_rng(5)
    v = rng.standard_normal((400, d)).astype(np.float32)
    n, codes = codec.v_encode(v, bits)
    y = hadamard.fwht_f32(v).astype(np.float64) / n.astype(np.float64)[:, None]
    c, _ = lloyd_max.table_f32(bits)
    near = np.argmin(np.abs(y[..., None] - c.astype(np.float64)), axis=-1)
    # fp32 y differs from fp64 y by ~1e-7; allow mismatches only within that of a threshold
    _, t = lloyd_max.table_f32(bits)
    close = np.min(np.abs(y[..., None] - t.astype(np.float64)), axis=-1) < 1e-5
    assert np.all((codes == near) | close)
    assert np.mean(codes == near) > 0.999


def test_v_tie_goes_to_lower_code():
    # a coordinate exactly on a threshold takes the lower code (strict comparison)
    d, bits = 64, 3
    _, thr = lloyd_max.table_f32(bits)
    v = np.zeros((1, d), dtype=np.float32)
    v[0, 0] = 1.0  # H e_0 = all ones; n = 1 -> y_i = 1 for every i
    n, codes = codec.v_encode(v, bits)
    assert n[0] == 1.0
    expected = int(np.sum(np.float32(1.0) > thr))
    assert np.all(codes == expected)
    v2 = np.zeros((1, d), dtype=np.float32)
    v2[0, 0] = 1.0
    v2[0, 1] = 1.0  # H(e0 + e1): entries 2 or 0; n = sqrt(2); y = 0 on half the coords
    _, c2 = codec.v_encode(v2, bits)
    z = hadamard.fwht_f32(v2)[0]
    assert np.all(c2[0][z == 0] == 3)  # y = 0 equals tau_3 = 0: not greater, so code 3 (of 0..7)


def test_v_zero_vector():
    n, codes = codec.v_encode(np.zeros((3, 128), dtype=np.float32), 3)
    assert not n.any() and not codes.any()
    assert not codec.v_decode(n, codes, 3).any()


@pytest.mark.parametrize("bits,lo,hi", [(2, 0.9, 1.0), (3, 0.9, 1.0), (4, 0.9, 1.0)])
@pytest.mark.parametrize("d", [64, 128])
def test_v_relative_mse_band(bits, d, lo, hi):
    # ||v - v_hat||^2 / ||v||^2 = ||y - c||^2 / d: the per-coordinate Lloyd-Max distortion
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((2000, d)) * rng.lognormal(0, 0.5, d)).astype(np.float32)
    n, codes = codec.v_encode(v, bits)
    vh = codec.v_decode(n, codes, bits)
    rel = np.mean(np.sum((v - vh) ** 2, axis=1) / np.sum(v.astype(np.float64) ** 2, axis=1))
    c, t = lloyd_max.lloyd_max_normal(bits)
    dmse = lloyd_max.mse_closed_form(c, t)
    assert lo * dmse <= rel <= hi * dmse


def test_v_decode_is_inverse_transform_of_centroids():
    # v_hat = (n/d) H c: applying the fp32 FWHT to v_hat recovers n * c exactly enough
    rng = np.random.default_rng(7)
    v = rng.standard_normal((10, 64)).astype(np.float32)
    n, codes = codec.v_encode(v, 3)
    vh = codec.v_decode(n, codes, 3)
    c, _ = lloyd_max.table_f32(3)
    back = vh @ hadamard.hadamard_matrix(64).astype(np.float64)
    assert np.allclose(back, n[:, None] * c.astype(np.float64)[codes], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- packing
def test_pack_worked_examples():
    ex = json.load(open(os.path.join(GOLD, "pack_examples.json")))
    for case in ex["cases"]:
        b = case["bits"]
        codes = np.zeros((8, 64), dtype=np.uint8)
        codes[:, 0] = case["codes"]
        packed = codec.pack_group(codes, b)
        assert packed.size == 64 * b
        assert packed[:b].tobytes().hex() == case["bytes_hex"]
        assert not packed[b:].any()
        # the same field placed at dimension 5 lands at bytes [5b, 6b)
        codes2 = np.zeros((8, 64), dtype=np.uint8)
        codes2[:, 5] = case["codes"]
        p2 = codec.pack_group(codes2, b)
        assert p2[5 * b:6 * b].tobytes().hex() == case["bytes_hex"]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_pack_roundtrip_and_vectorised_agrees(bits, d):
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 2 ** bits, size=(3, 40, d)).astype(np.uint8)
    packed = codec.pack_codes(codes, bits)
    assert packed.shape == (3, 5, d * bits)
    assert np.array_equal(codec.unpack_codes(packed, d, bits), codes)
    for a in range(3):
        for g in range(5):
            assert np.array_equal(packed[a, g], codec.pack_group(codes[a, 8 * g:8 * g + 8], bits))


# ---- randomised rotation (sign vector before the FWHT), a codec variant
@pytest.mark.parametrize("d", [64, 128])
def test_signed_rotation_is_orthogonal_and_plain_when_all_positive(d):
    rng = np.random.default_rng(d)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    h = hadamard.hadamard_matrix(d).astype(np.float64)
    t = h @ np.diag(s)
    assert np.array_equal(t.T @ t, d * np.eye(d))
    v = rng.standard_normal((20, d)).astype(np.float32)
    n0, c0 = codec.v_encode(v, 3)
    n1, c1 = codec.v_encode(v, 3, np.ones(d))
    assert np.array_equal(n0, n1) and np.array_equal(c0, c1)
    assert np.array_equal(codec.v_decode(n0, c0, 3), codec.v_decode(n1, c1, 3, np.ones(d)))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_all_negative_signs_mirror_the_codes(bits):
    """Negating every coordinate negates y, and the symmetric table maps code c to 2^b - 1 - c."""
    rng = np.random.default_rng(bits)
    v = rng.standard_normal((50, 64)).astype(np.float32)
    n0, c0 = codec.v_encode(v, bits)
    n1, c1 = codec.v_encode(v, bits, -np.ones(64))
    assert np.array_equal(n0, n1)
    # except where y lies exactly on a threshold (a tie takes the lower code on both sides);
    # here that is y == 0, which the transform of -v also gives as +0.0
    y = hadamard.fwht_f32(v) * (np.float32(1) / n0)[:, None]
    _, thr = lloyd_max.table_f32(bits)
    tie = np.isin(y, thr)
    assert np.array_equal(c1.astype(int)[~tie], ((1 << bits) - 1 - c0.astype(int))[~tie])
    assert np.array_equal(c1[tie], c0[tie])
    rows = ~tie.any(axis=1)  # vectors without a tie decode to the same values
    np.testing.assert_allclose(codec.v_decode(n1, c1, bits, -np.ones(64))[rows], codec.v_decode(n0, c0, bits)[rows],
                               rtol=0, atol=1e-12)


def test_signed_rotation_fixes_hadamard_aligned_vectors():
    """A vector along a Hadamard row becomes one spike under the plain FWHT (the codec clips it);
    random signs spread it, so the error returns to the Lloyd-Max level."""
    d, bits = 128, 3
    rng = np.random.default_rng(9)
    h = hadamard.hadamard_matrix(d).astype(np.float32)
    v = h[rng.integers(0, d, 64)] * rng.lognormal(0.0, 1.0, (64, 1)).astype(np.float32)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)

    def rel_mse(signs):
        n, c = codec.v_encode(v, bits, signs)
        vh = codec.v_decode(n, c, bits, signs)
        return float(np.mean(np.sum((vh - v) ** 2, axis=1) / np.sum(v.astype(np.float64) ** 2, axis=1)))

    plain, signed = rel_mse(None), rel_mse(s)
    assert plain > 0.5                      # the spike at sqrt(d) = 11.3 is clipped to 2.15
    assert signed < 2.0 * 0.03455           # near D_3 for 3 bits


def test_signs_from_mask_bit_order():
    m = bytes([0b00000101] + [0] * 15)
    s = codec.signs_from_mask(m, 128)
    assert s[0] == -1 and s[1] == 1 and s[2] == -1 and np.all(s[3:] == 1)


# ---- last-bit conventions, pinned by hand-worked fp32 examples ---------------------------------
# Each example is an input on which the plausible alternative readings give different bytes.
# The intermediate values are written out as fp32 bit patterns so that each step can be checked
# with any correctly rounded fp32 calculator; the assertions are on the oracle's own output.

def _f(bits: int) -> np.float32:
    return np.frombuffer(int(bits).to_bytes(4, "little"), dtype=np.float32)[0]


def test_fwht_stage_order_is_ascending_half_width():
    """PolyKV explainer, section 2.B names the FWHT; the reading fixes butterflies with half-width
    1, 2, 4, ... (ascending).  x = (1, e, -1, 0, 0, ...), e = 2^-24, d = 128:
      ascending:  h=1 -> (fl(1+e), fl(1-e), -1, -1) = (1, 1-e, -1, -1)   [1+e is a tie -> even: 1]
                  h=2 -> z0 = 1 + (-1) = 0,  z1 = (1-e) - 1 = -e,  z2 = 2,  z3 = fl(2-e) = 2 [tie -> even]
      descending: the h >= 4 stages copy the block, h=2 -> (0, e, 2, e), h=1 -> z0 = 0 + e = e
    So z0 is +0 in the ascending order and 2^-24 in the descending one, and its 3-bit code is
    3 (y = 0 is not above the middle threshold 0) against 4.  The stages h >= 4 combine the first
    4-block with zero blocks, so the whole output is the 4-point result repeated."""
    e = np.float32(2.0 ** -24)
    x = np.zeros(128, np.float32)
    x[0], x[1], x[2] = 1.0, e, -1.0
    z = hadamard.fwht_f32(x)
    want = np.tile(np.array([0.0, -e, 2.0, 2.0], np.float32), 32)
    assert np.array_equal(z.view(np.uint32), want.view(np.uint32))  # bitwise: +0, not -0 or e
    n, codes = codec.v_encode(x[None], 3)
    # n = sqrt(fl(fl(1 + e^2) + 1)) = sqrt(2) rounded = 0x3fb504f3; y2 = y3 = 2 * fl(1/n) ~ 1.4142 -> code 6
    assert n[0].view(np.uint32) == 0x3FB504F3
    assert list(codes[0][:4]) == [3, 3, 6, 6] and np.array_equal(codes[0], np.tile(codes[0][:4], 32))


def test_v_normalisation_multiplies_by_the_rounded_reciprocal():
    """Reading: y = z * fl(1/n) (one fp32 division for the reciprocal, then fp32 products), not
    fl(z / n).  x = (a, b, 0, ...), d = 128, a = 0x3f553488, b = 0x3d2f22b9:
      a*a = 0x3f319075, b*b = 0x3aefa0fb, sum = 0x3f320845, n = sqrt = 0x3f557c6a
      z_even = fl(a + b) = 0x3f6026b4,  r = fl(1/n) = 0x3f997d7b
      z_even * r = 0x3f866500 = 1.049957275390625, which is exactly the 3-bit threshold tau_5
      fl(z_even / n) = 0x3f866501, one ulp above tau_5
    With the strict count the product reading gives code 5 (a tie goes to the lower code), the
    quotient reading code 6.  Odd coordinates: y = fl(a - b) * r = 0.9474 -> code 5."""
    a, b = _f(0x3F553488), _f(0x3D2F22B9)
    x = np.zeros(128, np.float32)
    x[0], x[1] = a, b
    _, thr = lloyd_max.table_f32(3)
    assert thr[5].view(np.uint32) == 0x3F866500
    n, codes = codec.v_encode(x[None], 3)
    assert n[0].view(np.uint32) == 0x3F557C6A
    assert np.all(codes[0] == 5)


def test_k_quotient_is_a_division_rounded_half_to_even():
    """Reading: q = rint(fl(k / s)), round half to even, s = fl(amax / 127).
    amax = 0x40b7c408 (5.742679...), k = 0x4082f381 (4.092224...):
      s = fl(amax / 127) = 0x3d393675
      fl(k / s) = 90.5 exactly          -> rint half-even = 90 (half away from zero would give 91)
      fl(k * fl(1/s)) = 90.50000762...  -> 91 (the reciprocal reading)
    and -k gives -90 (symmetric)."""
    amax, k = _f(0x40B7C408), _f(0x4082F381)
    s, q = codec.k_quantize(np.array([amax, k, -k], np.float32))
    assert np.float32(s).view(np.uint32) == 0x3D393675
    assert list(q) == [127, 90, -90]


# ---- codec variants (ablations): K per token, K per channel, corrected V norm ----------------------

def test_k_per_token_hand_worked():
    """One scale per K vector, the q8_0 rule on each vector alone.  Row 0: amax 254 -> s = 2,
    codes 254/2 = 127, 1/2 = 0.5 -> 0 (half to even), -127/2 = -63.5 -> -64, 0.5/2 -> 0.
    Row 1: the hand-worked division pin (90.5 -> 90).  Row 2: zeros -> s = 0, codes 0."""
    k = np.zeros((3, 4), np.float32)
    k[0] = [254.0, 1.0, -127.0, 0.5]
    k[1, :2] = [_f(0x40B7C408), _f(0x4082F381)]
    s, q = codec.k_quantize_per_token(k)
    assert s[0] == 2.0 and s[1].view(np.uint32) == 0x3D393675 and s[2] == 0.0
    assert q.tolist() == [[127, 0, -64, 0], [127, 90, 0, 0], [0, 0, 0, 0]]


def test_k_per_token_bounds():
    rng = np.random.default_rng(7)
    k = (rng.standard_normal((50, 128)) * rng.lognormal(0, 1, (50, 1))).astype(np.float32)
    s, q = codec.k_quantize_per_token(k)
    top = np.argmax(np.abs(k), axis=-1)
    assert np.all(np.abs(q[np.arange(50), top]) == 127)
    err = np.abs(k.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))


def test_k_per_channel_hand_worked_and_later_appends_clamp():
    """Channel 0: [127, -63.5, 1.5] -> s = 1, codes 127, -64 (half to even), 2; channel 1 all zero
    -> s = 0, codes 0.  A later block keeps the first block's scales: 300 clamps to 127, and the
    zero-scale channel stays 0 whatever its values (stored codes are never re-quantised)."""
    k = np.array([[127.0, 0.0], [-63.5, 0.0], [1.5, 0.0]], np.float32)
    s = codec.k_channel_scales(k)
    assert s.tolist() == [1.0, 0.0]
    assert codec.k_quantize_per_channel(k, s).tolist() == [[127, 0], [-64, 0], [2, 0]]
    later = np.array([[300.0, 5.0], [-2.5, -7.0]], np.float32)
    assert codec.k_quantize_per_channel(later, s).tolist() == [[127, 0], [-2, 0]]


def test_corrected_norm_reconstructs_a_basis_vector_exactly():
    """v = e_0: H v is the all-ones vector, y = 1 everywhere, the 3-bit code of 1 is 5 (between
    the thresholds 0.5005 and 1.04996), so c_hat = c_5 * ones and ||c_hat|| = sqrt(d) c_5.  The
    plain norm decodes to (1/d) H (c_5 ones) = c_5 e_0 (shrunk to 0.756); the corrected norm
    n' = sqrt(d) / (sqrt(d) c_5) = 1 / c_5 decodes to e_0 itself."""
    cent, _ = lloyd_max.table_f32(3)
    for d in (64, 128):
        v = np.zeros((1, d), np.float32)
        v[0, 0] = 1.0
        n0, c0 = codec.v_encode(v, 3)
        n1, c1 = codec.v_encode(v, 3, corrected_norm=True)
        assert np.all(c0 == 5) and np.array_equal(c0, c1)
        assert n0[0] == 1.0 and abs(float(n1[0]) * float(cent[5]) - 1.0) <= 2.0 ** -22  # n' = 1 / c_5 (2 ulp)
        plain = codec.v_decode(n0, c0, 3)[0]
        corr = codec.v_decode(n1, c1, 3)[0]
        assert abs(plain[0] - cent[5]) < 1e-7 and np.max(np.abs(plain[1:])) < 1e-7
        assert abs(corr[0] - 1.0) < 2e-7 and np.max(np.abs(corr[1:])) < 1e-7


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_corrected_norm_keeps_the_input_norm(bits, d):
    """||v_hat|| = (n'/d) ||H c_hat|| = n' ||c_hat|| / sqrt(d) = ||v|| up to fp32 rounding; the codes
    are the plain codec's; zero vectors keep norm 0."""
    rng = np.random.default_rng(bits * d)
    v = (rng.standard_normal((200, d)) * rng.lognormal(0, 1, (200, 1))).astype(np.float32)
    v[3] = 0.0
    n0, c0 = codec.v_encode(v, bits)
    n1, c1 = codec.v_encode(v, bits, corrected_norm=True)
    assert np.array_equal(c0, c1) and n1[3] == 0.0
    vn = np.linalg.norm(v.astype(np.float64), axis=-1)
    got = np.linalg.norm(codec.v_decode(n1, c1, bits), axis=-1)
    ok = vn > 0
    assert np.all(np.abs(got[ok] - vn[ok]) <= 4e-7 * vn[ok])
    # the plain norm's decode is shorter by ||c_hat|| / sqrt(d), which is below 1 on average
    plain = np.linalg.norm(codec.v_decode(n0, c0, bits), axis=-1)
    assert np.mean(plain[ok] / vn[ok]) < 1.0

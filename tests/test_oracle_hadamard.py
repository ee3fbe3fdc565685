"""Pins of the oracle's Hadamard transform and norm against closed forms.

PolyKV explainer, section 2.B (value rotation by the FWHT).  The pins are
mathematical facts of the Sylvester Hadamard matrix, not restatements of the
oracle's code: the closed form H[i][j] = (-1)^popcount(i & j), H @ H = d I,
exactness of fp32 butterflies on small integers, and Parseval's identity.
"""
import numpy as np
import pytest

from oracle import hadamard

DIMS = [1, 2, 4, 8, 16, 32, 64, 128]


@pytest.mark.parametrize("d", DIMS)
def test_sylvester_matches_popcount_closed_form(d):
    h = hadamard.hadamard_matrix(d)
    i = np.arange(d)[:, None]
    j = np.arange(d)[None, :]
    pc = np.vectorize(lambda x: bin(int(x)).count("1"))(i & j)
    assert np.array_equal(h, np.where(pc % 2 == 0, 1, -1))


@pytest.mark.parametrize("d", DIMS)
def test_h_squared_is_d_identity(d):
    h = hadamard.hadamard_matrix(d)
    assert np.array_equal(h @ h, d * np.eye(d, dtype=np.int64))
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_of_unit_vectors_gives_columns(d):
    h = hadamard.hadamard_matrix(d)
    eye = np.eye(d, dtype=np.float32)
    cols = hadamard.fwht_f32(eye)  # row j = FWHT(e_j)
    assert np.array_equal(cols, h.T.astype(np.float32))


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_h_h_is_d_identity_in_fp32(d):
    # H @ H = d I computed entirely by the fp32 butterflies (exact: small integers)
    eye = np.eye(d, dtype=np.float32)
    hh = hadamard.fwht_f32(hadamard.fwht_f32(eye))
    assert np.array_equal(hh, d * eye)


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_exact_on_small_integers(d):
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1000, size=(50, d)).astype(np.float32)
    ref = x.astype(np.int64) @ hadamard.hadamard_matrix(d).T
    assert np.array_equal(hadamard.fwht_f32(x), ref.astype(np.float32))


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_error_bound_and_parseval(d):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, d)).astype(np.float32)
    z = hadamard.fwht_f32(x).astype(np.float64)
    ref = x.astype(np.float64) @ hadamard.hadamard_matrix(d).astype(np.float64)
    # log2(d) stages, each adding at most one rounding of a partial sum <= sum |x|
    bound = np.log2(d) * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(axis=1, keepdims=True) * 2
    assert np.all(np.abs(z - ref) <= bound)
    lhs = (z ** 2).sum(axis=1)
    rhs = d * (x.astype(np.float64) ** 2).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-6)


def test_norm_exact_cases_and_bound():
    x = np.zeros((3, 64), dtype=np.float32)
    x[0, 0], x[0, 5] = 3.0, 4.0
    x[1, :] = 1.0  # sqrt(64) = 8
    n = hadamard.norm_f32(x)
    assert n[0] == 5.0 and n[1] == 8.0 and n[2] == 0.0
    rng = np.random.default_rng(3)
    for d in (64, 128):
        y = rng.standard_normal((500, d)).astype(np.float32) * rng.lognormal(0, 0.5, d).astype(np.float32)
        got = hadamard.norm_f32(y).astype(np.float64)
        ref = np.sqrt((y.astype(np.float64) ** 2).sum(axis=1))
        assert np.all(np.abs(got - ref) <= (np.log2(d) + 2) * 2.0 ** -24 * ref)


def test_tree_order_is_the_halving_tree():
    # Cases where association matters in fp32 (the ulp of 2^24 is 2, so 2^24 + 1 rounds
    # to 2^24).  The halving tree pairs element i with i + d/2 first.
    # squares [1, 2^24, 1, 1]: halving (1+1), (2^24+1) -> 2 + 2^24 = 2^24 + 2;
    # left-to-right ((1 + 2^24) + 1) + 1 would give 2^24.
    x2 = np.array([1.0, 2.0 ** 12, 1.0, 1.0], dtype=np.float32)
    assert hadamard.sumsq_tree_f32(x2) == np.float32(2.0 ** 24 + 2)
    # squares [2^24, 0, 1, 1]: halving (2^24+1), (0+1) -> 2^24 + 1 -> 2^24;
    # adjacent pairs (2^24+0), (1+1) would give 2^24 + 2.
    x3 = np.array([2.0 ** 12, 0.0, 1.0, 1.0], dtype=np.float32)
    assert hadamard.sumsq_tree_f32(x3) == np.float32(2.0 ** 24)

"""Checks of the seeded input generators (shapes, determinism, bf16 rounding, bit mix)."""
import numpy as np

import workloads as wl


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], dtype=np.float32)
    b = wl.f32_to_bf16_bits(x)
    back = wl.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                       # tie between 1 and 1 + 2^-7: even mantissa wins
    assert back[2] == np.float32(1.0 + 2 ** -6)  # tie between 1 + 2^-7 and 1 + 2^-6: even wins
    assert back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_slices_are_deterministic_and_independent():
    w = wl.LLAMA3_8B.replace(n_layers=2, pool_tokens=40, n_agents=3, sfx_tokens=5)
    a = w.pool_k(0, 1)
    b = w.pool_k(0, 1)
    assert np.array_equal(a.raw, b.raw) and a.raw.dtype == np.uint16
    assert a.f32.shape == (8, 40, 128)
    assert not np.array_equal(w.pool_k(0, 0).raw, a.raw)
    assert not np.array_equal(w.pool_v(0, 1).raw, a.raw)
    assert w.queries(3, 2).f32.shape == (2, 32, 128)
    assert w.sfx_k(1, 0).f32.shape == (8, 5, 128)


def test_distributions():
    w = wl.TINY
    k = w.pool_k(0, 0).f32
    assert k.dtype == np.float32
    big = np.sum(np.std(k[0], axis=0) > 4.0)
    assert big == 2  # two outlier channels scaled by 8
    w2 = wl.SMOLLM2.replace(n_layers=1, pool_tokens=400)
    kk = w2.pool_k(0, 0).f32
    assert np.sum(np.std(kk, axis=1) > 5.0) == 20  # round(1% of 32 * 64) channels scaled by 10


def test_mixed_bits_average_three():
    w = wl.QWEN3_32B_MIXED
    for p in range(w.n_pools):
        b = w.v_bits(p)
        assert b.shape == (64,) and sorted(set(b.tolist())) == [2, 3, 4]
        assert b.mean() == 3.0 and (b == 3).sum() == 22
    assert not np.array_equal(w.v_bits(0), w.v_bits(1))


def test_suffix_length_modes():
    assert wl.LLAMA3_8B.sfx_len(0) == 1 and wl.LLAMA3_8B.sfx_len(127) == 128
    assert wl.LLAMA3_8B_LONG.sfx_len(5) == 256
    assert wl.TINY.sfx_len(0) == 0

"""Pins of the oracle's fp64 decode attention.

PolyKV explainer, section 2.A (PooledAgent: agents attend over the pool's
decoded K/V plus their own new tokens); section 2.B (dequantisation by
centroid lookup and inverse FWHT).  Pins: scalar brute force on tiny inputs,
PyTorch's CPU scaled_dot_product_attention in float64, special cases with
closed-form answers, permutation invariance, GQA sharing, independence of
agents, and equality of the rotated-domain form with decode-then-attend.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, codec, pool_image


def brute(q, k, v, sigma):
    """Scalar loops over the definition softmax(sigma q.k) v, no vector ops."""
    R, d = len(q), len(q[0])
    out = []
    for r in range(R):
        s = [sigma * sum(q[r][i] * k[t][i] for i in range(d)) for t in range(len(k))]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        out.append([sum(w[t] * v[t][i] for t in range(len(k))) / z for i in range(d)])
    return np.array(out)


def test_matches_scalar_brute_force():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((13, 8)) * 2
    v = rng.standard_normal((13, 8))
    got = attention.attend(q, k, v)
    ref = brute(q.tolist(), k.tolist(), v.tolist(), 1 / math.sqrt(8))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 128))
    k = rng.standard_normal((300, 128)) * 3
    v = rng.standard_normal((300, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None], torch.from_numpy(v)[None, None]
    )[0, 0].numpy()
    assert np.allclose(attention.attend(q, k, v), ref, rtol=1e-12, atol=1e-13)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((1, 64))
    o = attention.attend(rng.standard_normal((5, 64)), rng.standard_normal((1, 64)), v)
    assert np.allclose(o, np.repeat(v, 5, axis=0), rtol=0, atol=1e-15)


def test_zero_query_returns_mean_value():
    rng = np.random.default_rng(14)
    k = rng.standard_normal((50, 64))
    v = rng.standard_normal((50, 64))
    assert np.allclose(attention.attend(np.zeros((1, 64)), k, v)[0], v.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_dominant_score_selects_its_value():
    rng = np.random.default_rng(15)
    k = rng.standard_normal((40, 64))
    v = rng.standard_normal((40, 64))
    q = 200.0 * k[17:18] / np.linalg.norm(k[17])
    k[17] *= 5.0
    assert np.allclose(attention.attend(q, k, v)[0], v[17], atol=1e-9)


def test_token_permutation_invariance():
    rng = np.random.default_rng(16)
    q = rng.standard_normal((2, 64))
    k = rng.standard_normal((30, 64))
    v = rng.standard_normal((30, 64))
    p = rng.permutation(30)
    assert np.allclose(attention.attend(q, k, v), attention.attend(q, k[p], v[p]), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rotated_form_equals_decode_then_attend(bits):
    rng = np.random.default_rng(17)
    d, T, S = 128, 77, 9
    k = (rng.standard_normal((T, d)) * rng.lognormal(0, 0.5, d)).astype(np.float32)
    v = (rng.standard_normal((T, d)) * rng.lognormal(0, 0.5, d)).astype(np.float32)
    s, kq = codec.k_quantize(k)
    n, codes = codec.v_encode(v, bits)
    khat = codec.k_dequantize(s, kq)
    vhat = codec.v_decode(n, codes, bits)
    q = rng.standard_normal((4, d))
    ks = rng.standard_normal((S, d))
    vs = rng.standard_normal((S, d))
    a = attention.attend_pool_and_suffix(q, khat, vhat, ks, vs)
    b = attention.rotated_form(q, np.full(T, s), kq, n, codes, bits, ks, vs)
    assert np.max(np.abs(a - b)) < 1e-12


def test_decode_call_gqa_sharing_and_agent_independence():
    rng = np.random.default_rng(18)
    L, Hkv, G, d, T, S = 2, 2, 3, 64, 40, 5
    img = pool_image.PoolImage(L, Hkv, d, T, [3, 2])
    img.append(0, rng.standard_normal((L, Hkv, T, d)).astype(np.float32),
               rng.standard_normal((L, Hkv, T, d)).astype(np.float32))
    sk = rng.standard_normal((3, L, Hkv, S, d))
    sv = rng.standard_normal((3, L, Hkv, S, d))
    q = rng.standard_normal((3, L, Hkv * G, d))
    lens = [0, 3, 5]
    args = dict(decoded=lambda p, l, g: img.decoded_layer(l, g), k_sfx=lambda a, l: sk[a, l],
                v_sfx=lambda a, l: sv[a, l], n_kv_heads=Hkv)
    out = attention.decode_call(q, [0, 0, 0], sfx_len=lens, **args)
    # heads of one group attend to the same K/V: equal queries give equal outputs
    q2 = q.copy()
    q2[1, 0, 1] = q2[1, 0, 0]
    out2 = attention.decode_call(q2, [0, 0, 0], sfx_len=lens, **args)
    assert np.allclose(out2[1, 0, 1], out2[1, 0, 0], rtol=0, atol=1e-14)
    # an agent's output does not depend on the other agents in the call
    solo = attention.decode_call(q[1:2], [0], sfx_len=[3], decoded=args["decoded"],
                                 k_sfx=lambda a, l: sk[1, l], v_sfx=lambda a, l: sv[1, l], n_kv_heads=Hkv)
    assert np.allclose(solo[0], out[1], rtol=0, atol=1e-13)
    # head h uses kv head h // G
    khat, vhat = img.decoded_layer(1, 1)
    ref = attention.attend_pool_and_suffix(q[2, 1, 4:5], khat, vhat, sk[2, 1, 1, :5], sv[2, 1, 1, :5])
    assert np.allclose(out[2, 1, 4], ref[0], rtol=0, atol=1e-13)


def test_max_rel_error_definition():
    ref = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0]])
    out = ref + np.array([[0.002, 0.0, 0.0], [1e-7, 0.0, 0.0]])
    assert attention.max_rel_error(out, ref) == pytest.approx(max(0.002 / 2.0, 1e-7 / 1e-6))


def test_private_segment_equals_a_second_append_block():
    """A pool appended in two blocks decodes to the same K/V (K scales are per block, V codes per
    token) as a pool of the first block plus a private segment of the second, so attending to
    pool + private segment must give exactly what attending to the two-block pool gives."""
    rng = np.random.default_rng(7)
    H, d, Hq = 2, 64, 4
    k1, v1 = rng.standard_normal((1, H, 40, d)).astype(np.float32), rng.standard_normal((1, H, 40, d)).astype(np.float32)
    k2 = (3 * rng.standard_normal((1, H, 24, d))).astype(np.float32)
    v2 = (0.5 * rng.standard_normal((1, H, 24, d))).astype(np.float32)
    whole = pool_image.PoolImage(1, H, d, 64, [3])
    whole.append(0, k1, v1)
    whole.append(0, k2, v2)
    first = pool_image.PoolImage(1, H, d, 40, [3])
    first.append(0, k1, v1)
    second = pool_image.PoolImage(1, H, d, 24, [3])
    second.append(0, k2, v2)
    q = rng.standard_normal((2, 1, Hq, d))
    ks = rng.standard_normal((2, 1, H, 5, d))
    vs = rng.standard_normal((2, 1, H, 5, d))
    ref = attention.decode_call(q, [0, 0], lambda p, l, g: whole.decoded_layer(l, g), lambda a, l: ks[a, l],
                                lambda a, l: vs[a, l], [5, 3], H)
    out = attention.decode_call(q, [0, 0], lambda p, l, g: first.decoded_layer(l, g), lambda a, l: ks[a, l],
                                lambda a, l: vs[a, l], [5, 3], H,
                                private=lambda a, l, g: second.decoded_layer(l, g))
    assert np.array_equal(out, ref)
    # an agent without a private segment (None) is unaffected by the others having one
    mixed = attention.decode_call(q, [0, 0], lambda p, l, g: first.decoded_layer(l, g), lambda a, l: ks[a, l],
                                  lambda a, l: vs[a, l], [5, 3], H,
                                  private=lambda a, l, g: second.decoded_layer(l, g) if a == 0 else None)
    plain = attention.decode_call(q, [0, 0], lambda p, l, g: first.decoded_layer(l, g), lambda a, l: ks[a, l],
                                  lambda a, l: vs[a, l], [5, 3], H)
    assert np.array_equal(mixed[0], ref[0]) and np.array_equal(mixed[1], plain[1])
    assert not np.allclose(plain[0], ref[0])  # the segment does change the output

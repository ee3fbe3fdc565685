"""Pins of the pool layout and of the pool's size claims.

PolyKV explainer: section 2 (compression-ratio equation) gives
16 / ((8 + 3) / 2) = 2.91x against bf16; section 2.A and section 4 (memory
efficiency) say the pool is stored once and its size does not depend on the
number of agents; section 4 quotes 15 agents at 4K going from 19.8 GB to
0.45 GB, a 44x ratio.  QKVShare blog, section 2.1: KV bytes =
2 * tokens * hidden * layers * bytes per element.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec, pool_image


def test_layout_regions_and_alignment():
    lay = pool_image.layout(3, 2, 64, 100, [2, 3, 4])
    assert lay.tc == 128
    assert lay.kq == 0
    assert lay.vn == pool_image._align(3 * 2 * 128 * 64)
    assert lay.ks == pool_image._align(lay.vn + 3 * 2 * 128 * 4)
    assert lay.vmax == pool_image._align(lay.ks + 3 * 128 * 4)
    sizes = [2 * 128 * 64 * b // 8 for b in (2, 3, 4)]
    assert np.diff(lay.vc).tolist() == sizes
    for off in [lay.kq, lay.vn, lay.ks, lay.vmax, *lay.vc, lay.amax, lay.total]:
        assert off % 256 == 0
    assert lay.total >= lay.amax + 3 * 4


def test_ratio_without_norm_is_32_over_11():
    # per token and kv head at d = 128: K 8 bits, V 3 bits per element, against bf16 K and V
    d = 128
    compressed_bits = d * 8 + d * 3
    bf16_bits = 2 * d * 16
    assert Fraction(bf16_bits, compressed_bits) == Fraction(16, Fraction(11, 2)) == Fraction(32, 11)


@pytest.mark.parametrize("d,b,per_token,ratio", [(64, 3, 92, 2.783), (128, 3, 180, 2.844),
                                                   (128, 2, 164, 3.122), (128, 4, 196, 2.612)])
def test_bytes_per_token_with_norm(d, b, per_token, ratio):
    assert d + d * b // 8 + 4 == per_token
    assert abs(4 * d / per_token - ratio) < 1e-3


def test_pool_size_independent_of_agents_and_fifteen_agent_ratio():
    # Llama-3-8B shape: 32 layers, 8 kv heads, d 128, 4096 tokens, 3-bit V
    lay = pool_image.layout(32, 8, 128, 4096, [3] * 32)
    bf16_one = pool_image.bf16_kv_bytes(32, 8, 128, 4096)
    assert bf16_one == 536_870_912
    # the pool is one object: N agents read the same bytes
    for n_agents in (1, 3, 10, 15):
        total_private = n_agents * bf16_one
        ratio = total_private / lay.total
        assert ratio == pytest.approx(n_agents * bf16_one / lay.total)
    r15 = 15 * bf16_one / lay.total
    # the pages' 19.8 / 0.45 = 44 is ~15 x 2.91 (= 43.6); with the 4-byte norm and
    # per-token K scale this layout gives about 42.6
    assert 42.0 < r15 < 43.6
    assert abs(19.8 / 0.45 - 15 * 16 / 5.5) < 0.5


def test_bf16_formula_matches_blog_example():
    # QKVShare blog, section 2.1: 7B, 32 layers, hidden 4096, 2048 tokens, FP16 -> about 1 GB
    assert pool_image.bf16_kv_bytes(32, 32, 128, 2048) == 2 * 2048 * 4096 * 32 * 2
    assert abs(pool_image.bf16_kv_bytes(32, 32, 128, 2048) / 2 ** 30 - 1.0) < 1e-9


def test_appends_are_write_once_blocks():
    rng = np.random.default_rng(9)
    img = pool_image.PoolImage(2, 2, 64, 80, [3, 2])
    k1 = rng.standard_normal((2, 2, 37, 64)).astype(np.float32)
    v1 = rng.standard_normal((2, 2, 37, 64)).astype(np.float32)
    img.append(0, k1, v1)
    snap_kq = img.kq.copy()
    snap_codes = img.codes.copy()
    k2 = 5 * rng.standard_normal((2, 2, 20, 64)).astype(np.float32)
    v2 = rng.standard_normal((2, 2, 20, 64)).astype(np.float32)
    img.append(0, k2, v2)
    assert img.n_tokens.tolist() == [57, 57]
    assert np.array_equal(img.kq[:, :, :37], snap_kq[:, :, :37])
    assert np.array_equal(img.codes[:, :, :37], snap_codes[:, :, :37])
    for l in range(2):
        s1, _ = codec.k_quantize(k1[l])
        s2, _ = codec.k_quantize(k2[l])
        assert np.all(img.ks[l, :37] == s1) and np.all(img.ks[l, 37:57] == s2)
        assert np.array_equal(img.vmax[l], np.maximum(img.vn[l, :, :37].max(1), img.vn[l, :, 37:57].max(1)))
    with pytest.raises(ValueError):
        img.append(0, np.concatenate([k2, k2], axis=2), np.concatenate([v2, v2], axis=2))  # 57 + 40 > 80
    # packed groups: bits of tokens not yet written are zero
    packed = img.packed_codes(1)  # layer 1 has 2-bit codes
    assert packed.shape == (2, 96 // 8, 64 * 2)
    assert not packed[:, 8:].any()  # groups 8.. hold tokens 64.. which do not exist
    un = codec.unpack_codes(packed, 64, 2)
    assert not un[:, 57:].any()


def test_image_bytes_place_every_region():
    rng = np.random.default_rng(10)
    img = pool_image.PoolImage(2, 1, 64, 40, [3, 4])
    img.append(0, rng.standard_normal((2, 1, 40, 64)).astype(np.float32),
               rng.standard_normal((2, 1, 40, 64)).astype(np.float32))
    buf = img.image()
    lay = img.lay
    assert buf.size == lay.total
    kq = buf[:2 * 1 * lay.tc * 64].view(np.int8).reshape(2, 1, lay.tc, 64)
    assert np.array_equal(kq, img.kq)
    vn = buf[lay.vn:lay.vn + 2 * lay.tc * 4].view(np.float32).reshape(2, 1, lay.tc)
    assert np.array_equal(vn, img.vn)
    vc1 = buf[lay.vc[1]:lay.vc[2]].reshape(1, lay.tc // 8, 64 * 4)
    assert np.array_equal(vc1, img.packed_codes(1))
    assert not buf[lay.amax:].any()


def test_shard_decodes_like_the_whole_pool_and_tiles_it():
    """A kv-head shard decodes each of its heads exactly as the whole pool does, and the
    shards of a partition of the heads hold exactly the whole pool's per-head data."""
    rng = np.random.default_rng(5)
    L, H, d, T = 3, 4, 64, 70
    img = pool_image.PoolImage(L, H, d, 96, [2, 3, 4])
    img.append(0, rng.standard_normal((L, H, T, d)), rng.standard_normal((L, H, T, d)))
    assert np.array_equal(img.shard(0, H).image(), img.image())
    parts = [(0, 1), (1, 2), (3, 1)]
    shards = [img.shard(h0, hc) for h0, hc in parts]
    for (h0, hc), sh in zip(parts, shards):
        assert sh.lay.total == pool_image.layout(L, hc, d, 96, [2, 3, 4]).total
        for l in range(L):
            for g in range(hc):
                kf, vf = img.decoded_layer(l, h0 + g)
                ks_, vs_ = sh.decoded_layer(l, g)
                assert np.array_equal(kf, ks_) and np.array_equal(vf, vs_)
    assert np.array_equal(np.concatenate([s.kq for s in shards], axis=1), img.kq)
    assert np.array_equal(np.concatenate([s.codes for s in shards], axis=1), img.codes)
    assert np.array_equal(np.concatenate([s.vmax for s in shards], axis=1), img.vmax)
    for s in shards:
        assert np.array_equal(s.ks, img.ks)
    with pytest.raises(ValueError):
        img.shard(3, 2)


@pytest.mark.parametrize("k_scale", [pool_image.K_TOKEN, pool_image.K_CHANNEL])
def test_variant_layouts_and_decoding(k_scale):
    """Per-token scales take [L][Hkv][tc] floats, per-channel ones [L][Hkv][d] (and a per-channel
    amax scratch); decoding uses each token's or channel's scale; a later append keeps the
    first block's channel scales and every earlier byte."""
    L, H, d, cap = 2, 3, 64, 70
    lay = pool_image.layout(L, H, d, cap, [3, 2], k_scale)
    base = pool_image.layout(L, H, d, cap, [3, 2])
    ks_bytes = L * H * lay.tc * 4 if k_scale == pool_image.K_TOKEN else L * H * d * 4
    assert lay.vmax - lay.ks >= ks_bytes and lay.vmax - lay.ks < ks_bytes + 256
    assert lay.total >= base.total
    rng = np.random.default_rng(5)
    img = pool_image.PoolImage(L, H, d, cap, [3, 2], k_scale=k_scale)
    k1 = rng.standard_normal((L, H, 40, d)).astype(np.float32)
    v1 = rng.standard_normal((L, H, 40, d)).astype(np.float32)
    img.append(0, k1, v1)
    before = img.image().copy()
    k2 = 3.0 * rng.standard_normal((L, H, 30, d)).astype(np.float32)
    img.append(0, k2, rng.standard_normal((L, H, 30, d)).astype(np.float32))
    after = img.image()
    assert np.array_equal(after[lay.kq:lay.kq + L * H * lay.tc * d].reshape(L, H, lay.tc, d)[:, :, :40],
                          before[lay.kq:lay.kq + L * H * lay.tc * d].reshape(L, H, lay.tc, d)[:, :, :40])
    khat, _ = img.decoded_layer(1, 2)
    if k_scale == pool_image.K_TOKEN:
        s, q = codec.k_quantize_per_token(k2[1, 2])
        assert np.array_equal(khat[40:], s[:, None].astype(np.float64) * q)
    else:
        s = codec.k_channel_scales(k1[1, 2])
        assert np.array_equal(img.ks[1, 2], s)
        assert np.array_equal(khat[40:], s[None, :].astype(np.float64) * codec.k_quantize_per_channel(k2[1, 2], s))
        assert np.max(np.abs(img.kq[1, 2, 40:70])) == 127  # the larger later block clamps
    sh = img.shard(1, 2)
    assert np.array_equal(sh.decoded_layer(0, 1)[0], img.decoded_layer(0, 2)[0])

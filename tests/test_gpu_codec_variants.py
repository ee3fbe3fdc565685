"""GPU parity of the codec variants measured as ablations: K int8 per token and per
channel, and the corrected V norm ||v|| sqrt(d) / ||c_hat||.

The pages name a per-tensor K scale and a per-vector V norm (PolyKV explainer,
section 2.B); the QKVShare blog (section 3.2) weighs per-tensor, per-token and
per-channel granularity.  Pool images must equal the oracle's byte for byte
(per-channel scales from the first append, later appends clamping; appends
starting inside a code group; mixed bits; rotation signs), and decode outputs
must stay within 1e-3 of the fp64 oracle on both pool kernels, with suffixes,
row blocks, private segments and kv-head shards.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention, pool_image
from quantized_shared_kv_amd import polykv as pk

pytestmark = pytest.mark.gpu

TOL = 1e-3
TOK, CHAN = pk.KSCALE_TOKEN, pk.KSCALE_CHANNEL
VARIANTS = {"k_token": (TOK, 0), "k_channel": (CHAN, 0), "v_corrected": (0, 1), "k_token_v_corrected": (TOK, 1),
            "k_channel_v_corrected": (CHAN, 1)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()
    yield


def H():
    import gpu_helpers

    return gpu_helpers


IMAGE_CASES = {
    "gqa_bf16_d128_mixed_two_appends": (wl.LLAMA3_8B.replace(n_layers=3, pool_tokens=157, v_bits_mode="mixed"), 3,
                                        [101, 56]),
    "d64_fp32_three_appends": (wl.TINY.replace(n_layers=2, n_kv_heads=2, n_q_heads=2, pool_tokens=90,
                                               v_bits_mode="mixed"), 2, [5, 3, 82]),
    "mha_bf16_d64_outlier_channels": (wl.SMOLLM2.replace(n_layers=2, n_q_heads=4, n_kv_heads=4, pool_tokens=77), 2,
                                      None),
}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("case", sorted(IMAGE_CASES))
def test_variant_images_bit_exact(case, variant):
    w, layers, chunks = IMAGE_CASES[case]
    ks, vn = VARIANTS[variant]
    print(f"[variants] image {case} {variant}", flush=True)
    dp, ref = H().build_pair(w, 0, layers=layers, chunks=chunks, k_scale=ks, v_norm=vn)
    mism = H().compare_image(dp, ref)
    assert all(v == 0 for v in mism.values()), mism


def test_per_channel_later_append_clamps_on_device():
    """A second append larger than the first: its codes clamp at +-127 under the first block's
    channel scales, exactly as the oracle's."""
    h = H()
    print("[variants] per-channel clamp", flush=True)
    rng = np.random.default_rng(12)
    L, Hh, d = 1, 2, 128
    dp = h.DevicePool(L, Hh, d, 64, [3], k_scale=CHAN)
    ref = pool_image.PoolImage(L, Hh, d, 64, [3], k_scale=pool_image.K_CHANNEL)
    for scale, n in ((1.0, 20), (5.0, 30)):
        k = (scale * rng.standard_normal((L, Hh, n, d))).astype(np.float32)
        v = rng.standard_normal((L, Hh, n, d)).astype(np.float32)
        ref.append(0, k, v)
        dp.append(0, torch.from_numpy(k).to(h.DEV), torch.from_numpy(v).to(h.DEV))
    assert np.max(np.abs(ref.kq[0, :, 20:50])) == 127
    mism = h.compare_image(dp, ref)
    assert all(x == 0 for x in mism.values()), mism


DECODE = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=300, sfx_tokens=24)


@pytest.mark.parametrize("kernel", [pk.KERNEL_DEFAULT, pk.KERNEL_VALU])
@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_variant_decode_matches_oracle(variant, kernel):
    """15 agents (60 rows; per-channel pools take fp16 hi + lo query operands: row blocks of 48)."""
    h = H()
    ks, vn = VARIANTS[variant]
    print(f"[variants] decode {variant} kernel={kernel}", flush=True)
    A = 15
    dp, ref = h.build_pair(DECODE, 0, layers=2, k_scale=ks, v_norm=vn)
    q, q32 = h.make_queries(DECODE, 0, range(A))
    sk, sv, fk, fv = h.make_suffix(DECODE, range(A), 2)
    lens = [(3 * a) % 25 for a in range(A)]
    out = h.run_decode([dp.pool] * A, q, (sk, sv), lens, kernel=kernel)
    want = h.oracle_decode(q32, [0] * A, [ref], fk, fv, lens, DECODE.n_kv_heads)
    assert np.all(np.isfinite(out))
    err = attention.max_rel_error(out, want)
    assert err <= TOL, err


@pytest.mark.parametrize("prv_scale", [TOK, CHAN])
def test_variant_private_segments_and_mixed_launch(prv_scale):
    """A per-tensor shared pool with per-token or per-channel private pools (the segment kernel takes
    per-token ones; per-channel ones go through the pool kernel's split records)."""
    h = H()
    print(f"[variants] private pools k_scale={prv_scale}", flush=True)
    A = 5
    dp, ref = h.build_pair(DECODE, 0, layers=2)
    priv = []
    for a in range(A):
        n = 30 + 11 * a
        p = h.DevicePool(2, DECODE.n_kv_heads, DECODE.head_dim, n, [3, 2], k_scale=prv_scale, v_norm=a % 2)
        r = pool_image.PoolImage(2, DECODE.n_kv_heads, DECODE.head_dim, n, [3, 2], k_scale=prv_scale,
                                 corrected_norm=bool(a % 2))
        kk = [DECODE.pool_k(1 + a, l) for l in range(2)]
        vv = [DECODE.pool_v(1 + a, l) for l in range(2)]
        r.append(0, np.stack([x.f32[:, :n] for x in kk]), np.stack([x.f32[:, :n] for x in vv]))
        p.append(0, h.stack_layers([h._slice(x, 0, n) for x in kk]), h.stack_layers([h._slice(x, 0, n) for x in vv]))
        priv.append((p, r))
    q, q32 = h.make_queries(DECODE, 2, range(A))
    sk, sv, fk, fv = h.make_suffix(DECODE, range(A), 2)
    lens = [0, 4, 9, 24, 1]
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=h.DEV)
    prv = [p.pool for p, _ in priv]
    wsb = pk.agent_decode_attention([dp.pool] * A, q, out, 0, sk, sv, lens, private_pools=prv)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
    pk.agent_decode_attention([dp.pool] * A, q, out, 0, sk, sv, lens, workspace=ws, private_pools=prv)
    torch.cuda.synchronize()
    want = attention.decode_call(q32, [0] * A, lambda p, l, g: ref.decoded_layer(l, g), fk, fv, lens,
                                 DECODE.n_kv_heads, private=lambda a, l, g: priv[a][1].decoded_layer(l, g))
    err = attention.max_rel_error(out.cpu().numpy().astype(np.float64), want)
    assert err <= TOL, err


@pytest.mark.parametrize("k_scale", [TOK, CHAN])
def test_variant_shards(k_scale):
    """kv-head shards of per-token / per-channel pools carry those heads' K scales: images equal the
    oracle's shard, and decoding a shard reproduces the whole pool's outputs for its heads."""
    h = H()
    print(f"[variants] shards k_scale={k_scale}", flush=True)
    w = DECODE.replace(n_kv_heads=4, n_q_heads=16)
    dp, ref = h.build_pair(w, 0, layers=2, k_scale=k_scale, v_norm=1)
    q, _ = h.make_queries(w, 0, range(3))
    whole = h.run_decode([dp.pool] * 3, q)
    sh_ref = ref.shard(1, 2)
    sd = h.DevicePool.empty_for(pk.make_config(2, 2, w.head_dim, w.pool_tokens, w.v_bits(0)[:2], k_scale=k_scale,
                                               v_norm=1))
    sd.pool = pk.pool_shard(dp.pool, 1, 2, sd.buf.data_ptr(), sd.buf.numel())
    mism = h.compare_image(sd, sh_ref)
    assert all(x == 0 for x in mism.values()), mism
    G = w.n_q_heads // w.n_kv_heads
    part = h.run_decode([sd.pool] * 3, q[:, :, G:3 * G].contiguous())
    assert np.array_equal(part, whole[:, :, G:3 * G])

"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Pool images must match the oracle bit for bit on every defined byte (K codes,
V norms, K scales, per-head max norm, packed V code groups).  Decode outputs
must match the fp64 oracle within 1e-3 max relative error per output vector,
||o - o_ref||_inf / max(||o_ref||_inf, 1e-6), with fp32 accumulation on the GPU.
Sizes span several 32-token tiles, ragged tails, mid-group appends, mixed
bit widths, shared and distinct pools, empty and full suffixes.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention, pool_image
from quantized_shared_kv_amd import polykv as pk

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()
    yield


def H():
    import gpu_helpers

    return gpu_helpers


# ---------------------------------------------------------------- quantise
QUANT_CASES = {
    "tiny_fp32_d64": (wl.TINY, None, None),
    "gqa_bf16_d128_ragged": (wl.LLAMA3_8B.replace(n_layers=3, pool_tokens=300, v_bits_mode="mixed"), 3, None),
    "mha_bf16_d64_ragged": (wl.SMOLLM2.replace(n_layers=2, n_q_heads=4, n_kv_heads=4, pool_tokens=77), 2, None),
    "appends_mid_group": (wl.LLAMA3_8B.replace(n_layers=2, pool_tokens=157, v_bits_mode="mixed"), 2, [37, 20, 1, 99]),
    "appends_d64_fp32": (wl.TINY.replace(n_layers=3, n_kv_heads=2, n_q_heads=2, pool_tokens=90, v_bits_mode="mixed"),
                         3, [5, 3, 82]),
}


@pytest.mark.parametrize("case", sorted(QUANT_CASES))
def test_pool_image_bit_exact(case):
    w, layers, chunks = QUANT_CASES[case]
    print(f"[quant] {case}", flush=True)
    dp, ref = H().build_pair(w, 0, layers=layers, chunks=chunks)
    mism = H().compare_image(dp, ref)
    assert all(v == 0 for v in mism.values()), mism
    assert list(dp.pool.n_tokens[:ref.lay.n_layers]) == ref.n_tokens.tolist()


def test_pool_image_zero_inputs_and_single_token():
    h = H()
    print("[quant] zero inputs", flush=True)
    L, Hkv, d = 2, 2, 128
    dp = h.DevicePool(L, Hkv, d, 64, [3, 2])
    ref = pool_image.PoolImage(L, Hkv, d, 64, [3, 2])
    rng = np.random.default_rng(21)
    k = rng.standard_normal((L, Hkv, 9, d)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, 9, d)).astype(np.float32)
    k[1] = 0.0                  # layer 1: amax = 0 -> scale 0, codes 0
    v[0, 1, 3] = 0.0            # a zero V vector -> norm 0, codes 0
    v[1, 0, ::2] = 0.0
    for kk, vv in ((k[:, :, :1], v[:, :, :1]), (k[:, :, 1:], v[:, :, 1:])):  # a single-token append first
        ref.append(0, kk, vv)
        dp.append(0, torch.from_numpy(np.ascontiguousarray(kk)).to(h.DEV), torch.from_numpy(np.ascontiguousarray(vv)).to(h.DEV))
    mism = h.compare_image(dp, ref)
    assert all(x == 0 for x in mism.values()), mism


def test_pool_bytes_do_not_depend_on_agents():
    # the same pool bytes serve 1, 3, 10 and 15 agents: decode never writes the pool
    h = H()
    w = wl.LLAMA3_8B.replace(n_layers=1, pool_tokens=96, n_agents=15)
    dp, _ = h.build_pair(w, 0)
    before = dp.host_bytes().copy()
    for n in (1, 3, 10, 15):
        q, _ = h.make_queries(w, 0, range(n))
        h.run_decode([dp.pool] * n, q)
        assert np.array_equal(dp.host_bytes(), before)
    assert dp.buf.numel() == pk.pool_bytes(dp.cfg)


# ---------------------------------------------------------------- decode
def _decode_case(w, layers, sfx_lens, kernel, splits=0, layer_begin=0, distinct=False):
    h = H()
    A = len(sfx_lens)
    n_pools = A if distinct else 1
    pairs = [h.build_pair(w, p, layers=layers) for p in range(n_pools)]
    lc = layers - layer_begin
    q, q32 = h.make_queries(w, 0, range(A))
    q = q[:, layer_begin:].contiguous()
    q32 = q32[:, layer_begin:]
    sfx = None
    ksf = vsf = None
    if max(sfx_lens) > 0:
        kd, vd, ksf0, vsf0 = h.make_suffix(w, range(A), layers)
        sfx = (kd[:, layer_begin:].contiguous(), vd[:, layer_begin:].contiguous())
        ksf = lambda a, l: ksf0(a, l + layer_begin)  # noqa: E731
        vsf = lambda a, l: vsf0(a, l + layer_begin)  # noqa: E731
    pools = [pairs[a if distinct else 0][0].pool for a in range(A)]
    out = h.run_decode(pools, q, sfx, sfx_lens, layer_begin=layer_begin, kernel=kernel, splits=splits)
    ref = h.oracle_decode(q32, [a if distinct else 0 for a in range(A)], [p[1] for p in pairs], ksf, vsf,
                          sfx_lens, w.n_kv_heads, layer_begin=layer_begin)
    assert out.shape == ref.shape and np.all(np.isfinite(out))
    return attention.max_rel_error(out, ref), out


KERNELS = [pk.KERNEL_VALU, pk.KERNEL_MFMA]

DECODE_CASES = {
    "tiny_fp32": (wl.TINY, 1, [0, 0, 0, 0], False),
    "gqa_d128_shared_sfx": (wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=300,
                                                 sfx_tokens=64), 2, [0, 1, 7, 33, 64], False),
    "mha_d64_grow": (wl.SMOLLM2.replace(n_layers=2, n_q_heads=4, n_kv_heads=4, pool_tokens=77, sfx_tokens=16), 2,
                     [1, 9, 16], False),
    "distinct_mixed_bits": (wl.QWEN3_32B_MIXED.replace(n_layers=3, n_q_heads=8, n_kv_heads=2, pool_tokens=100,
                                                       sfx_tokens=16, n_agents=3, n_pools=3), 3, [16, 16, 16], True),
    "g8_rows_over_32": (wl.QWEN3_32B_MIXED.replace(n_layers=1, n_q_heads=16, n_kv_heads=2, pool_tokens=64,
                                                   sfx_tokens=8, n_agents=5, n_pools=1, v_bits_mode="uniform3"),
                        1, [8, 0, 3, 8, 1], False),
    "g16_two_suffix_passes": (wl.LLAMA3_8B.replace(n_layers=1, n_q_heads=32, n_kv_heads=2, pool_tokens=130,
                                                   sfx_tokens=70), 1, [70, 65], False),
    "tiny_fp32_with_suffix": (wl.TINY.replace(sfx_tokens=40, sfx_mode="fixed"), 1, [40, 0, 7, 33], False),
}


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", sorted(DECODE_CASES))
def test_decode_matches_oracle(case, kernel):
    w, layers, lens, distinct = DECODE_CASES[case]
    print(f"[decode] {case} kernel={kernel}", flush=True)
    err, _ = _decode_case(w, layers, lens, kernel, distinct=distinct)
    assert err <= TOL, err


# suffixes past one 256-token chunk of the suffix kernel, every group size it specialises
LONG_SUFFIX_CASES = {
    "g4_d128_chunk_edges": (wl.LLAMA3_8B.replace(n_layers=1, n_kv_heads=2, n_q_heads=8, pool_tokens=64,
                                                 sfx_tokens=600), [600, 256, 257, 513, 1, 0]),
    "g1_d128": (wl.LLAMA3_8B.replace(n_layers=1, n_kv_heads=2, n_q_heads=2, pool_tokens=40, sfx_tokens=300),
                [300, 17, 256]),
    "g2_d128": (wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=4, pool_tokens=40, sfx_tokens=290),
                [290, 129]),
    "g3_d64": (wl.SMOLLM2.replace(n_layers=1, n_kv_heads=2, n_q_heads=6, pool_tokens=50, sfx_tokens=300),
               [300, 255, 0]),
    "g6_d128": (wl.LLAMA3_8B.replace(n_layers=1, n_kv_heads=2, n_q_heads=12, pool_tokens=40, sfx_tokens=270),
                [270, 31]),
    "g8_d64": (wl.SMOLLM2.replace(n_layers=1, n_kv_heads=1, n_q_heads=8, pool_tokens=40, sfx_tokens=520),
               [520, 512]),
}


@pytest.mark.parametrize("case", sorted(LONG_SUFFIX_CASES))
def test_decode_long_suffix(case):
    w, lens = LONG_SUFFIX_CASES[case]
    print(f"[decode] long suffix {case}", flush=True)
    err, _ = _decode_case(w, w.n_layers, lens, pk.KERNEL_MFMA)
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("splits", [1, 3, 50])
def test_decode_split_plans_agree(splits, kernel):
    print(f"[decode] splits={splits} kernel={kernel}", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=1, n_kv_heads=2, n_q_heads=8, pool_tokens=333, sfx_tokens=8)
    err, _ = _decode_case(w, 1, [8, 2, 0], kernel, splits=splits)
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", KERNELS)
def test_decode_layer_subrange_and_empty_pool(kernel):
    print(f"[decode] layer_begin / empty pool kernel={kernel}", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=3, n_kv_heads=2, n_q_heads=4, pool_tokens=70, sfx_tokens=8)
    err, _ = _decode_case(w, 3, [4, 8], kernel, layer_begin=1)
    assert err <= TOL, err
    # a pool without tokens: outputs are attention over the suffix alone
    h = H()
    dp = h.DevicePool(1, 2, 128, 32, [3])
    q, q32 = h.make_queries(w.replace(n_layers=1), 0, range(2))
    kd, vd, ksf, vsf = h.make_suffix(w.replace(n_layers=1), range(2), 1)
    out = h.run_decode([dp.pool] * 2, q, (kd, vd), [5, 1], kernel=kernel)
    for a, S in enumerate([5, 1]):
        for hh in range(4):
            ref = attention.attend(q32[a, 0, hh:hh + 1], ksf(a, 0)[hh // 2, :S], vsf(a, 0)[hh // 2, :S])
            assert attention.max_rel_error(out[a, 0, hh:hh + 1], ref) <= TOL


@pytest.mark.parametrize("kernel", KERNELS)
def test_decode_is_deterministic_and_batch_independent(kernel):
    print(f"[decode] determinism kernel={kernel}", flush=True)
    h = H()
    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=200, sfx_tokens=8)
    dp, _ = h.build_pair(w, 0)
    q, _ = h.make_queries(w, 0, range(4))
    kd, vd, _, _ = h.make_suffix(w, range(4), 2)
    a = h.run_decode([dp.pool] * 4, q, (kd, vd), [3, 8, 0, 5], kernel=kernel)
    b = h.run_decode([dp.pool] * 4, q, (kd, vd), [3, 8, 0, 5], kernel=kernel)
    assert np.array_equal(a, b)
    solo = h.run_decode([dp.pool], q[1:2].contiguous(), (kd[1:2].contiguous(), vd[1:2].contiguous()), [8],
                        kernel=kernel)
    assert np.max(np.abs(solo[0] - a[1])) <= 1e-6 * max(1.0, np.max(np.abs(a[1])))


@pytest.mark.parametrize("kernel", KERNELS)
def test_decode_interleaved_pools(kernel):
    # agents of two pools interleaved in the call: the launch regroups them by pool
    print(f"[decode] interleaved pools kernel={kernel}", flush=True)
    h = H()
    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=150, sfx_tokens=8, n_pools=2)
    pairs = [h.build_pair(w, p, layers=2) for p in range(2)]
    pool_of = [0, 1, 0, 1, 1, 0]
    A = len(pool_of)
    q, q32 = h.make_queries(w, 3, range(A))
    kd, vd, ksf, vsf = h.make_suffix(w, range(A), 2)
    lens = [8, 0, 3, 8, 1, 5]
    out = h.run_decode([pairs[p][0].pool for p in pool_of], q, (kd, vd), lens, kernel=kernel)
    ref = h.oracle_decode(q32, pool_of, [p[1] for p in pairs], ksf, vsf, lens, w.n_kv_heads)
    assert attention.max_rel_error(out, ref) <= TOL


def _ramp_pool(h, slope, T=300, Hkv=2, d=128, seed=5):
    """A pool whose keys grow (slope > 0) or shrink along the tokens in one direction u."""
    rng = np.random.default_rng(seed)
    u = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    ramp = np.arange(T, dtype=np.float64) / T
    base = ramp if slope > 0 else 1.0 - ramp
    k = (abs(slope) * base[None, :, None] * u[None, None, :]
         + 0.1 * rng.standard_normal((Hkv, T, d)))[None].astype(np.float32)
    v = rng.standard_normal((1, Hkv, T, d)).astype(np.float32)
    dp = h.DevicePool(1, Hkv, d, T, [3])
    ref = pool_image.PoolImage(1, Hkv, d, T, [3])
    ref.append(0, k, v)
    dp.append(0, torch.from_numpy(k).to(h.DEV), torch.from_numpy(v).to(h.DEV))
    return dp, ref, u


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("qdtype", ["bf16", "f32"])
@pytest.mark.parametrize("slope", [2.0, -2.0])
def test_decode_scores_far_from_first_tokens(kernel, qdtype, slope):
    # Scores that rise by ~65 log2 units along the pool (slope > 0: far above any
    # reference taken from the first tokens) or fall from them (slope < 0); rows of
    # one kv head mix agents whose queries point along +u, -u and half of +u.
    h = H()
    print(f"[decode] ramp slope={slope} q={qdtype} kernel={kernel}", flush=True)
    dp, ref, u = _ramp_pool(h, slope)
    G, A = 4, 3
    scale = np.array([2.0, -2.0, 1.0])
    q32 = (scale[:, None, None, None] * np.broadcast_to(u, (A, 1, 2 * G, 128))).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(q32)).to(h.DEV)
    if qdtype == "bf16":
        q = q.to(torch.bfloat16)  # +-2, +-1: exact in bf16
    for splits in (0, 3):
        out = h.run_decode([dp.pool] * A, q, kernel=kernel, splits=splits)
        exp = h.oracle_decode(q32.astype(np.float64), [0] * A, [ref], None, None, [0] * A, 2)
        err = attention.max_rel_error(out, exp)
        assert err <= TOL, (splits, err)


def test_zero_agents_is_a_no_op():
    h = H()
    dp = h.DevicePool(1, 1, 64, 32, [3])
    q = torch.zeros((0, 1, 1, 64), dtype=torch.bfloat16, device=h.DEV)
    out = torch.zeros((0, 1, 1, 64), dtype=torch.float32, device=h.DEV)
    assert pk.agent_decode_attention([], q, out) == 0


def test_last_bit_conventions_on_device():
    """The hand-worked inputs of the oracle's last-bit pins, encoded by the device: K quotient
    by division rounded half to even (90.5 -> 90), ascending FWHT stage order (a coordinate
    that is +0 only in that order -> the lower code), V normalised by the rounded reciprocal
    (a coordinate landing exactly on a threshold -> the lower code).  Expected values are the
    literals worked out by hand in the oracle's tests."""
    from oracle import codec

    h = H()
    print("[quant] last-bit conventions", flush=True)
    f = lambda b: np.frombuffer(int(b).to_bytes(4, "little"), dtype=np.float32)[0]  # noqa: E731
    d = 128
    k = np.zeros((1, 1, 3, d), np.float32)
    k[0, 0, 0, 0], k[0, 0, 1, 0], k[0, 0, 2, 0] = f(0x40B7C408), f(0x4082F381), -f(0x4082F381)
    v = np.zeros((1, 1, 3, d), np.float32)
    v[0, 0, 0, :3] = [1.0, 2.0 ** -24, -1.0]
    v[0, 0, 1, :2] = [f(0x3F553488), f(0x3D2F22B9)]
    dp = h.DevicePool(1, 1, d, 32, [3])
    dp.append(0, torch.from_numpy(k).to(h.DEV), torch.from_numpy(v).to(h.DEV))
    buf = dp.host_bytes()
    lay = pool_image.layout(1, 1, d, 32, [3])
    kq = buf[lay.kq:lay.kq + 32 * d].view(np.int8).reshape(32, d)
    assert list(kq[:3, 0]) == [127, 90, -90] and not kq[:3, 1:].any()
    assert list(buf[lay.ks:lay.ks + 12].view(np.uint32)) == [0x3D393675] * 3
    assert list(buf[lay.vn:lay.vn + 12].view(np.uint32)) == [0x3FB504F3, 0x3F557C6A, 0]
    codes = codec.unpack_codes(buf[lay.vc[0]:lay.vc[1]].reshape(4, d * 3), d, 3)
    assert np.array_equal(codes[0], np.tile(np.array([3, 3, 6, 6], np.uint8), 32))
    assert np.all(codes[1] == 5) and np.all(codes[2] == 0)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("tokens,splits", [(2080, 65), (2600, 82)])
def test_merge_of_more_than_64_records(tokens, splits, kernel):
    """k_merge spreads a row's split records over the 64 lanes and sums them in groups: rows with
    more than 64 records (65 splits of a 2080-token pool, 82 of a 2600-token one: one 32-token
    tile each; then plus the 22 splits of a 700-token private pool shared by all three agents,
    12 rows) take several lane rounds, the private pool's records starting past the boundary."""
    h = H()
    print(f"[decode] merge of >64 records tokens={tokens} splits={splits} kernel={kernel}", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=1, n_kv_heads=1, n_q_heads=4, pool_tokens=tokens, sfx_tokens=24, n_agents=3)
    A = 3
    dp, ref = h.build_pair(w, 0, layers=1)
    n = 700
    pp = h.DevicePool(1, 1, w.head_dim, n, [3])
    pr = pool_image.PoolImage(1, 1, w.head_dim, n, [3])
    kt, vt = w.pool_k(7, 0), w.pool_v(7, 0)
    pr.append(0, kt.f32[None, :, :n], vt.f32[None, :, :n])
    pp.append(0, h.stack_layers([h._slice(kt, 0, n)]), h.stack_layers([h._slice(vt, 0, n)]))
    q, q32 = h.make_queries(w, 2, range(A))
    sk, sv, fk, fv = h.make_suffix(w, range(A), 1)
    lens = [24, 0, 9]
    for prv in (None, [pp.pool] * A):
        out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=h.DEV)
        wsb = pk.agent_decode_attention([dp.pool] * A, q, out, 0, sk, sv, lens, kernel=kernel, splits=splits,
                                        private_pools=prv)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
        pk.agent_decode_attention([dp.pool] * A, q, out, 0, sk, sv, lens, workspace=ws, kernel=kernel, splits=splits,
                                  private_pools=prv)
        torch.cuda.synchronize()
        want = attention.decode_call(
            q32, [0] * A, lambda p, l, g: ref.decoded_layer(l, g), fk, fv, lens, 1,
            private=(lambda a, l, g: pr.decoded_layer(l, g)) if prv is not None else None)
        err = attention.max_rel_error(out.cpu().numpy().astype(np.float64), want)
        assert err <= TOL, (prv is not None, err)


def test_single_layer_calls_match_the_all_layer_call():
    """The same decode step as one all-layer call (one split per (layer, kv head), the pool kernel
    finishing the rows after the separate native-window kernel) and as single-layer calls (token
    splits, the window's workgroups inside the pool launch, k_merge): outputs agree to summation
    order, and both match the oracle."""
    print("[decode] single-layer calls vs all-layer call", flush=True)
    h = H()
    w = wl.LLAMA3_8B.replace(n_layers=2, pool_tokens=700, sfx_tokens=40, n_agents=15)
    A, L, Hq = w.n_agents, w.n_layers, w.n_q_heads
    dp, ref = h.build_pair(w, 0)
    q, q32 = h.make_queries(w, 0, range(A))
    kd, vd, ksf, vsf = h.make_suffix(w, range(A), L)
    lens = [(7 * a) % 41 for a in range(A)]
    whole = h.run_decode([dp.pool] * A, q, (kd, vd), lens, splits=1)  # the fused form
    per = np.concatenate([h.run_decode([dp.pool] * A, q[:, l:l + 1].contiguous(),
                                       (kd[:, l:l + 1].contiguous(), vd[:, l:l + 1].contiguous()), lens, layer_begin=l)
                          for l in range(L)], axis=1)
    assert attention.max_rel_error(per, whole) <= 1e-5
    want = h.oracle_decode(q32, [0] * A, [ref], ksf, vsf, lens, w.n_kv_heads)
    assert attention.max_rel_error(whole, want) <= TOL
    assert attention.max_rel_error(per, want) <= TOL

"""GPU parity at the limits of one call's plan and of the pool shape.

A decode call holds at most 128 agents and 16 pools per launch; larger calls
are split into several launches (a pool's agents may span launches).  These
cases go past both limits, and a pool uses the maximum of 128 layers with a
call over a layer sub-range.  Outputs against the fp64 oracle within 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention
from quantized_shared_kv_amd import polykv as pk

from gpu_helpers import build_pair, make_queries, make_suffix, oracle_decode, run_decode

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()


def test_more_than_16_pools_in_one_call():
    print("[limits] 20 pools", flush=True)
    w = wl.SMOLLM2.replace(n_layers=2, n_q_heads=4, n_kv_heads=2, pool_tokens=45, n_agents=20, n_pools=20,
                           sfx_tokens=6)
    pairs = [build_pair(w, p) for p in range(20)]
    q, q32 = make_queries(w, 0, range(20))
    sk, sv, fk, fv = make_suffix(w, range(20), w.n_layers)
    lens = [a % 7 for a in range(20)]
    out = run_decode([d.pool for d, _ in pairs], q, (sk, sv), lens)
    want = oracle_decode(q32, list(range(20)), [r for _, r in pairs], fk, fv, lens, w.n_kv_heads)
    assert attention.max_rel_error(out, want) <= TOL


@pytest.mark.parametrize("kernel", [pk.KERNEL_DEFAULT, pk.KERNEL_VALU])
def test_more_than_128_agents_in_one_call(kernel):
    print(f"[limits] 140 agents kernel {kernel}", flush=True)
    w = wl.SMOLLM2.replace(n_layers=1, n_q_heads=2, n_kv_heads=2, pool_tokens=70, n_agents=140, n_pools=1,
                           sfx_tokens=4)
    d0, r0 = build_pair(w, 0)
    d1, r1 = build_pair(w.replace(pool_tokens=33), 0)
    pools = [d0.pool if a % 3 else d1.pool for a in range(140)]  # two shared pools, interleaved agents
    q, q32 = make_queries(w, 1, range(140))
    sk, sv, fk, fv = make_suffix(w, range(140), 1)
    lens = [a % 5 for a in range(140)]
    out = run_decode(pools, q, (sk, sv), lens, kernel=kernel)
    want = oracle_decode(q32, [0 if a % 3 else 1 for a in range(140)], [r0, r1], fk, fv, lens, w.n_kv_heads)
    assert attention.max_rel_error(out, want) <= TOL


def test_128_layers_and_a_layer_subrange():
    print("[limits] 128 layers", flush=True)
    w = wl.TINY.replace(n_layers=128, pool_tokens=40, n_agents=2, v_bits_mode="mixed")
    dp, ref = build_pair(w, 0)
    assert list(dp.pool.n_tokens[:128]) == [40] * 128
    for lb, lc in ((0, 128), (77, 51)):
        qs = [w.queries(0, a) for a in range(2)]
        q = torch.stack([torch.from_numpy(np.ascontiguousarray(t.f32[lb:lb + lc])) for t in qs]).cuda()
        q32 = np.stack([t.f32[lb:lb + lc] for t in qs])
        out = run_decode([dp.pool] * 2, q, layer_begin=lb)
        want = attention.decode_call(q32, [0, 0], lambda p, l, g: ref.decoded_layer(lb + l, g), None, None, [0, 0],
                                     w.n_kv_heads)
        assert attention.max_rel_error(out, want) <= TOL, (lb, lc)


@pytest.mark.parametrize("kernel", [pk.KERNEL_MFMA, pk.KERNEL_VALU])
@pytest.mark.parametrize("scale", [0.05, 0.37])
def test_explicit_softmax_scale(kernel, scale):
    """A caller-given softmax scale instead of 1/sqrt(d) (0.37 is ~4x the default at d 128:
    a sharper softmax, so scores leave the first step's reference faster)."""
    print(f"[limits] softmax scale {scale} kernel {kernel}", flush=True)
    from oracle import attention as att

    from gpu_helpers import DEV

    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=150, n_agents=3, sfx_tokens=11)
    dp, ref = build_pair(w, 0)
    q, q32 = make_queries(w, 0, range(3))
    sk, sv, fk, fv = make_suffix(w, range(3), 2)
    lens = [0, 4, 11]
    out = torch.empty((3, 2, 8, 128), dtype=torch.float32, device=DEV)
    wsb = pk.agent_decode_attention([dp.pool] * 3, q, out, 0, sk, sv, lens, softmax_scale=scale, kernel=kernel)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    pk.agent_decode_attention([dp.pool] * 3, q, out, 0, sk, sv, lens, workspace=ws, softmax_scale=scale, kernel=kernel)
    torch.cuda.synchronize()
    want = att.decode_call(q32, [0] * 3, lambda p, l, g: ref.decoded_layer(l, g), fk, fv, lens, 2, sigma=scale)
    assert att.max_rel_error(out.cpu().numpy().astype(np.float64), want) <= TOL


def test_stream_read_folds_every_word():
    """The streaming-read kernel (the measurements' HBM read ceiling) reads every word: the XOR of its
    per-wavefront results equals the XOR of the buffer's 32-bit words, for sizes that are and are not
    multiples of the grid's stride."""
    import numpy as np
    import torch

    from quantized_shared_kv_amd import polykv as pk

    rng = np.random.default_rng(4)
    for n in (4, 4 * 1000003, 1 << 22):
        host = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
        src = torch.from_numpy(host.view(np.int32)).cuda()
        sink = torch.zeros(pk.stream_read_sink_words(), dtype=torch.int32, device="cuda")
        pk.stream_read(src, sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), n

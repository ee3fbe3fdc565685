"""GPU parity of decode with per-agent private compressed segments.

An agent's recent tokens stay native (bf16) in its window; when the window
overflows, its oldest tokens are quantized once into the agent's own pool with
the same write path as the shared pool (CoMixKV news article, incremental
quantization: recent states native, older ones compressed, never rewritten).
The agent then attends to shared pool + private segment + window.  Compared
with the oracle's fp64 attention over the concatenated decoded tokens.
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
KERNELS = [pk.KERNEL_VALU, pk.KERNEL_MFMA]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()
    yield


def H():
    import gpu_helpers

    return gpu_helpers


def _private_pools(w, agents, layers, rolled, blocks):
    """Per agent: (DevicePool, PoolImage) holding the first rolled[a] tokens of its own window,
    appended in `blocks` roll-overs; None where rolled[a] is None."""
    h = H()
    out = []
    for a in agents:
        n = rolled[a]
        if n is None:
            out.append(None)
            continue
        bits = [3] * layers
        cap = max(n, 1)
        dp = h.DevicePool(layers, w.n_kv_heads, w.head_dim, cap, bits)
        ref = pool_image.PoolImage(layers, w.n_kv_heads, w.head_dim, cap, bits)
        ks = [w.sfx_k(a, l) for l in range(layers)]
        vs = [w.sfx_v(a, l) for l in range(layers)]
        edges = np.linspace(0, n, blocks + 1).astype(int)
        for t0, t1 in zip(edges[:-1], edges[1:]):
            if t1 == t0:
                continue
            ref.append(0, np.stack([x.f32[:, t0:t1] for x in ks]), np.stack([x.f32[:, t0:t1] for x in vs]))
            dp.append(0, h.stack_layers([h._slice(x, t0, t1 - t0) for x in ks]),
                      h.stack_layers([h._slice(x, t0, t1 - t0) for x in vs]))
        out.append((dp, ref))
    return out


# (workload, layers, rolled-over tokens per agent (None: no private pool), window lengths, roll-over blocks)
CASES = {
    "g4_ragged_and_empty": (wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=300,
                                                 sfx_tokens=120), 2, [70, None, 33, 0], [40, 17, 1, 0], 1),
    "g4_two_rollovers": (wl.LLAMA3_8B.replace(n_layers=1, n_kv_heads=2, n_q_heads=8, pool_tokens=96,
                                              sfx_tokens=160), 1, [128, 64, 96], [32, 96, 64], 2),
    "mha_d64": (wl.SMOLLM2.replace(n_layers=2, n_q_heads=4, n_kv_heads=4, pool_tokens=77, sfx_tokens=64), 2,
                [40, 24, None], [24, 40, 64], 1),
    "g8_all_private": (wl.QWEN3_32B_MIXED.replace(n_layers=1, n_q_heads=16, n_kv_heads=2, pool_tokens=64,
                                                  sfx_tokens=64, n_agents=5, n_pools=1, v_bits_mode="uniform3"),
                       1, [8, 16, 24, 32, 40], [8, 8, 8, 8, 8], 1),
}


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_with_private_segments(case, kernel):
    h = H()
    w, layers, rolled, window, blocks = CASES[case]
    A = len(rolled)
    print(f"[private] {case} kernel={kernel}", flush=True)
    dp, ref = h.build_pair(w, 0, layers=layers)
    priv = _private_pools(w, range(A), layers, rolled, blocks)
    q, q32 = h.make_queries(w, 0, range(A))
    # each agent's window is its suffix tokens after the rolled-over ones
    S = w.sfx_tokens
    kd, vd, ksf, vsf = h.make_suffix(w, range(A), layers)
    off = [r or 0 for r in rolled]
    cap = max(window) if max(window) > 0 else 1
    wk = torch.zeros((A, layers, w.n_kv_heads, cap, w.head_dim), dtype=kd.dtype, device=kd.device)
    wv = torch.zeros_like(wk)
    for a in range(A):
        assert off[a] + window[a] <= S
        wk[a, :, :, :window[a]] = kd[a, :, :, off[a]:off[a] + window[a]]
        wv[a, :, :, :window[a]] = vd[a, :, :, off[a]:off[a] + window[a]]
    out = torch.full((A, layers, w.n_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device=h.DEV)
    pools = [dp.pool] * A
    prv = [p[0].pool if p is not None else None for p in priv]
    wsb = pk.agent_decode_attention(pools, q, out, 0, wk, wv, window, kernel=kernel, private_pools=prv)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
    pk.agent_decode_attention(pools, q, out, 0, wk, wv, window, workspace=ws, kernel=kernel, private_pools=prv)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    r = attention.decode_call(
        q32, [0] * A, lambda p, l, g: ref.decoded_layer(l, g),
        lambda a, l: ksf(a, l)[:, off[a]:], lambda a, l: vsf(a, l)[:, off[a]:], window, w.n_kv_heads,
        private=lambda a, l, g: priv[a][1].decoded_layer(l, g) if priv[a] is not None else None)
    assert np.all(np.isfinite(o))
    err = attention.max_rel_error(o, r)
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", KERNELS)
def test_private_segment_equals_second_append_block(kernel):
    """Shared pool of blocks 1 + 2 (two appends) vs shared pool of block 1 plus each agent's
    private pool holding block 2: the decoded tokens are identical, so the outputs agree."""
    h = H()
    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=200, sfx_tokens=8)
    A, n1 = 3, 136
    both, _ = h.build_pair(w, 0, layers=2, chunks=[n1, w.pool_tokens - n1])
    first = h.DevicePool(2, w.n_kv_heads, w.head_dim, n1, w.v_bits(0)[:2])
    second = h.DevicePool(2, w.n_kv_heads, w.head_dim, w.pool_tokens - n1, w.v_bits(0)[:2])
    ks = [w.pool_k(0, l) for l in range(2)]
    vs = [w.pool_v(0, l) for l in range(2)]
    first.append(0, h.stack_layers([h._slice(x, 0, n1) for x in ks]), h.stack_layers([h._slice(x, 0, n1) for x in vs]))
    second.append(0, h.stack_layers([h._slice(x, n1, w.pool_tokens - n1) for x in ks]),
                  h.stack_layers([h._slice(x, n1, w.pool_tokens - n1) for x in vs]))
    q, _ = h.make_queries(w, 0, range(A))
    kd, vd, _, _ = h.make_suffix(w, range(A), 2)
    lens = [8, 3, 0]
    o_both = h.run_decode([both.pool] * A, q, (kd, vd), lens, kernel=kernel)
    out = torch.full_like(q, float("nan"), dtype=torch.float32)
    wsb = pk.agent_decode_attention([first.pool] * A, q, out, 0, kd, vd, lens, kernel=kernel,
                                    private_pools=[second.pool] * A)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
    pk.agent_decode_attention([first.pool] * A, q, out, 0, kd, vd, lens, workspace=ws, kernel=kernel,
                              private_pools=[second.pool] * A)
    torch.cuda.synchronize()
    o_split = out.cpu().numpy().astype(np.float64)
    assert attention.max_rel_error(o_split, o_both) <= 1e-5

"""Parity at the full sizes of the workloads, in the launch configuration the benchmark times.

At full size the oracle cannot check every output, so each case:

* builds every pool of the workload on the device at its full size and bit widths;
  the sampled (pool, layer) slices come from the seeded workload generators, the
  rest (only where generating them on the host would take minutes) from a seeded
  device-side draw of the same shape and value recipe (N(0, 1) times LogNormal(0, 0.5)
  channel scales for the LogNormal workloads);
* compares the pool image of every sampled layer byte for byte with the oracle's
  encoding of that layer (the codec is per layer, so one layer is checked alone);
* runs all-layer decode calls for all agents with the default kernel and plan
  (what ``bench.py`` times) at the workload's decode steps -- every step of the
  64-step SmolLM2 job (its suffix grows 1 .. 64), steps {0, middle, last} of the
  others -- and compares sampled output rows of each with the oracle's fp64
  attention over its own decoded pool plus the agent's bf16 suffix (1e-3);
* checks properties of every output row: finite, and within the range of the
  value vectors it averages (attention is a convex combination).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention, pool_image
from quantized_shared_kv_amd import polykv as pk

from gpu_helpers import DEV, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()
    yield

TOL = 1e-3

# workload, decode steps (suffix length is min(step + 1, S) for growing suffixes), every layer from the host
FULL_CASES = {
    "smollm2_L24_H32_d64_T1851_A3": (wl.SMOLLM2, list(range(64)), True),
    "llama3_8b_L32_d128_T4096_A15": (wl.LLAMA3_8B, [0, 63, 127], True),
    "llama3_8b_long_T7194_S256_A15": (wl.LLAMA3_8B_LONG, [0, 15, 31], False),
    "qwen3_32b_comix_L64_T8064_A8_pools8": (wl.QWEN3_32B_MIXED, [0, 7, 15], False),
}


def _bf16_dev(t) -> torch.Tensor:
    return to_device(t).to(torch.bfloat16) if t.dtype != "bf16" else to_device(t)


def _sfx_len(w, step):
    return min(step + 1, w.sfx_tokens) if w.sfx_mode == "grow" else w.sfx_tokens


def _layer_bytes(buf: np.ndarray, lay, l: int, T: int):
    """The defined bytes of layer l of a device pool image."""
    H, d, tc = lay.n_kv_heads, lay.head_dim, lay.tc
    kq = buf[lay.kq + l * H * tc * d:lay.kq + (l + 1) * H * tc * d].view(np.int8).reshape(H, tc, d)[:, :T]
    vn = buf[lay.vn + l * H * tc * 4:lay.vn + (l + 1) * H * tc * 4].view(np.uint32).reshape(H, tc)[:, :T]
    ks = buf[lay.ks + l * tc * 4:lay.ks + (l + 1) * tc * 4].view(np.uint32)[:T]
    vmax = buf[lay.vmax + l * H * 4:lay.vmax + (l + 1) * H * 4].view(np.uint32)
    b = lay.bits[l]
    vc = buf[lay.vc[l]:lay.vc[l + 1]].reshape(H, tc // 8, d * b)[:, :(T + 7) // 8]
    return kq, vn, ks, vmax, vc


@pytest.mark.parametrize("case", sorted(FULL_CASES))
def test_full_size_pool_and_decode(case):
    w, steps, host_all = FULL_CASES[case]
    print(f"[fullsize] {case}", flush=True)
    A, L, Hkv, Hq, d, T, S = w.n_agents, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.pool_tokens, w.sfx_tokens
    G = Hq // Hkv
    n_pools = w.n_pools
    pool_of = [a % n_pools for a in range(A)]
    s_agents = sorted({0, A // 2, A - 1})
    s_layers = sorted({0, L // 2, L - 1})
    s_pools = sorted({pool_of[a] for a in s_agents})
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1234)

    def device_draw(shape):
        """A seeded device draw with the workload's value recipe (channel scales on the last axis)."""
        x = torch.randn(shape, generator=gen, device=DEV)
        if w.dist == "lognormal_channels":
            x = x * torch.exp(0.5 * torch.randn((Hkv,) + (1,) * (len(shape) - 2) + (d,), generator=gen, device=DEV))
        return x.to(torch.bfloat16)

    def host_slice(kind, idx, l):
        return host_all or (l in s_layers and idx in (s_pools if kind == "pool" else s_agents))

    # ---- pools, appended layer by layer
    pools, bufs, refs = [], [], {}
    for p in range(n_pools):
        bits = w.v_bits(p)
        cfg = pk.make_config(L, Hkv, d, T, bits)
        nbytes = pk.pool_bytes(cfg)
        buf = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        pool = pk.pool_build(cfg, buf.data_ptr(), nbytes)
        for l in range(L):
            if host_slice("pool", p, l):
                kt, vt = w.pool_k(p, l), w.pool_v(p, l)
                kd, vd = _bf16_dev(kt)[None].contiguous(), _bf16_dev(vt)[None].contiguous()
                if p in s_pools and l in s_layers:
                    ref = pool_image.PoolImage(1, Hkv, d, T, [bits[l]])
                    ref.append(0, kt.f32[None], vt.f32[None])
                    refs[(p, l)] = ref
            else:
                kd = device_draw((Hkv, T, d))[None].contiguous()
                vd = device_draw((Hkv, T, d))[None].contiguous()
            pk.pool_quantize_append(pool, l, kd, vd)
        pools.append(pool)
        bufs.append(buf)
    torch.cuda.synchronize()

    # ---- the sampled layers' images, byte for byte
    for (p, l), ref in refs.items():
        lay = pool_image.layout(L, Hkv, d, T, w.v_bits(p))
        kq, vn, ks, vmax, vc = _layer_bytes(bufs[p].cpu().numpy(), lay, l, T)
        assert np.array_equal(kq, ref.kq[0, :, :T]), (p, l, "kq")
        assert np.array_equal(vn, ref.vn[0, :, :T].view(np.uint32)), (p, l, "vn")
        assert np.array_equal(ks, ref.ks[0, :T].view(np.uint32)), (p, l, "ks")
        assert np.array_equal(vmax, ref.vmax[0].view(np.uint32)), (p, l, "vmax")
        assert np.array_equal(vc, ref.packed_codes(0)[:, :(T + 7) // 8]), (p, l, "vc")

    # ---- suffixes and queries
    sfx_k = torch.empty((A, L, Hkv, S, d), dtype=torch.bfloat16, device=DEV)
    sfx_v = torch.empty_like(sfx_k)
    sfx_host = {}
    for a in range(A):
        for l in range(L):
            if host_slice("agent", a, l):
                kt, vt = w.sfx_k(a, l), w.sfx_v(a, l)
                sfx_k[a, l].copy_(_bf16_dev(kt))
                sfx_v[a, l].copy_(_bf16_dev(vt))
                if a in s_agents and l in s_layers:
                    sfx_host[(a, l)] = (kt.f32, vt.f32)
            else:
                sfx_k[a, l].copy_(device_draw((Hkv, S, d)))
                sfx_v[a, l].copy_(device_draw((Hkv, S, d)))
    agent_pools = [pools[pool_of[a]] for a in range(A)]
    decoded = {}
    worst = 0.0
    for step in steps:
        worst = max(worst, _check_step(case, w, step, agent_pools, bufs, refs, sfx_k, sfx_v, sfx_host, pool_of,
                                       s_agents, s_layers, decoded))
    print(f"[fullsize] {case}: {len(steps)} decode steps, worst sampled error {worst:.2e}", flush=True)


def _check_step(case, w, step, agent_pools, bufs, refs, sfx_k, sfx_v, sfx_host, pool_of, s_agents, s_layers,
                decoded):
    """One all-layer decode call at `step` (default kernel and plan) and its checks; returns the
    worst sampled error."""
    A, L, Hkv, Hq, d, T = w.n_agents, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.pool_tokens
    G = Hq // Hkv
    n_pools = w.n_pools
    s_len = _sfx_len(w, step)
    qs = [w.queries(step, a) for a in range(A)]
    q = torch.stack([to_device(t) for t in qs]).contiguous()
    out = torch.full((A, L, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    lens = [s_len] * A
    ws_bytes = pk.agent_decode_attention(agent_pools, q, out, 0, sfx_k, sfx_v, lens)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    pk.agent_decode_attention(agent_pools, q, out, 0, sfx_k, sfx_v, lens, workspace=ws)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)

    # properties of every row: finite, inside the range of what it averages (a decoded pool value
    # is at most its vector's norm times the largest centroid, below 3 for 2-4 bits; suffix values
    # by their own maximum)
    assert np.all(np.isfinite(o)), (case, step)
    vmax_all = np.zeros((A, L))
    for p in range(n_pools):
        lay = pool_image.layout(L, Hkv, d, T, w.v_bits(p))
        vm = bufs[p][lay.vmax:lay.vmax + L * Hkv * 4].cpu().numpy().view(np.float32).reshape(L, Hkv)
        for a in range(A):
            if pool_of[a] == p:
                vmax_all[a] = 3.0 * vm.max(axis=1)
    smax = sfx_v[:, :, :, :s_len].abs().amax(dim=(2, 3, 4)).float().cpu().numpy()
    bound = np.maximum(vmax_all, smax)[:, :, None, None] * 1.001
    assert np.all(np.abs(o) <= bound), (case, step)

    # ---- sampled rows against the oracle
    worst = 0.0
    heads = sorted({0, Hq // 2 + 1, Hq - 1})
    for a in s_agents:
        for l in s_layers:
            ref = refs[(pool_of[a], l)]
            ksf, vsf = sfx_host[(a, l)]
            for h in heads:
                g = h // G
                if (pool_of[a], l, g) not in decoded:
                    decoded[(pool_of[a], l, g)] = ref.decoded_layer(0, g)
                khat, vhat = decoded[(pool_of[a], l, g)]
                r = attention.attend_pool_and_suffix(qs[a].f32[l, h:h + 1], khat, vhat,
                                                     ksf[g, :s_len], vsf[g, :s_len])[0]
                err = attention.max_rel_error(o[a, l, h][None], r[None])
                worst = max(worst, err)
                assert err <= TOL, (case, step, a, l, h, err)
    return worst

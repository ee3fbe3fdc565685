"""GPU parity of the CoMixKV sensitivity kernel and the controller end to end.

comix_sensitivity (one workgroup per (agent, layer), fp32 online softmax over
the native window; bf16 operands take the matrix-core kernel, fp32 ones the
vector kernel) against the oracle's fp64 definition: small ragged cases
(empty, one-token and odd windows, GQA 4 and 8, MHA d 64, fp32 and bf16, more
than 32 and more than 64 query rows per kv head), and sampled entries at the Qwen3-32B shape
(8 agents, 64 layers, 64/8 heads, 128-token windows, 8 recent steps).  Then
the allocation on the device-measured sensitivities equals the oracle's
allocation on the oracle's sensitivities whenever their greedy choices are not
within rounding of a tie.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import comixkv
from quantized_shared_kv_amd import polykv as pk

from gpu_helpers import DEV, to_device

pytestmark = pytest.mark.gpu
RTOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()


def _inputs(w, R, dtype):
    """Recent queries [R][A][L][Hq][d] and windows [A][L][Hkv][S][d] from the workload's seeded slices."""
    A, L = w.n_agents, w.n_layers
    q = torch.stack([torch.stack([to_device(w.queries(r, a)) for a in range(A)]) for r in range(R)]).contiguous()
    k = torch.stack([torch.stack([to_device(w.sfx_k(a, l)) for l in range(L)]) for a in range(A)]).contiguous()
    v = torch.stack([torch.stack([to_device(w.sfx_v(a, l)) for l in range(L)]) for a in range(A)]).contiguous()
    if dtype == "f32":
        q, k, v = q.float(), k.float(), v.float()
    return q, k, v


CASES = {
    "g4_bf16_ragged": (wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, n_agents=3, sfx_tokens=37),
                       3, [37, 0, 5], "bf16"),
    "mha_d64_f32": (wl.SMOLLM2.replace(n_layers=2, n_q_heads=4, n_kv_heads=4, n_agents=2, sfx_tokens=64),
                    2, [1, 64], "f32"),
    "g8_40_rows": (wl.QWEN3_32B_MIXED.replace(n_layers=2, n_agents=2, sfx_tokens=50), 5, [50, 13], "bf16"),
    "g8_d64_bf16": (wl.SMOLLM2.replace(n_layers=3, n_q_heads=16, n_kv_heads=2, n_agents=2, sfx_tokens=9),
                    1, [9, 4], "bf16"),
    # 9 steps x 8 heads = 72 rows per kv head: the matrix-core kernel's second pass over the window
    "g8_72_rows_bf16": (wl.QWEN3_32B_MIXED.replace(n_layers=2, n_agents=2, sfx_tokens=37), 9, [37, 20], "bf16"),
    "g4_72_rows_f32": (wl.LLAMA3_8B.replace(n_layers=1, n_kv_heads=2, n_q_heads=8, n_agents=2, sfx_tokens=33),
                       18, [33, 1], "f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sensitivity_matches_oracle(name):
    w, R, lens, dtype = CASES[name]
    print(f"[comix] case {name}", flush=True)
    q, k, v = _inputs(w, R, dtype)
    out = torch.full((w.n_agents, w.n_layers), float("nan"), dtype=torch.float32, device=DEV)
    pk.comix_sensitivity(q, k, v, lens, out)
    torch.cuda.synchronize()
    want = comixkv.sensitivity(q.float().cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy(), lens,
                               w.n_kv_heads)
    got = out.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=RTOL, atol=0)
    assert np.all(got[np.array(lens) == 0] == 0.0)
    # deterministic: a second call writes the same bits
    out2 = torch.empty_like(out)
    pk.comix_sensitivity(q, k, v, lens, out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_sensitivity_qwen3_32b_shape_sampled():
    """Full Qwen3-32B CoMixKV shape: device-seeded windows and queries, 12 sampled (agent, layer) checked."""
    A, L, Hq, Hkv, d, S, R = 8, 64, 64, 8, 128, 128, 8
    print("[comix] qwen3-32b shape", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    q = torch.randn((R, A, L, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    scale = torch.exp(0.5 * torch.randn((1, L, Hkv, 1, d), generator=g, device=DEV))
    k = (torch.randn((A, L, Hkv, S, d), generator=g, device=DEV) * scale).to(torch.bfloat16)
    v = (torch.randn((A, L, Hkv, S, d), generator=g, device=DEV) * scale.flip(1)).to(torch.bfloat16)
    lens = [128, 1, 77, 128, 0, 64, 128, 5]
    out = torch.empty((A, L), dtype=torch.float32, device=DEV)
    pk.comix_sensitivity(q, k, v, lens, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(got[4] == 0.0) and np.all(got >= 0)
    rng = np.random.default_rng(0)
    for a, l in zip(rng.integers(0, A, 12), rng.integers(0, L, 12)):
        want = comixkv.sensitivity(q[:, a:a + 1, l:l + 1].float().cpu().numpy(),
                                   k[a:a + 1, l:l + 1].float().cpu().numpy(),
                                   v[a:a + 1, l:l + 1].float().cpu().numpy(), [lens[a]], Hkv)[0, 0]
        assert abs(got[a, l] - want) <= RTOL * max(want, 1e-30), (a, l, got[a, l], want)


def test_controller_end_to_end_matches_oracle():
    """Sensitivities on the device, bits from the library, against the oracle's on its own sensitivities."""
    w, R, lens, _ = CASES["g8_40_rows"]
    w = w.replace(n_layers=6, n_agents=3)
    lens = [50, 31, 8]
    q, k, v = _inputs(w, R, "bf16")
    out = torch.empty((w.n_agents, w.n_layers), dtype=torch.float32, device=DEV)
    pk.comix_sensitivity(q, k, v, lens, out)
    torch.cuda.synchronize()
    s_dev = out.cpu().numpy().ravel()
    s_ref = comixkv.sensitivity(q.float().cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy(), lens,
                                w.n_kv_heads).ravel()
    cost = np.stack([comixkv.block_cost(256, w.n_kv_heads, w.head_dim)] * s_dev.size)
    err = [pk.lloyd_max_distortion(b) ** 0.5 for b in (2, 3, 4)]
    budget = int(cost[:, 1].sum())  # the bytes of 3 bits everywhere
    bits = pk.comix_allocate_bits(s_dev, cost, err, budget)
    want = comixkv.allocate(s_ref.astype(np.float32), cost, comixkv.error_factors(), budget)
    # equal unless two items' upgrade gains (equal costs: s * (e[b] - e[b + 1])) are within the
    # sensitivities' rounding of each other, which could order the greedy choices differently
    e = comixkv.error_factors()
    gains = sorted([(x * (e[0] - e[1]), i) for i, x in enumerate(s_ref)] + [(x * (e[1] - e[2]), i) for i, x in enumerate(s_ref)])
    close = any(i != j and abs(x - y) <= 1e-4 * max(x, y) for (x, i), (y, j) in zip(gains, gains[1:]))
    if not close:
        assert bits == list(want)
    assert int(cost[np.arange(s_dev.size), np.array(bits) - 2].sum()) <= budget
    assert comixkv.objective(s_ref, comixkv.error_factors(), bits) <= comixkv.objective(
        s_ref, comixkv.error_factors(), [3] * s_dev.size) + 1e-12


def test_refresh_cycle_end_to_end():
    """A CoMixKV refresh cycle on the device: three agents quantise their first 64-token
    blocks at widths chosen from device sensitivities; one exits; the two left refresh on
    their newer windows and quantise their second blocks, which get the freed bytes.

    Checked: widths equal the oracle's refresh cycle on the same sensitivities; every block's
    image equals the oracle's encoding byte for byte; the first blocks' bytes do not change
    when the second blocks are written; the second widths are no narrower than the same
    refresh without the exit; decoding each agent over its two blocks (first as its pool,
    second as its private pool) plus its last 32 native tokens matches the fp64 oracle.
    """
    from oracle import attention, pool_image

    import gpu_helpers as h

    print("[comix] refresh cycle", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=4, n_kv_heads=2, n_q_heads=8, n_agents=3, sfx_tokens=160)
    A, L, Hkv, Hq, d = w.n_agents, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim
    blk, cap, win, R = 64, 128, 96, 2
    q, k_all, v_all = _inputs(w, R, "bf16")
    err = [pk.lloyd_max_distortion(b) ** 0.5 for b in (2, 3, 4)]

    def row(tokens):
        return [tokens * (Hkv * (d + d * b // 8 + 4) + 4) for b in (2, 3, 4)]

    budget = int(0.93 * A * L * row(cap)[1])
    cycle = comixkv.RefreshCycle(budget, L, Hkv, d)
    for a in range(A):
        cycle.start(a, cap)

    def sensitivities(agents, t0):
        out = torch.empty((len(agents), L), dtype=torch.float32, device=DEV)
        pk.comix_sensitivity(q[:, agents].contiguous(), k_all[agents, :, :, t0:t0 + win].contiguous(),
                             v_all[agents, :, :, t0:t0 + win].contiguous(), [win] * len(agents), out)
        torch.cuda.synchronize()
        return {a: out[i].cpu().numpy() for i, a in enumerate(agents)}

    def allocate(agents, sens, done, held):
        s = np.concatenate([sens[a] for a in agents]).astype(np.float32)
        bits = pk.comix_allocate_bits(s, [row(cap - done)] * s.size, err, budget - held)
        return {a: bits[i * L:(i + 1) * L] for i, a in enumerate(agents)}

    def quantize(a, bits, t0):
        dp = h.DevicePool(L, Hkv, d, blk, bits)
        dp.append(0, k_all[a, :, :, t0:t0 + blk].contiguous(), v_all[a, :, :, t0:t0 + blk].contiguous())
        ref = pool_image.PoolImage(L, Hkv, d, blk, bits)
        ref.append(0, k_all[a, :, :, t0:t0 + blk].float().cpu().numpy(),
                   v_all[a, :, :, t0:t0 + blk].float().cpu().numpy())
        assert all(x == 0 for x in h.compare_image(dp, ref).values()), (a, t0)
        return dp, ref

    # refresh 1: all three agents, windows [0, 96)
    sens = sensitivities([0, 1, 2], 0)
    w1 = allocate([0, 1, 2], sens, 0, 0)
    assert {a: [int(x) for x in b] for a, b in cycle.refresh(sens).items()} == w1
    cycle.commit(w1, blk)
    first = {a: quantize(a, w1[a], 0) for a in range(A)}
    snap = {a: first[a][0].host_bytes().copy() for a in range(A)}
    held = sum(row(blk)[b - 2] for a in range(A) for b in w1[a])
    # agent 2 exits
    freed = cycle.exit(2)
    assert freed == sum(row(blk)[b - 2] for b in w1[2])
    del first[2]
    # refresh 2: agents 0 and 1 on windows [64, 160)
    sens = sensitivities([0, 1], blk)
    w2 = allocate([0, 1], sens, blk, held - freed)
    assert {a: [int(x) for x in b] for a, b in cycle.refresh(sens).items()} == w2
    # the same refresh without the exit: agent 2's block and remaining capacity still counted
    sens_x = dict(sens)
    sens_x[2] = np.zeros(L, dtype=np.float32)
    no_exit = allocate([0, 1, 2], sens_x, blk, held)
    assert all(x >= y for a in (0, 1) for x, y in zip(w2[a], no_exit[a]))
    assert sum(w2[a].count(4) for a in (0, 1)) > sum(no_exit[a].count(4) for a in (0, 1))
    cycle.commit(w2, blk)
    second = {a: quantize(a, w2[a], blk) for a in (0, 1)}
    for a in (0, 1):
        assert np.array_equal(first[a][0].host_bytes(), snap[a]), a
    assert [[list(b) for _, b in cycle.blocks[a]] for a in (0, 1)] == [[list(w1[a]), list(w2[a])] for a in (0, 1)]

    # decode: each agent over its two blocks and its last 32 native tokens
    agents = [0, 1]
    S = 160 - cap
    qd = q[-1, agents].contiguous()
    sk = k_all[agents, :, :, cap:].contiguous()
    sv = v_all[agents, :, :, cap:].contiguous()
    out = torch.full(tuple(qd.shape), float("nan"), dtype=torch.float32, device=DEV)
    pools = [first[a][0].pool for a in agents]
    prv = [second[a][0].pool for a in agents]
    wsb = pk.agent_decode_attention(pools, qd, out, 0, sk, sv, [S] * 2, private_pools=prv)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    pk.agent_decode_attention(pools, qd, out, 0, sk, sv, [S] * 2, workspace=ws, private_pools=prv)
    torch.cuda.synchronize()
    skh, svh = sk.float().cpu().numpy(), sv.float().cpu().numpy()
    want = attention.decode_call(
        qd.float().cpu().numpy(), [0, 1], lambda p, l, g: first[agents[p]][1].decoded_layer(l, g),
        lambda i, l: skh[i, l], lambda i, l: svh[i, l], [S] * 2, Hkv,
        private=lambda i, l, g: second[agents[i]][1].decoded_layer(l, g))
    e = attention.max_rel_error(out.cpu().numpy().astype(np.float64), want)
    assert e <= 1e-3, e

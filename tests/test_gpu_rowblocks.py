"""GPU parity of the matrix-core pool kernel above 64 rows per pool (row blocks).

PolyKV explainer, section 2.A: every agent reads the one shared pool, and the
explainer's summary speaks of 15 or more agents at once.  One workgroup of
the matrix-core kernel holds at most 64 query rows (48 with fp32 queries);
a pool with more rows (agents x query heads per kv head) is split into
balanced row blocks, one workgroup each, placed on the same XCD so that the
blocks share its L2 while they read the pool's bytes.  Checked against the
fp64 oracle at the Llama-3-8B head shape (head_dim 128, 4 q heads per kv
head): 17, 20 and 32 agents (68, 80, 128 rows), fp32 queries past 48 rows,
row blocks together with token splits (partial records and k_merge) and with
private segments.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention
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


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("agents", [17, 20, 32])
def test_row_blocks_match_oracle(agents, splits):
    h = H()
    print(f"[rowblocks] agents={agents} splits={splits}", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=330, n_agents=agents,
                             sfx_tokens=20)
    dp, ref = h.build_pair(w, 0, layers=2)
    q, q32 = h.make_queries(w, 3, range(agents))
    sk, sv, fk, fv = h.make_suffix(w, range(agents), 2)
    lens = [(5 * a) % 21 for a in range(agents)]
    out = h.run_decode([dp.pool] * agents, q, (sk, sv), lens, kernel=pk.KERNEL_MFMA, splits=splits)
    want = h.oracle_decode(q32, [0] * agents, [ref], fk, fv, lens, w.n_kv_heads)
    assert np.all(np.isfinite(out))
    err = attention.max_rel_error(out, want)
    assert err <= TOL, err
    # the default kernel choice is the matrix-core kernel too, with the same outputs
    out2 = h.run_decode([dp.pool] * agents, q, (sk, sv), lens, splits=splits)
    assert np.array_equal(out, out2)


def test_row_blocks_fp32_queries():
    """fp32 queries take hi + lo operands: at most 48 rows per block (13 agents = 52 rows -> 2 blocks)."""
    h = H()
    print("[rowblocks] fp32 queries", flush=True)
    w = wl.TINY.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, head_dim=128, pool_tokens=200, n_agents=13)
    dp, ref = h.build_pair(w, 0, layers=2)
    q, q32 = h.make_queries(w, 0, range(13))
    assert q.dtype == torch.float32
    out = h.run_decode([dp.pool] * 13, q, kernel=pk.KERNEL_MFMA)
    want = h.oracle_decode(q32, [0] * 13, [ref], None, None, [0] * 13, w.n_kv_heads)
    err = attention.max_rel_error(out, want)
    assert err <= TOL, err


def test_row_blocks_mixed_pools_and_segments():
    """A launch mixing a 72-row pool, a 12-row pool and private segments."""
    h = H()
    print("[rowblocks] mixed pools and segments", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=140, n_agents=21, n_pools=2,
                             sfx_tokens=12)
    big, rbig = h.build_pair(w, 0, layers=2)
    small, rsmall = h.build_pair(w.replace(pool_tokens=97), 1, layers=2)
    pool_of = [0 if a < 18 else 1 for a in range(21)]
    segs = {}
    for a in (2, 19):  # one agent of each shared pool has a private segment
        n = 40 + a
        dp = h.DevicePool(2, w.n_kv_heads, w.head_dim, n, [3, 3])
        from oracle import pool_image

        rp = pool_image.PoolImage(2, w.n_kv_heads, w.head_dim, n, [3, 3])
        ks = [w.pool_k(5 + a, l) for l in range(2)]
        vs = [w.pool_v(5 + a, l) for l in range(2)]
        rp.append(0, np.stack([x.f32[:, :n] for x in ks]), np.stack([x.f32[:, :n] for x in vs]))
        dp.append(0, h.stack_layers([h._slice(x, 0, n) for x in ks]), h.stack_layers([h._slice(x, 0, n) for x in vs]))
        segs[a] = (dp, rp)
    q, q32 = h.make_queries(w, 1, range(21))
    sk, sv, fk, fv = h.make_suffix(w, range(21), 2)
    lens = [a % 13 for a in range(21)]
    pools = [big.pool if p == 0 else small.pool for p in pool_of]
    prv = [segs[a][0].pool if a in segs else None for a in range(21)]
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=h.DEV)
    wsb = pk.agent_decode_attention(pools, q, out, 0, sk, sv, lens, private_pools=prv)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
    pk.agent_decode_attention(pools, q, out, 0, sk, sv, lens, workspace=ws, private_pools=prv)
    torch.cuda.synchronize()
    refs = [rbig, rsmall]
    want = attention.decode_call(
        q32, pool_of, lambda p, l, g: refs[p].decoded_layer(l, g), fk, fv, lens, w.n_kv_heads,
        private=lambda a, l, g: segs[a][1].decoded_layer(l, g) if a in segs else None)
    err = attention.max_rel_error(out.cpu().numpy().astype(np.float64), want)
    assert err <= TOL, err

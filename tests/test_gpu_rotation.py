"""GPU parity of the randomised-rotation codec variant (a sign vector before the FWHT).

A pool whose config carries a sign mask must encode bit-exactly like the
oracle's codec with the same signs, and decode within 1e-3 of the oracle's fp64
attention over its decoded values, through every finish path: the fused finish
of the matrix-core kernel, and split records merged by k_merge (the vector
kernel, or the matrix-core kernel with two splits).  One launch may mix pools
with different signs; a private segment uses its shared pool's signs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention, pool_image
from quantized_shared_kv_amd import polykv as pk

from gpu_helpers import (DEV, DevicePool, compare_image, make_queries, make_suffix, oracle_decode, run_decode,
                         stack_layers, _slice)

pytestmark = pytest.mark.gpu
TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()


def signed_pair(w, pool_id, signs, layers=None, chunks=None, capacity=None):
    """(device pool, oracle image) of the workload's pool tokens appended in `chunks` (from token 0)."""
    L = w.n_layers if layers is None else layers
    cap = capacity or w.pool_tokens
    bits = w.v_bits(pool_id)[:L]
    dp = DevicePool(L, w.n_kv_heads, w.head_dim, cap, bits, v_signs=signs)
    ref = pool_image.PoolImage(L, w.n_kv_heads, w.head_dim, cap, bits, signs)
    ks = [w.pool_k(pool_id, l) for l in range(L)]
    vs = [w.pool_v(pool_id, l) for l in range(L)]
    t = 0
    for n_ in chunks or [w.pool_tokens]:
        ref.append(0, np.stack([x.f32[:, t:t + n_] for x in ks]), np.stack([x.f32[:, t:t + n_] for x in vs]))
        dp.append(0, stack_layers([_slice(x, t, n_) for x in ks]), stack_layers([_slice(x, t, n_) for x in vs]))
        t += n_
    return dp, ref


CASES = {
    "gqa_d128_mixed": wl.LLAMA3_8B.replace(n_layers=3, pool_tokens=203, v_bits_mode="mixed", n_agents=3,
                                           sfx_tokens=21),
    "mha_d64": wl.SMOLLM2.replace(n_layers=2, n_q_heads=4, n_kv_heads=4, pool_tokens=77, n_agents=2, sfx_tokens=9),
    "tiny_fp32": wl.TINY.replace(n_layers=2, pool_tokens=96, v_bits_mode="mixed"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_signed_pool_image_bit_exact(case):
    w = CASES[case]
    print(f"[rot] image {case}", flush=True)
    signs = wl.rotation_signs(3, w.head_dim)
    dp, ref = signed_pair(w, 0, signs, chunks=[w.pool_tokens // 3, w.pool_tokens - w.pool_tokens // 3])
    bad = compare_image(dp, ref)
    assert all(v == 0 for v in bad.values()), bad


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("kernel,splits", [(pk.KERNEL_MFMA, 0), (pk.KERNEL_MFMA, 2), (pk.KERNEL_VALU, 0)])
def test_signed_pool_decode_matches_oracle(case, kernel, splits):
    w = CASES[case]
    print(f"[rot] decode {case} kernel {kernel} splits {splits}", flush=True)
    signs = wl.rotation_signs(4, w.head_dim)
    dp, ref = signed_pair(w, 0, signs)
    A, L = w.n_agents, w.n_layers
    q, q32 = make_queries(w, 0, range(A))
    lens = [min(w.sfx_tokens, 3 * a + 1) for a in range(A)] if w.sfx_tokens else None
    sfx = None
    fk = fv = None
    if lens:
        sk, sv, fk, fv = make_suffix(w, range(A), L)
        sfx = (sk, sv)
    out = run_decode([dp.pool] * A, q, sfx, lens, kernel=kernel, splits=splits)
    want = oracle_decode(q32, [0] * A, [ref], fk, fv, lens or [0] * A, w.n_kv_heads)
    err = attention.max_rel_error(out, want)
    assert err <= TOL, err


def test_launch_mixing_signed_and_plain_pools():
    w = CASES["gqa_d128_mixed"].replace(n_pools=2, n_agents=4)
    print("[rot] mixed launch", flush=True)
    s0 = wl.rotation_signs(5, w.head_dim)
    d0, r0 = signed_pair(w, 0, s0)
    d1, r1 = signed_pair(w, 1, None)
    A, L = 4, w.n_layers
    pools = [d0.pool, d1.pool, d0.pool, d1.pool]
    q, q32 = make_queries(w, 2, range(A))
    sk, sv, fk, fv = make_suffix(w, range(A), L)
    lens = [0, 5, 21, 1]
    for kernel in (pk.KERNEL_MFMA, pk.KERNEL_VALU):
        out = run_decode(pools, q, (sk, sv), lens, kernel=kernel)
        want = oracle_decode(q32, [0, 1, 0, 1], [r0, r1], fk, fv, lens, w.n_kv_heads)
        assert attention.max_rel_error(out, want) <= TOL


def test_private_segment_with_the_same_signs():
    """Pool + private segment with the same signs: both against the oracle's pool holding the
    two blocks (the segment path, one agent of 4 rows, runs the segment kernel)."""
    w = CASES["gqa_d128_mixed"].replace(n_agents=1, pool_tokens=150)
    print("[rot] private segment", flush=True)
    signs = wl.rotation_signs(6, w.head_dim)
    both, ref = signed_pair(w, 0, signs, chunks=[100, 50])
    shared, _ = signed_pair(w, 0, signs, chunks=[100], capacity=100)
    L = w.n_layers
    cfg = pk.make_config(L, w.n_kv_heads, w.head_dim, 50, w.v_bits(0)[:L], v_signs=signs)
    buf = torch.empty(pk.pool_bytes(cfg), dtype=torch.uint8, device=DEV)
    seg = pk.pool_build(cfg, buf.data_ptr(), buf.numel())
    ks = [w.pool_k(0, l) for l in range(L)]
    vs = [w.pool_v(0, l) for l in range(L)]
    pk.pool_quantize_append(seg, 0, stack_layers([_slice(x, 100, 50) for x in ks]),
                            stack_layers([_slice(x, 100, 50) for x in vs]))
    q, q32 = make_queries(w, 0, range(1))
    a = run_decode([both.pool], q)
    want = oracle_decode(q32, [0], [ref], None, None, [0], w.n_kv_heads)
    out = torch.empty((1, L, w.n_q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(pk.agent_decode_attention([shared.pool], q, out, 0, private_pools=[seg]), 256),
                     dtype=torch.uint8, device=DEV)
    pk.agent_decode_attention([shared.pool], q, out, 0, workspace=ws, private_pools=[seg])
    torch.cuda.synchronize()
    b = out.cpu().numpy().astype(np.float64)
    assert attention.max_rel_error(a, want) <= TOL
    assert attention.max_rel_error(b, want) <= TOL

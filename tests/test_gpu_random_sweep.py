"""GPU parity over a seeded random sweep of small decode configurations, through the C ABI.

Each case draws its shapes from a fixed seed: layers, kv heads, query group size (1 to 8),
pool tokens (ragged, 1 to 700), agents (1 to 40, so up to 320 rows per kv head: several row
blocks at the larger groups), shared or per-agent pools, uniform 3-bit or mixed 2/3/4-bit layers, the
value recipe and dtype of one of the named workloads, and each agent's native-window
length (0 to the capacity), and the codec variant (K scale per tensor, token or channel; plain
or corrected V norm); odd cases decode a random layer sub-range with 2 to 8 forced token splits
(the split-record launch and its merge).  The pool image must match the oracle byte for byte and the
attention outputs the fp64 oracle within 1e-3, as in the fixed cases; the sweep adds the
combinations those do not name.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention
from quantized_shared_kv_amd import polykv as pk

pytestmark = pytest.mark.gpu

TOL = 1e-3
N_CASES = 48


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()
    yield


def _case(i):
    """Workload, layer count, window lengths and kernel of sweep case i (seeded)."""
    rng = np.random.default_rng(1000 + i)
    base = [wl.LLAMA3_8B, wl.SMOLLM2, wl.TINY, wl.QWEN3_32B_MIXED][i % 4]
    hkv = int(rng.integers(1, 5))
    g = [1, 2, 3, 4, 6, 8][(i + i // 6) % 6]  # every group size, against each workload in turn
    distinct = bool(rng.random() < 0.25)  # one pool per agent (at most 8 agents then)
    agents = int(rng.integers(1, 9 if distinct else 41))
    cap = int(rng.choice([0, 8, 64, 130]))
    w = base.replace(n_layers=int(rng.integers(1, 4)), n_kv_heads=hkv, n_q_heads=hkv * g,
                     pool_tokens=int(rng.integers(1, 701)), n_agents=agents,
                     n_pools=agents if distinct else 1, sfx_tokens=cap,
                     sfx_mode="fixed" if cap else "none",
                     v_bits_mode="mixed" if rng.random() < 0.5 else "uniform3", seed=int(rng.integers(0, 1 << 16)))
    lens = [int(rng.integers(0, cap + 1)) for _ in range(agents)] if cap else [0] * agents
    kernel = pk.KERNEL_DEFAULT if i % 3 else pk.KERNEL_VALU
    # the codec variant: K scale per tensor (the pages'), per token or per channel; plain or
    # corrected V norm
    k_scale = [pk.KSCALE_TENSOR, pk.KSCALE_TOKEN, pk.KSCALE_CHANNEL][int(rng.integers(0, 3))]
    v_norm = pk.VNORM_CORRECTED if rng.random() < 0.3 else pk.VNORM_PLAIN
    return w, w.n_layers, lens, distinct, kernel, k_scale, v_norm


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode_matches_oracle(i):
    import gpu_helpers as h

    w, layers, lens, distinct, kernel, k_scale, v_norm = _case(i)
    print(f"[sweep] case {i}: d={w.head_dim} dtype={w.dtype} L={layers} Hkv={w.n_kv_heads} G={w.group} "
          f"T={w.pool_tokens} A={w.n_agents} pools={w.n_pools} bits={w.v_bits_mode} lens={lens} "
          f"kernel={kernel} k_scale={k_scale} v_norm={v_norm}", flush=True)
    A = w.n_agents
    n_pools = A if distinct else 1
    pairs = [h.build_pair(w, p, layers=layers, k_scale=k_scale, v_norm=v_norm) for p in range(n_pools)]
    for dp, ref in pairs:
        bad = h.compare_image(dp, ref)
        assert not any(bad.values()), bad
    q, q32 = h.make_queries(w, 0, range(A))
    sfx = None
    ksf = vsf = None
    if max(lens) > 0:
        kd, vd, ksf, vsf = h.make_suffix(w, range(A), layers)
        sfx = (kd, vd)
    pools = [pairs[a if distinct else 0][0].pool for a in range(A)]
    # half the cases decode a layer sub-range with forced token splits (the split-record pool launch,
    # its window workgroups and k_merge); the others every layer with the planner's choice
    rng = np.random.default_rng(5000 + i)
    lb, splits = 0, 0
    if i % 2:
        lb = int(rng.integers(0, layers))
        splits = int(rng.integers(2, 9))
        q = q[:, lb:].contiguous()
        q32 = q32[:, lb:]
        if sfx is not None:
            sfx = (sfx[0][:, lb:].contiguous(), sfx[1][:, lb:].contiguous())
            ksf0, vsf0 = ksf, vsf
            ksf = lambda a, l: ksf0(a, l + lb)  # noqa: E731
            vsf = lambda a, l: vsf0(a, l + lb)  # noqa: E731
    print(f"[sweep] case {i}: layers {lb}..{layers - 1}, splits {splits or 'auto'}", flush=True)
    out = h.run_decode(pools, q, sfx, lens, layer_begin=lb, kernel=kernel, splits=splits)
    ref = h.oracle_decode(q32, [a if distinct else 0 for a in range(A)], [p[1] for p in pairs], ksf, vsf,
                          lens, w.n_kv_heads, layer_begin=lb)
    assert out.shape == ref.shape and np.all(np.isfinite(out))
    err = attention.max_rel_error(out, ref)
    print(f"[sweep] case {i}: max relative error {err:.2e}", flush=True)
    assert err <= TOL, err

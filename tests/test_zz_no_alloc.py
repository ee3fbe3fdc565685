"""The allocation-free decode entry point against the workspace one, through the C ABI.

agent_decode_attention_noalloc runs the same kernels and plan with the partial
records in the library's per-device scratch array.  Two calls in a row (the
second smaller, so the array holds the first call's records when it starts)
must give exactly the outputs of agent_decode_attention with a caller
workspace, and a call past the array's size is rejected before any launch.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from quantized_shared_kv_amd import polykv as pk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()
    yield


def _call_pair(h, w, layers, agents, sfx_len, kernel, private=None):
    """(outputs of the workspace entry point, outputs of the allocation-free one)."""
    dp, _ = h.build_pair(w, 0, layers=layers)
    q, _ = h.make_queries(w, 0, range(agents))
    kd, vd, _, _ = h.make_suffix(w, range(agents), layers)
    pools = [dp.pool] * agents
    prv = None if private is None else [p.pool if p is not None else None for p in private]
    a = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=h.DEV)
    b = torch.full_like(a, float("nan"))
    wsb = pk.agent_decode_attention(pools, q, a, 0, kd, vd, sfx_len, kernel=kernel, private_pools=prv)
    assert wsb <= pk.noalloc_scratch_bytes()
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
    pk.agent_decode_attention(pools, q, a, 0, kd, vd, sfx_len, workspace=ws, kernel=kernel, private_pools=prv)
    pk.agent_decode_attention_noalloc(pools, q, b, 0, kd, vd, sfx_len, kernel=kernel, private_pools=prv)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


@pytest.mark.parametrize("kernel", [pk.KERNEL_DEFAULT, pk.KERNEL_VALU])
def test_noalloc_equals_workspace_entry_point(kernel):
    import gpu_helpers as h

    print(f"[noalloc] kernel={kernel}", flush=True)
    big = wl.LLAMA3_8B.replace(n_layers=4, n_kv_heads=4, n_q_heads=16, pool_tokens=700, sfx_tokens=96)
    small = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=130, sfx_tokens=20)
    # first a larger call, then a smaller one that reads the array after it
    for w, agents, lens in ((big, 15, [3 * a + 1 for a in range(15)]), (small, 5, [0, 20, 7, 1, 13])):
        a, b = _call_pair(h, w, w.n_layers, agents, lens, kernel)
        assert np.all(np.isfinite(a))
        assert np.array_equal(a, b), float(np.max(np.abs(a - b)))


def test_noalloc_with_split_records_and_segments():
    """Split partial records (k_merge) and private-segment records also come from the array."""
    import gpu_helpers as h

    print("[noalloc] splits and segments", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=300, sfx_tokens=24)
    A = 4
    dp, _ = h.build_pair(w, 0, layers=2)
    priv = []
    for a in range(A):
        n = 16 + 8 * a
        p = h.DevicePool(2, w.n_kv_heads, w.head_dim, n, [3, 3])
        ks = [w.pool_k(1 + a, l) for l in range(2)]
        vs = [w.pool_v(1 + a, l) for l in range(2)]
        p.append(0, h.stack_layers([h._slice(x, 0, n) for x in ks]), h.stack_layers([h._slice(x, 0, n) for x in vs]))
        priv.append(p)
    q, _ = h.make_queries(w, 0, range(A))
    kd, vd, _, _ = h.make_suffix(w, range(A), 2)
    for splits in (3, 0):  # three splits per kv head (k_merge), then the fused default
        a = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=h.DEV)
        b = torch.full_like(a, float("nan"))
        args = ([dp.pool] * A, q)
        kw = dict(sfx_k=kd, sfx_v=vd, sfx_len=[5, 0, 24, 9], splits=splits, private_pools=[x.pool for x in priv])
        wsb = pk.agent_decode_attention(*args, a, 0, **kw)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
        pk.agent_decode_attention(*args, a, 0, workspace=ws, **kw)
        pk.agent_decode_attention_noalloc(*args, b, 0, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_noalloc_rejects_calls_past_the_array():
    """A call needing more than the array is rejected before any launch (PKV_ENOSPACE),
    and its output buffer is left untouched."""
    import gpu_helpers as h

    print("[noalloc] too large", flush=True)
    w = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=1024, sfx_tokens=8)
    dp, _ = h.build_pair(w, 0, layers=2)
    A = 128
    q = torch.zeros((A, 2, 8, 128), dtype=torch.bfloat16, device=h.DEV)
    out = torch.full((A, 2, 8, 128), 7.0, dtype=torch.float32, device=h.DEV)
    # 32 splits of 4 (layer, kv head) units for 512 rows: 8.5M floats of split records, past 32 MiB
    need = pk.agent_decode_attention([dp.pool] * A, q, out, 0, kernel=pk.KERNEL_VALU, splits=32)
    assert need > pk.noalloc_scratch_bytes()
    with pytest.raises(pk.PolyKVError) as e:
        pk.agent_decode_attention_noalloc([dp.pool] * A, q, out, 0, kernel=pk.KERNEL_VALU, splits=32)
    assert e.value.code == -4
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))

"""GPU parity with large and outlier queries, through the C ABI.

The matrix-core pool kernel and the segment kernel feed queries to fp16
operands.  A query row is first multiplied by an exact power of two so that
its largest element stays below 2^15 (the scores are multiplied back), and the
int8 K codes enter as exact fp16 values, so the fp32 accumulation error stays
at the size of q . k itself.  These cases check that against the fp64 oracle
at the 1e-3 bar, on the Llama-3-8B head shape (head_dim 128, 4 q heads per kv
head, 15 agents = 60 rows per kv head): query outlier channels scaled x30,
x100 and x300, bf16 elements above fp16's largest finite value (65504), whole
rows far past it and far below 1, fp32 queries, and a private segment decoded
by the segment kernel.  The vector kernel (fp32 arithmetic) runs the same
cases as a reference point.

Queries past fp16's range are paired with a pool whose K values are scaled down
by an exact power of two, so that the scores stay in the range where fp32
arithmetic resolves them (tens of nats).  Scores of 1e5 nats and more, with keys
tied in their dominant term, differ from fp64 by more than the bar in any fp32
computation (the vector kernel measured 6.7e-3 on such rows); that limit is
stated in include/polykv.h and is not what these cases test.
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
W = wl.LLAMA3_8B.replace(n_layers=2, n_kv_heads=2, n_q_heads=8, pool_tokens=300, sfx_tokens=24)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()
    yield


def H():
    import gpu_helpers

    return gpu_helpers


def _queries(q32: np.ndarray, dtype: str):
    """Device queries of dtype ("bf16" | "f32") and their exact fp32 values."""
    if dtype == "f32":
        x = np.ascontiguousarray(q32, dtype=np.float32)
        return torch.from_numpy(x).to(H().DEV), x
    bits = wl.f32_to_bf16_bits(q32)
    return (torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(H().DEV),
            wl.bf16_bits_to_f32(bits))


def _decode_and_check(dp, ref, q, q32, kernel, sfx_len, private=None):
    h = H()
    A, L = q.shape[0], q.shape[1]
    kd, vd, ksf, vsf = h.make_suffix(W, range(A), L)
    out = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=h.DEV)
    pools = [dp.pool] * A
    prv = None if private is None else [p[0].pool if p is not None else None for p in private]
    wsb = pk.agent_decode_attention(pools, q, out, 0, kd, vd, sfx_len, kernel=kernel, private_pools=prv)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=h.DEV)
    pk.agent_decode_attention(pools, q, out, 0, kd, vd, sfx_len, workspace=ws, kernel=kernel, private_pools=prv)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    r = attention.decode_call(
        q32, [0] * A, lambda p, l, g: ref.decoded_layer(l, g), ksf, vsf, sfx_len, W.n_kv_heads,
        private=None if private is None else
        (lambda a, l, g: private[a][1].decoded_layer(l, g) if private[a] is not None else None))
    assert np.all(np.isfinite(o))
    return attention.max_rel_error(o, r)


def _base_queries(A):
    return np.stack([W.queries(0, a).f32 for a in range(A)]).astype(np.float64)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("factor", [30, 100, 300])
def test_outlier_query_channels(factor, kernel):
    """Every query row has 4 channels (the same 4 in every row) scaled by `factor`."""
    h = H()
    print(f"[qrange] outlier channels x{factor} kernel={kernel}", flush=True)
    A = 15
    dp, ref = h.build_pair(W, 0, layers=W.n_layers)
    q = _base_queries(A)
    rng = np.random.default_rng(factor)
    ch = rng.choice(W.head_dim, size=4, replace=False)
    q[..., ch] *= factor
    qd, q32 = _queries(q, "bf16")
    err = _decode_and_check(dp, ref, qd, q32, kernel, [5 + a for a in range(A)])
    assert err <= TOL, err


def _scaled_pool(pool_id, k_scale_log2, n=None):
    """(DevicePool, PoolImage) of W's pool `pool_id` with K times 2^k_scale_log2 (exact in bf16)."""
    h = H()
    L, n = W.n_layers, n or W.pool_tokens
    bits = [3] * L
    dp = h.DevicePool(L, W.n_kv_heads, W.head_dim, n, bits)
    ref = pool_image.PoolImage(L, W.n_kv_heads, W.head_dim, n, bits)
    kb = np.stack([wl.f32_to_bf16_bits(W.pool_k(pool_id, l).f32[:, :n] * np.float32(2.0 ** k_scale_log2))
                   for l in range(L)])
    vb = np.stack([W.pool_v(pool_id, l).raw[:, :n] for l in range(L)])
    ref.append(0, wl.bf16_bits_to_f32(kb), wl.bf16_bits_to_f32(vb))
    dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(h.DEV)  # noqa: E731
    dp.append(0, dev(kb), dev(vb))
    return dp, ref


def _past_fp16_rows(A):
    """Rows past fp16's range and far from 1, mixed with ordinary rows of the same pool."""
    q = _base_queries(A)
    q[0, 0, 1, 7] = 1.0e5            # one bf16 element above 65504
    q[1, 1, 5, 100] = -7.0e5         # one large negative element
    q[2, :, :] *= 5.0e3              # whole rows just under 2^15 (no rescale, large sums of |q|)
    q[3, 1, :] *= 3.0e5              # whole rows past it (rescaled)
    q[4, 0, 2] *= 1.0e-4             # a row far below 1
    q[5, 0, 3, :] = 0.0              # an all-zero row
    q[6, 1, 0, :64] *= 1.0e6         # half a row past the range, half ordinary
    return q


@pytest.mark.parametrize("kernel", KERNELS)
def test_bf16_queries_past_fp16_range(kernel):
    h = H()
    print(f"[qrange] bf16 past fp16 range kernel={kernel}", flush=True)
    A = 15
    dp, ref = _scaled_pool(0, -14)
    qd, q32 = _queries(_past_fp16_rows(A), "bf16")
    assert np.max(np.abs(q32)) > 65504
    err = _decode_and_check(dp, ref, qd, q32, kernel, [0] + [min(3 * a, W.sfx_tokens) for a in range(1, A)])
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", KERNELS)
def test_fp32_queries_past_fp16_range(kernel):
    """fp32 queries (split into fp16 hi + lo operands on the matrix cores): 12 agents = 48 rows."""
    h = H()
    print(f"[qrange] fp32 past fp16 range kernel={kernel}", flush=True)
    A = 12
    dp, ref = _scaled_pool(0, -24)
    q = _past_fp16_rows(A) * 1024.0
    q[7, 0, 4, 9] = 2.0e9            # fp32 far past every fp16 value
    qd, q32 = _queries(q, "f32")
    err = _decode_and_check(dp, ref, qd, q32, kernel, [2 * a for a in range(A)])
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", KERNELS)
def test_segment_queries_past_fp16_range(kernel):
    """Agents with private segments (decoded by the segment kernel with bf16 queries)."""
    h = H()
    print(f"[qrange] segment past fp16 range kernel={kernel}", flush=True)
    A = 7
    dp, ref = _scaled_pool(0, -14)
    private = [_scaled_pool(1 + a, -14, n=20 + 9 * a) for a in range(A)]
    qd, q32 = _queries(_past_fp16_rows(A), "bf16")
    err = _decode_and_check(dp, ref, qd, q32, kernel, [4] * A, private=private)
    assert err <= TOL, err

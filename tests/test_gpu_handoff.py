"""GPU checks of pool handoff (export header + image bytes -> import) and kv-head shards.

Handoff: a pool built on the device is exported (header + image bytes through
host memory) and imported into a fresh buffer; the imported image must equal
the original byte for byte, and decoding must give bit-identical outputs.
Shards: the pool split into kv-head ranges by pool_shard; each shard's image
must equal the oracle's layout-level shard of its own encoding of the same
inputs (every defined byte), and decoding each shard with the matching
query-head groups must reproduce the whole pool's outputs for those heads bit
for bit (same split plan), and match the fp64 oracle within 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention
from quantized_shared_kv_amd import polykv as pk

from gpu_helpers import DEV, DevicePool, build_pair, compare_image, make_queries, make_suffix, run_decode, oracle_decode

pytestmark = pytest.mark.gpu
KERNELS = [pk.KERNEL_VALU, pk.KERNEL_MFMA]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pk.lib()


def _workload():
    # mixed bits per layer, GQA 4, a ragged pool (not a multiple of 32 tokens)
    return wl.QWEN3_32B_MIXED.replace(n_layers=3, n_q_heads=16, n_kv_heads=4, pool_tokens=203, n_agents=3,
                                      n_pools=1, sfx_tokens=19)


@pytest.mark.parametrize("kernel", KERNELS)
def test_export_import_round_trip(kernel):
    print(f"[handoff] round trip kernel {kernel}", flush=True)
    w = _workload()
    dp, ref = build_pair(w, 0)
    hdr = pk.pool_export_header(dp.pool)
    host = dp.buf.cpu()                                  # the image through host memory
    buf2 = torch.empty(hdr.image_bytes, dtype=torch.uint8, device=DEV)
    buf2.copy_(host)
    p2 = pk.pool_import(hdr, buf2.data_ptr(), buf2.numel())
    torch.cuda.synchronize()
    assert torch.equal(buf2.cpu(), host)
    A = w.n_agents
    q, _ = make_queries(w, 0, range(A))
    sk, sv, _, _ = make_suffix(w, range(A), w.n_layers)
    lens = [0, 7, 19]
    o1 = run_decode([dp.pool] * A, q, (sk, sv), lens, kernel=kernel)
    o2 = run_decode([p2] * A, q, (sk, sv), lens, kernel=kernel)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("kernel", KERNELS)
def test_shards_reproduce_the_whole_pool(kernel):
    print(f"[handoff] shards kernel {kernel}", flush=True)
    w = _workload()
    dp, ref = build_pair(w, 0)
    A, G, H, d, L = w.n_agents, w.group, w.n_kv_heads, w.head_dim, w.n_layers
    q, q32 = make_queries(w, 1, range(A))
    sk, sv, fk, fv = make_suffix(w, range(A), L)
    lens = [5, 0, 19]
    whole = run_decode([dp.pool] * A, q, (sk, sv), lens, kernel=kernel, splits=1)
    want = oracle_decode(q32, [0] * A, [ref], fk, fv, lens, H)
    assert attention.max_rel_error(whole, want) <= 1e-3
    for h0, hc in ((0, 1), (1, 2), (3, 1)):
        sbuf = DevicePool.empty_for(pk.make_config(L, hc, d, w.pool_tokens, w.v_bits(0)))
        sbuf.pool = pk.pool_shard(dp.pool, h0, hc, sbuf.buf.data_ptr(), sbuf.buf.numel())
        assert list(sbuf.pool.n_tokens[:L]) == list(dp.pool.n_tokens[:L])
        bad = compare_image(sbuf, ref.shard(h0, hc))
        assert all(v == 0 for v in bad.values()), (h0, hc, bad)
        qs = q[:, :, h0 * G:(h0 + hc) * G].contiguous()
        sks, svs = sk[:, :, h0:h0 + hc].contiguous(), sv[:, :, h0:h0 + hc].contiguous()
        part = run_decode([sbuf.pool] * A, qs, (sks, svs), lens, kernel=kernel, splits=1)
        assert np.array_equal(part, whole[:, :, h0 * G:(h0 + hc) * G]), (h0, hc)


def test_shards_at_the_llama3_8b_shape():
    """Full Llama-3-8B pool (32 layers, 8 kv heads, 4096 tokens, 15 agents, 128-token windows) split
    into 8 one-head shards: every region of each shard equals the matching slice of the whole image,
    and each shard's decode equals the whole pool's rows for its heads bit for bit (one split each)."""
    print("[handoff] llama3-8b shards", flush=True)
    L, H, Hq, d, T, A, S = 32, 8, 32, 128, 4096, 15, 128
    G = Hq // H
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    k = (torch.randn((L, H, T, d), generator=g, device=DEV) * 1.3).to(torch.bfloat16)
    v = torch.randn((L, H, T, d), generator=g, device=DEV).to(torch.bfloat16)
    whole = DevicePool(L, H, d, T, [3] * L)
    whole.append(0, k, v)
    q = torch.randn((A, L, Hq, d), generator=g, device=DEV).to(torch.bfloat16)
    sk = torch.randn((A, L, H, S, d), generator=g, device=DEV).to(torch.bfloat16)
    sv = torch.randn((A, L, H, S, d), generator=g, device=DEV).to(torch.bfloat16)
    lens = [1 + 9 * a for a in range(A)]
    ref = run_decode([whole.pool] * A, q, (sk, sv), lens, splits=1)
    img = whole.buf
    P = whole.pool
    tc = P.tc
    for h in range(H):
        sh = DevicePool.empty_for(pk.make_config(L, 1, d, T, [3] * L))
        sh.pool = pk.pool_shard(P, h, 1, sh.buf.data_ptr(), sh.buf.numel())
        Q = sh.pool
        b = sh.buf
        torch.cuda.synchronize()
        kq_w = img[P.off_kq:P.off_kq + L * H * tc * d].view(L, H, tc * d)[:, h]
        assert torch.equal(b[Q.off_kq:Q.off_kq + L * tc * d].view(L, tc * d), kq_w)
        vn_w = img[P.off_vn:P.off_vn + L * H * tc * 4].view(L, H, tc * 4)[:, h]
        assert torch.equal(b[Q.off_vn:Q.off_vn + L * tc * 4].view(L, tc * 4), vn_w)
        assert torch.equal(b[Q.off_ks:Q.off_ks + L * tc * 4], img[P.off_ks:P.off_ks + L * tc * 4])
        vm_w = img[P.off_vmax:P.off_vmax + L * H * 4].view(L, H, 4)[:, h]
        assert torch.equal(b[Q.off_vmax:Q.off_vmax + L * 4].view(L, 4), vm_w)
        for l in range(L):
            n = (tc // 8) * d * 3
            assert torch.equal(b[Q.off_vc[l]:Q.off_vc[l] + n], img[P.off_vc[l] + h * n:P.off_vc[l] + (h + 1) * n])
        part = run_decode([Q] * A, q[:, :, h * G:(h + 1) * G].contiguous(),
                          (sk[:, :, h:h + 1].contiguous(), sv[:, :, h:h + 1].contiguous()), lens, splits=1)
        assert np.array_equal(part, ref[:, :, h * G:(h + 1) * G]), h

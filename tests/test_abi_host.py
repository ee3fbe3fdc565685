"""Host-side checks of the C ABI (no GPU): symbols, struct mirrors, layout, tables, errors.

Nothing here enqueues device work: every call either is host-only
(pool_bytes, pool_build, the auxiliary queries, a workspace-size query) or
fails host-side validation before any launch.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import lloyd_max, pool_image
from quantized_shared_kv_amd import polykv as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "polykv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"pool_bytes", "pool_build", "pool_quantize_append", "agent_decode_attention",
                          "comix_sensitivity", "comix_allocate_bits", "pkv_lloyd_max_distortion",
                          "pool_export_header", "pool_import", "pool_shard"}
    lib = pk.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_struct_mirrors_match_c_sizes():
    lib = pk.lib()
    assert lib.pkv_abi_sizeof(0) == ctypes.sizeof(pk.PoolConfig)
    assert lib.pkv_abi_sizeof(1) == ctypes.sizeof(pk.Pool)
    assert lib.pkv_abi_sizeof(2) == ctypes.sizeof(pk.DecodeArgs)
    assert lib.pkv_abi_sizeof(3) == ctypes.sizeof(pk.ComixArgs)
    assert lib.pkv_abi_sizeof(4) == ctypes.sizeof(pk.PoolHeader)
    assert lib.pkv_abi_sizeof(5) == 0
    assert lib.pkv_version() == pk.ABI_VERSION


@pytest.mark.parametrize("shape", [(1, 1, 64, 512, [3]), (24, 32, 64, 1851, [3] * 24), (32, 8, 128, 4096, [3] * 32),
                                   (32, 8, 128, 7194, [3] * 32), (3, 2, 128, 33, [2, 4, 3]), (5, 3, 64, 1, [4] * 5)])
def test_layout_matches_oracle(shape):
    L, H, d, cap, bits = shape
    cfg = pk.make_config(L, H, d, cap, bits)
    ref = pool_image.layout(L, H, d, cap, bits)
    assert pk.pool_bytes(cfg) == ref.total
    pool = pk.pool_build(cfg, 256 * 1024, ref.total)  # a fake aligned address: host-only
    assert pool.tc == ref.tc and pool.bytes == ref.total
    assert (pool.off_kq, pool.off_vn, pool.off_ks, pool.off_vmax, pool.off_amax) == (ref.kq, ref.vn, ref.ks, ref.vmax,
                                                                                       ref.amax)
    assert list(pool.off_vc[:L + 1]) == ref.vc
    assert list(pool.n_tokens[:L]) == [0] * L


def test_pool_bytes_has_no_agent_dimension():
    # the only inputs are the pool shape: the same bytes serve any number of agents
    cfg = pk.make_config(32, 8, 128, 4096, 3)
    n = pk.pool_bytes(cfg)
    assert n == pool_image.layout(32, 8, 128, 4096, [3] * 32).total
    # 180 bytes per (token, kv head) plus one 4-byte scale per (token, layer), plus padding
    assert 0 <= n - (32 * 8 * 4096 * 180 + 32 * 4096 * 4 + 32 * 8 * 4) < 5 * 256 + 32 * 4 + 256


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_library_table_equals_oracle_table_bitwise(bits):
    # two independent solvers (C++ erfc, NumPy/SciPy ndtr) of the same fixed point
    c, t = pk.lloyd_max_table(bits)
    rc, rt = lloyd_max.table_f32(bits)
    assert np.array_equal(np.array(c, dtype=np.float32).view(np.uint32), rc.view(np.uint32))
    assert np.array_equal(np.array(t, dtype=np.float32).view(np.uint32), rt.view(np.uint32))


def test_lloyd_table_rejects_other_bits():
    with pytest.raises(pk.PolyKVError):
        pk.lloyd_max_table(5)


def test_config_errors():
    lib = pk.lib()
    assert lib.pool_bytes(None) == 0
    bad = [pk.make_config(0, 1, 64, 10, []), pk.make_config(1, 0, 64, 10, [3]), pk.make_config(1, 1, 96, 10, [3]),
           pk.make_config(1, 1, 64, 0, [3]), pk.make_config(2, 1, 64, 10, [3, 5]), pk.make_config(1, 1, 64, 10, [1])]
    for cfg in bad:
        assert pk.pool_bytes(cfg) == 0
    good = pk.make_config(2, 1, 64, 10, [3, 2])
    n = pk.pool_bytes(good)
    out = pk.Pool()
    assert lib.pool_build(ctypes.byref(good), ctypes.c_void_p(4096), n - 1, ctypes.byref(out)) == -4
    assert lib.pool_build(ctypes.byref(good), ctypes.c_void_p(4096 + 16), n, ctypes.byref(out)) == -1
    assert lib.pool_build(ctypes.byref(good), None, n, ctypes.byref(out)) == -1
    assert lib.pool_build(ctypes.byref(good), ctypes.c_void_p(4096), n, None) == -1
    assert lib.pool_build(ctypes.byref(bad[2]), ctypes.c_void_p(4096), n, ctypes.byref(out)) == -2


def _fake_pool(L=2, H=2, d=64, cap=100, bits=3):
    cfg = pk.make_config(L, H, d, cap, bits)
    return pk.pool_build(cfg, 1 << 20, pk.pool_bytes(cfg))


def test_quantize_append_validation_errors():
    lib = pk.lib()
    pool = _fake_pool()
    f = lib.pool_quantize_append
    k = ctypes.c_void_p(1 << 24)
    assert f(None, 0, 1, k, k, 0, 4, None) == -1
    assert f(ctypes.byref(pool), 0, 3, k, k, 0, 4, None) == -1           # layers out of range
    assert f(ctypes.byref(pool), -1, 1, k, k, 0, 4, None) == -1
    assert f(ctypes.byref(pool), 0, 1, k, k, 7, 4, None) == -2           # dtype
    assert f(ctypes.byref(pool), 0, 1, None, k, 0, 4, None) == -1
    assert f(ctypes.byref(pool), 0, 1, ctypes.c_void_p((1 << 24) + 4), k, 0, 4, None) == -1  # misaligned
    assert f(ctypes.byref(pool), 0, 1, k, k, 0, 101, None) == -3         # capacity
    assert f(ctypes.byref(pool), 0, 1, k, k, 0, -1, None) == -1
    assert f(ctypes.byref(pool), 0, 0, k, k, 0, 4, None) == 0            # empty: no-op
    assert f(ctypes.byref(pool), 0, 1, k, k, 0, 0, None) == 0
    pool.n_tokens[0] = 8                                                  # unequal layer counts
    assert f(ctypes.byref(pool), 0, 2, k, k, 0, 4, None) == -1
    assert list(pool.n_tokens[:2]) == [8, 0]


class _FakeT:
    """Minimal stand-in with the attributes the binding reads, for host-only calls."""

    def __init__(self, shape, ptr, dtype="bf16", is_cuda=True):
        import torch

        self.shape = tuple(shape)
        self._ptr = ptr
        self.dtype = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16}[dtype]
        self.is_cuda = is_cuda

    def data_ptr(self):
        return self._ptr

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)


def test_decode_workspace_query_and_errors():
    lib = pk.lib()
    pool = _fake_pool(L=2, H=2, d=64, cap=100)
    pool.n_tokens[0] = pool.n_tokens[1] = 70
    A, lc, hq, d = 3, 2, 4, 64
    q = _FakeT((A, lc, hq, d), 1 << 24)
    out = _FakeT((A, lc, hq, d), 1 << 25, "f32")
    ws = pk.agent_decode_attention([pool] * A, q, out)
    assert ws > 0 and ws % 4 == 0
    # suffix partials add records for every (agent, layer, q head)
    sk = _FakeT((A, lc, 2, 16, d), 1 << 26)
    ws2 = pk.agent_decode_attention([pool] * A, q, out, sfx_k=sk, sfx_v=sk, sfx_len=[0, 5, 16])
    assert ws2 >= ws + A * lc * hq * (2 + d) * 4
    with pytest.raises(pk.PolyKVError):  # sfx_len beyond capacity
        pk.agent_decode_attention([pool] * A, q, out, sfx_k=sk, sfx_v=sk, sfx_len=[0, 5, 17])
    with pytest.raises(pk.PolyKVError):  # heads not a multiple of kv heads
        pk.agent_decode_attention([pool] * A, _FakeT((A, lc, 3, d), 1 << 24), _FakeT((A, lc, 3, d), 1 << 25, "f32"))
    with pytest.raises(pk.PolyKVError):  # layers beyond the pool
        pk.agent_decode_attention([pool] * A, q, out, layer_begin=1)
    other = _fake_pool(L=2, H=2, d=128, cap=100)
    with pytest.raises(pk.PolyKVError):  # mixed head_dim
        pk.agent_decode_attention([pool, pool, other], q, out)
    pool.n_tokens[1] = 69
    with pytest.raises(pk.PolyKVError):  # unequal token counts across the call's layers
        pk.agent_decode_attention([pool] * A, q, out)
    pool.n_tokens[1] = 70
    for bad in ((_FakeT((A, lc, hq, d), (1 << 24) + 8), out), (q, _FakeT((A, lc, hq, d), (1 << 25) + 4, "f32"))):
        with pytest.raises(pk.PolyKVError):  # q and out must be 16-byte aligned
            pk.agent_decode_attention([pool] * A, *bad)
    with pytest.raises(pk.PolyKVError):  # suffix arrays too
        pk.agent_decode_attention([pool] * A, q, out, sfx_k=_FakeT((A, lc, 2, 16, d), (1 << 26) + 2), sfx_v=sk,
                                  sfx_len=[0, 5, 16])
    # size is independent of pointers and grows with distinct pools
    p2 = _fake_pool(L=2, H=2, d=64, cap=100)
    p2.n_tokens[0] = p2.n_tokens[1] = 70
    ws3 = pk.agent_decode_attention([pool, p2, pool], q, out)
    assert ws3 >= ws
    # too-small workspace is rejected before any launch
    a, keep = pk._decode_args([pool] * A, q, out, 0)
    size = ctypes.c_size_t(ws - 4)
    assert lib.agent_decode_attention(ctypes.byref(a), ctypes.c_void_p(1 << 27), ctypes.byref(size), None) == -4
    size = ctypes.c_size_t(ws)
    assert lib.agent_decode_attention(ctypes.byref(a), ctypes.c_void_p((1 << 27) + 4), ctypes.byref(size), None) == -1
    assert lib.agent_decode_attention(ctypes.byref(a), None, None, None) == -1
    a.q_dtype = 9
    assert lib.agent_decode_attention(ctypes.byref(a), None, ctypes.byref(size), None) == -2
    a.q_dtype = 1
    a.kernel = 7
    assert lib.agent_decode_attention(ctypes.byref(a), None, ctypes.byref(size), None) == -1
    a.kernel = 0
    a.n_agents = 0
    assert lib.agent_decode_attention(ctypes.byref(a), None, ctypes.byref(size), None) == 0 and size.value == 0
    del keep


def test_decode_private_pools_workspace_and_errors():
    """Private pools add their partial records to the workspace; they must match the shared
    pools' heads and head_dim, hold the call's layers uniformly, and not be a shared pool."""
    pool = _fake_pool(L=2, H=2, d=64, cap=100)
    pool.n_tokens[0] = pool.n_tokens[1] = 70
    A, lc, hq, d = 3, 2, 4, 64
    q = _FakeT((A, lc, hq, d), 1 << 24)
    out = _FakeT((A, lc, hq, d), 1 << 25, "f32")
    base = pk.agent_decode_attention([pool] * A, q, out)
    prv = _fake_pool(L=2, H=2, d=64, cap=40)
    prv.n_tokens[0] = prv.n_tokens[1] = 40
    ws = pk.agent_decode_attention([pool] * A, q, out, private_pools=[prv, None, None])
    G = hq // 2
    assert ws >= base + lc * 2 * 1 * G * (2 + d) * 4  # at least one split of the private pool's rows
    assert pk.agent_decode_attention([pool] * A, q, out, private_pools=[None] * A) == base
    empty = _fake_pool(L=2, H=2, d=64, cap=8)  # a private pool with no tokens is allowed
    pk.agent_decode_attention([pool] * A, q, out, private_pools=[empty, prv, None])
    with pytest.raises(pk.PolyKVError):  # head_dim differs from the shared pool's
        pk.agent_decode_attention([pool] * A, q, out, private_pools=[_fake_pool(L=2, H=2, d=128, cap=8), None, None])
    with pytest.raises(pk.PolyKVError):  # fewer layers than the call
        pk.agent_decode_attention([pool] * A, q, out, private_pools=[_fake_pool(L=1, H=2, d=64, cap=8), None, None])
    prv.n_tokens[1] = 39
    with pytest.raises(pk.PolyKVError):  # unequal token counts across the call's layers
        pk.agent_decode_attention([pool] * A, q, out, private_pools=[prv, None, None])
    prv.n_tokens[1] = 40
    with pytest.raises(pk.PolyKVError):  # a shared pool named as a private one
        pk.agent_decode_attention([pool] * A, q, out, private_pools=[pool, None, None])
    with pytest.raises(ValueError):  # one entry per agent
        pk.agent_decode_attention([pool] * A, q, out, private_pools=[prv])
    prv.cfg.v_signs[0] = 1
    with pytest.raises(pk.PolyKVError):  # a different V rotation from the shared pool's
        pk.agent_decode_attention([pool] * A, q, out, private_pools=[prv, None, None])
    pool.cfg.v_signs[0] = 1  # the same rotation on both
    pk.agent_decode_attention([pool] * A, q, out, private_pools=[prv, None, None])


def test_rotation_signs_in_the_config():
    import workloads as wl

    s = wl.rotation_signs(0, 64)
    cfg = pk.make_config(2, 2, 64, 40, [3, 3], v_signs=s)
    mask = bytes(cfg.v_signs)
    assert all(mask[i] == 0 for i in range(8, 16))
    assert [(mask[i // 8] >> (i % 8)) & 1 for i in range(64)] == [int(x < 0) for x in s]
    assert pk.pool_bytes(cfg) == pk.pool_bytes(pk.make_config(2, 2, 64, 40, [3, 3]))  # same layout
    cfg.v_signs[8] = 1  # a sign past head_dim 64
    assert pk.pool_bytes(cfg) == 0
    with pytest.raises(ValueError):
        pk.make_config(2, 2, 64, 40, [3, 3], v_signs=s[:10])


def test_binding_rejects_bad_tensors_before_any_launch():
    """The binding checks what the C side cannot see (dtypes, devices, suffix shapes) and
    raises ValueError before the library is called, so no kernel can write past a buffer."""
    pool = _fake_pool(L=2, H=2, d=64, cap=100)
    pool.n_tokens[0] = pool.n_tokens[1] = 70
    A, lc, hq, d = 3, 2, 4, 64
    q = _FakeT((A, lc, hq, d), 1 << 24)
    out = _FakeT((A, lc, hq, d), 1 << 25, "f32")
    sk = _FakeT((A, lc, 2, 16, d), 1 << 26)
    sv = _FakeT((A, lc, 2, 16, d), 1 << 27)
    pk.agent_decode_attention([pool] * A, q, out, sfx_k=sk, sfx_v=sv, sfx_len=[0, 5, 16])  # the good call
    bad_calls = {
        "bf16 out": dict(out=_FakeT((A, lc, hq, d), 1 << 25, "bf16")),
        "fp16 out": dict(out=_FakeT((A, lc, hq, d), 1 << 25, "f16")),
        "fp16 q": dict(q=_FakeT((A, lc, hq, d), 1 << 24, "f16")),
        "host q": dict(q=_FakeT((A, lc, hq, d), 1 << 24, is_cuda=False)),
        "host out": dict(out=_FakeT((A, lc, hq, d), 1 << 25, "f32", is_cuda=False)),
        "fp32 sfx_v with bf16 sfx_k": dict(sfx_v=_FakeT((A, lc, 2, 16, d), 1 << 27, "f32")),
        "suffix with fewer layers": dict(sfx_k=_FakeT((A, 1, 2, 16, d), 1 << 26), sfx_v=_FakeT((A, 1, 2, 16, d), 1 << 27)),
        "suffix with fewer agents": dict(sfx_k=_FakeT((2, lc, 2, 16, d), 1 << 26),
                                         sfx_v=_FakeT((2, lc, 2, 16, d), 1 << 27)),
        "suffix with other kv heads": dict(sfx_k=_FakeT((A, lc, 1, 16, d), 1 << 26),
                                           sfx_v=_FakeT((A, lc, 1, 16, d), 1 << 27)),
        "suffix with other head_dim": dict(sfx_k=_FakeT((A, lc, 2, 16, 2 * d), 1 << 26),
                                           sfx_v=_FakeT((A, lc, 2, 16, 2 * d), 1 << 27)),
        "host suffix": dict(sfx_k=_FakeT((A, lc, 2, 16, d), 1 << 26, is_cuda=False),
                            sfx_v=_FakeT((A, lc, 2, 16, d), 1 << 27, is_cuda=False)),
        "fp16 suffix": dict(sfx_k=_FakeT((A, lc, 2, 16, d), 1 << 26, "f16"),
                            sfx_v=_FakeT((A, lc, 2, 16, d), 1 << 27, "f16")),
        "sfx_k without sfx_v": dict(sfx_v=None),
    }
    for what, kw in bad_calls.items():
        args = dict(q=q, out=out, sfx_k=sk, sfx_v=sv)
        args.update(kw)
        with pytest.raises((ValueError, TypeError), match=""):
            pk.agent_decode_attention([pool] * A, args["q"], args["out"], sfx_k=args["sfx_k"], sfx_v=args["sfx_v"],
                                      sfx_len=[0, 5, 16])
        # and the same with a workspace: still rejected before the library is reached
        with pytest.raises((ValueError, TypeError)):
            pk.agent_decode_attention([pool] * A, args["q"], args["out"], sfx_k=args["sfx_k"], sfx_v=args["sfx_v"],
                                      sfx_len=[0, 5, 16], workspace=_FakeWs(1 << 28, 1 << 20)), what


def test_binding_rejects_a_workspace_without_address():
    """A zero-size workspace tensor has address 0, which the C call would take as a size query
    and so enqueue nothing; the binding raises instead."""
    pool = _fake_pool(L=2, H=2, d=64, cap=100)
    pool.n_tokens[0] = pool.n_tokens[1] = 70
    A, lc, hq, d = 3, 2, 4, 64
    q = _FakeT((A, lc, hq, d), 1 << 24)
    out = _FakeT((A, lc, hq, d), 1 << 25, "f32")
    with pytest.raises(ValueError, match="no device address"):
        pk.agent_decode_attention([pool] * A, q, out, workspace=_NullWs())


class _NullWs:
    """A zero-size device tensor stand-in: address 0."""

    def data_ptr(self):
        return 0

    def numel(self):
        return 0

    def element_size(self):
        return 1


class _FakeWs:
    """A workspace stand-in that must never reach the library in the tests that use it."""

    def __init__(self, ptr, n):
        self._ptr, self._n = ptr, n

    def data_ptr(self):
        raise AssertionError("the binding reached the library call")

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def test_stream_read_validation_is_host_side():
    """The streaming-read measurement kernel rejects bad arguments before any launch."""
    lib = pk.lib()
    f = lib.pkv_stream_read
    sink = ctypes.c_void_p(1 << 24)
    assert f(None, 16, sink, None) == -1
    assert f(ctypes.c_void_p(1 << 20), 16, None, None) == -1
    assert f(ctypes.c_void_p((1 << 20) + 8), 16, sink, None) == -1   # src not 16-byte aligned
    assert f(ctypes.c_void_p(1 << 20), 24, sink, None) == -1          # bytes not a multiple of 16
    assert lib.pkv_stream_read_sink_words() > 0


@pytest.mark.parametrize("k_scale", [0, 1, 2])
@pytest.mark.parametrize("v_norm", [0, 1])
def test_variant_layouts_match_oracle(k_scale, v_norm):
    for L, H, d, cap, bits in ((3, 2, 128, 33, [2, 4, 3]), (32, 8, 128, 4096, [3] * 32), (5, 3, 64, 1, [4] * 5)):
        cfg = pk.make_config(L, H, d, cap, bits, k_scale=k_scale, v_norm=v_norm)
        ref = pool_image.layout(L, H, d, cap, bits, k_scale)
        assert pk.pool_bytes(cfg) == ref.total
        pool = pk.pool_build(cfg, 256 * 1024, ref.total)
        assert (pool.off_ks, pool.off_vmax, pool.off_amax) == (ref.ks, ref.vmax, ref.amax)
        assert list(pool.off_vc[:L + 1]) == ref.vc


def test_variant_config_validation():
    cfg = pk.make_config(2, 2, 64, 40, [3, 3], k_scale=3)
    assert pk.pool_bytes(cfg) == 0 and pk.lib().pool_build(ctypes.byref(cfg), ctypes.c_void_p(4096), 1 << 20,
                                                          ctypes.byref(pk.Pool())) == -2
    cfg = pk.make_config(2, 2, 64, 40, [3, 3], v_norm=2)
    assert pk.pool_bytes(cfg) == 0
    cfg = pk.make_config(2, 2, 64, 40, [3, 3])
    cfg.reserved[1] = 1
    assert pk.pool_bytes(cfg) == 0

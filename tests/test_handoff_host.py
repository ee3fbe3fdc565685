"""Host-side checks of the pool handoff header and kv-head shards (no GPU).

pool_export_header / pool_import are host-only and must round-trip a
descriptor exactly and reject inconsistent headers; pool_shard validates on
the host before it enqueues any copy, so its error paths run here.  The
shard's layout must be the oracle's layout for the reduced head count.
"""
import ctypes

import pytest

from oracle import pool_image
from quantized_shared_kv_amd import polykv as pk

BASE = 1 << 20  # a fake 256-byte aligned device address: nothing is dereferenced on the host


def _pool(H=4, bits=(2, 3, 4), cap=100):
    cfg = pk.make_config(len(bits), H, 64, cap, list(bits))
    n = pk.pool_bytes(cfg)
    p = pk.pool_build(cfg, BASE, n)
    for l in range(len(bits)):
        p.n_tokens[l] = 70
    return p, n


def test_header_round_trip():
    p, n = _pool()
    h = pk.pool_export_header(p)
    assert h.magic == 0x31564B50 and h.image_bytes == n and h.abi_version == pk.ABI_VERSION
    q = pk.pool_import(h, 8 * BASE, n)
    assert q.base == 8 * BASE
    for f, _ in pk.Pool._fields_:
        if f != "base":
            a, b = getattr(p, f), getattr(q, f)
            assert (bytes(a) == bytes(b)) if hasattr(a, "_length_") or isinstance(a, ctypes.Structure) else a == b, f


def test_import_rejects_inconsistent_headers():
    p, n = _pool()
    f = pk.lib().pool_import

    def imp(h, buf=8 * BASE, nbytes=n):
        out = pk.Pool()
        return f(ctypes.byref(h), ctypes.c_void_p(buf), nbytes, ctypes.byref(out))

    good = pk.pool_export_header(p)
    assert imp(good) == 0
    for mutate, code in ((lambda h: setattr(h, "magic", 0), -1), (lambda h: setattr(h, "abi_version", 999), -1),
                         (lambda h: setattr(h, "image_bytes", n + 256), -1),
                         (lambda h: h.n_tokens.__setitem__(1, 101), -1), (lambda h: h.n_tokens.__setitem__(0, -1), -1),
                         (lambda h: setattr(h.cfg, "head_dim", 96), -2)):
        h = pk.pool_export_header(p)
        mutate(h)
        assert imp(h) == code
    assert imp(good, nbytes=n - 1) == -4
    assert imp(good, buf=8 * BASE + 64) == -1
    assert f(None, ctypes.c_void_p(8 * BASE), n, ctypes.byref(pk.Pool())) == -1
    bad = pk.Pool()
    assert pk.lib().pool_export_header(ctypes.byref(bad), ctypes.byref(pk.PoolHeader())) == -1


def test_shard_validation_runs_on_host():
    p, n = _pool()
    f = pk.lib().pool_shard
    need = pk.pool_bytes(pk.make_config(3, 2, 64, 100, [2, 3, 4]))
    assert need == pool_image.layout(3, 2, 64, 100, [2, 3, 4]).total

    def shard(h0, hc, buf=64 * BASE, nbytes=need):
        out = pk.Pool()
        return f(ctypes.byref(p), h0, hc, ctypes.c_void_p(buf), nbytes, ctypes.byref(out), None)

    assert shard(3, 2) == -1 and shard(-1, 1) == -1 and shard(0, 0) == -1
    assert shard(0, 2, nbytes=need - 1) == -4
    assert shard(0, 2, buf=64 * BASE + 128) == -1
    assert shard(0, 2, buf=BASE + 256) == -1  # overlaps the source image

"""Helpers for GPU parity tests: build pools on the device and in the oracle from the same inputs.

Inputs come from ``workloads`` (seeded, synthetic).  The device side goes
through the C ABI binding only; the oracle side through ``oracle`` only.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import attention, pool_image
from quantized_shared_kv_amd import polykv as pk

DEV = "cuda:0"


def to_device(t) -> torch.Tensor:
    """A workloads.Tensor's raw storage as a device tensor of its dtype."""
    raw = np.ascontiguousarray(t.raw)
    if t.dtype == "bf16":
        return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(raw).to(DEV)


class DevicePool:
    """A pool in a torch-owned device buffer."""

    def __init__(self, n_layers, n_kv_heads, head_dim, capacity, bits, v_signs=None, k_scale=0, v_norm=0):
        self._allocate(pk.make_config(n_layers, n_kv_heads, head_dim, capacity, bits, v_signs=v_signs,
                                      k_scale=k_scale, v_norm=v_norm))

    @classmethod
    def empty_for(cls, cfg) -> "DevicePool":
        """A buffer of pool_bytes(cfg) bytes with no descriptor built yet (self.pool unset)."""
        dp = cls.__new__(cls)
        dp.cfg = cfg
        dp.buf = torch.empty(pk.pool_bytes(cfg), dtype=torch.uint8, device=DEV)
        return dp

    def _allocate(self, cfg):
        self.cfg = cfg
        n = pk.pool_bytes(self.cfg)
        assert n > 0
        self.buf = torch.empty(n, dtype=torch.uint8, device=DEV)
        self.pool = pk.pool_build(self.cfg, self.buf.data_ptr(), n)

    def append(self, layer_begin, k: torch.Tensor, v: torch.Tensor):
        pk.pool_quantize_append(self.pool, layer_begin, k, v)

    def host_bytes(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.buf.cpu().numpy()


def stack_layers(tensors):
    """Stack per-layer workloads.Tensor [Hkv][n][d] into one device tensor [L][Hkv][n][d]."""
    return torch.stack([to_device(t) for t in tensors]).contiguous()


def build_pair(w, pool_id, layers=None, capacity=None, chunks=None, k_scale=0, v_norm=0):
    """(DevicePool, oracle PoolImage) for one pool of workload w, appended in the same chunks.

    chunks: list of token counts appended one after the other (default: all at once).
    k_scale, v_norm: the pool's codec variant (pkv K-scale granularity, corrected V norm).
    """
    L = w.n_layers if layers is None else layers
    bits = w.v_bits(pool_id)[:L]
    cap = capacity or w.pool_tokens
    dp = DevicePool(L, w.n_kv_heads, w.head_dim, cap, bits, k_scale=k_scale, v_norm=v_norm)
    ref = pool_image.PoolImage(L, w.n_kv_heads, w.head_dim, cap, bits, k_scale=k_scale, corrected_norm=bool(v_norm))
    ks = [w.pool_k(pool_id, l) for l in range(L)]
    vs = [w.pool_v(pool_id, l) for l in range(L)]
    chunks = chunks or [w.pool_tokens]
    t = 0
    for n in chunks:
        kk = np.stack([x.f32[:, t:t + n] for x in ks])
        vv = np.stack([x.f32[:, t:t + n] for x in vs])
        ref.append(0, kk, vv)
        kd = stack_layers([_slice(x, t, n) for x in ks])
        vd = stack_layers([_slice(x, t, n) for x in vs])
        dp.append(0, kd, vd)
        t += n
    return dp, ref


class _Sliced:
    def __init__(self, raw, dtype):
        self.raw = raw
        self.dtype = dtype


def _slice(t, start, n):
    return _Sliced(np.ascontiguousarray(t.raw[:, start:start + n]), t.dtype)


def compare_image(dp: DevicePool, ref: pool_image.PoolImage) -> dict:
    """Compare every defined byte of the device pool with the oracle; returns mismatch counts."""
    buf = dp.host_bytes()
    lay = ref.lay
    L, H, d, tc = lay.n_layers, lay.n_kv_heads, lay.head_dim, lay.tc
    T = int(ref.n_tokens[0])
    out = {}
    kq = buf[lay.kq:lay.kq + L * H * tc * d].view(np.int8).reshape(L, H, tc, d)
    out["kq"] = int(np.sum(kq[:, :, :T] != ref.kq[:, :, :T]))
    vn = buf[lay.vn:lay.vn + L * H * tc * 4].view(np.uint32).reshape(L, H, tc)
    out["vn"] = int(np.sum(vn[:, :, :T] != ref.vn[:, :, :T].view(np.uint32)))
    ks = buf[lay.ks:lay.ks + ref.ks.nbytes].view(np.uint32).reshape(ref.ks.shape)
    if lay.k_scale == pool_image.K_TENSOR:
        out["ks"] = int(np.sum(ks[:, :T] != ref.ks[:, :T].view(np.uint32)))
    elif lay.k_scale == pool_image.K_TOKEN:
        out["ks"] = int(np.sum(ks[:, :, :T] != ref.ks[:, :, :T].view(np.uint32)))
    else:
        out["ks"] = int(np.sum(ks != ref.ks.view(np.uint32)))
    vmax = buf[lay.vmax:lay.vmax + L * H * 4].view(np.uint32).reshape(L, H)
    out["vmax"] = int(np.sum(vmax != ref.vmax.view(np.uint32)))
    ngrp = (T + 7) // 8
    bad = 0
    for l in range(L):
        b = lay.bits[l]
        vc = buf[lay.vc[l]:lay.vc[l + 1]].reshape(H, tc // 8, d * b)
        bad += int(np.sum(vc[:, :ngrp] != ref.packed_codes(l)[:, :ngrp]))
    out["vc"] = bad
    return out


def make_queries(w, step, agents):
    """[A][L][Hq][d] device queries and their fp32 values for one decode step."""
    qs = [w.queries(step, a) for a in agents]
    dev = torch.stack([to_device(t) for t in qs]).contiguous()
    return dev, np.stack([t.f32 for t in qs])


def make_suffix(w, agents, layers):
    """Device suffix K/V [A][L][Hkv][S_cap][d] and host fp32 lookups by (agent index, layer)."""
    ks = [[w.sfx_k(a, l) for l in range(layers)] for a in agents]
    vs = [[w.sfx_v(a, l) for l in range(layers)] for a in agents]
    kd = torch.stack([torch.stack([to_device(t) for t in row]) for row in ks]).contiguous()
    vd = torch.stack([torch.stack([to_device(t) for t in row]) for row in vs]).contiguous()
    return kd, vd, (lambda i, l: ks[i][l].f32), (lambda i, l: vs[i][l].f32)


def run_decode(pools, q, sfx=None, sfx_len=None, layer_begin=0, kernel=pk.KERNEL_DEFAULT, splits=0):
    A, lc, hq, d = q.shape
    out = torch.full((A, lc, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    sk = sv = None
    if sfx is not None:
        sk, sv = sfx
    ws_bytes = pk.agent_decode_attention(pools, q, out, layer_begin, sk, sv, sfx_len, kernel=kernel, splits=splits)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    pk.agent_decode_attention(pools, q, out, layer_begin, sk, sv, sfx_len, workspace=ws, kernel=kernel, splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_decode(q_f32, pool_of_agent, refs, sfx_k, sfx_v, sfx_len, n_kv_heads, layer_begin=0):
    """fp64 oracle outputs [A][L][Hq][d] for agents whose pools are refs[pool_of_agent[a]]."""
    return attention.decode_call(
        q_f32, pool_of_agent,
        decoded=lambda p, l, g: refs[p].decoded_layer(layer_begin + l, g),
        k_sfx=sfx_k, v_sfx=sfx_v, sfx_len=sfx_len, n_kv_heads=n_kv_heads)

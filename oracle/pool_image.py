"""Byte layout of one shared pool, and an image builder that fills it.

PolyKV explainer, section 2.A (SharedKVPool): the shared context is encoded
once into one object; its memory does not depend on how many agents read it.
Section 4 (memory efficiency) reports the pool as constant in the agent count.

The layout is a choice made here (the pages give none).  For a pool of
L layers, Hkv kv heads, head dim d, capacity rounded up to tc (a multiple of
32 tokens) and per-layer V bit widths b_l, regions follow each other in this
order, each starting on a 256-byte boundary:

  Kq    int8  [L][Hkv][tc][d]         K codes
  Vn    f32   [L][Hkv][tc]            V norms
  Ks    f32   K scales, by the pool's K-scale granularity:
              per tensor  [L][tc]       the scale of the append block holding each token
              per token   [L][Hkv][tc]  one scale per stored K vector
              per channel [L][Hkv][d]   one scale per channel, from the first append
  Vmax  f32   [L][Hkv]                max V norm over the tokens in the pool
  Vc    u8    per layer l: [Hkv][tc/8][d * b_l]   packed V code groups
  amax  u32   [L] ([L][Hkv][d] per channel)   scratch of the quantiser (not part of the image)

K-scale granularities and the corrected V norm are codec variants measured as
ablations (the pages name the per-tensor scale and a per-vector norm).

A kv-head shard (``PoolImage.shard``) is the same pool restricted to a range
of kv heads: the per-head regions keep only those heads, per-tensor K scales
(one per token, shared by the heads) stay whole, per-token and per-channel ones
(per head) keep those heads, and the token counts are unchanged.
This is the layout-level definition the device copy must reproduce; each
(layer, kv head) decodes exactly as in the whole pool.

A later append writes new tokens after the existing ones and never rewrites
the codes, norms or scales of earlier tokens (CoMixKV news article,
"incremental quantization strategy": quantised blocks are not re-quantised);
each append is its own per-tensor K block with its own scale.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import codec

ALIGN = 256
TOKEN_ROUND = 32
K_TENSOR, K_TOKEN, K_CHANNEL = 0, 1, 2


def _align(x: int) -> int:
    return (x + ALIGN - 1) // ALIGN * ALIGN


@dataclass
class Layout:
    n_layers: int
    n_kv_heads: int
    head_dim: int
    capacity: int
    tc: int
    bits: tuple
    kq: int
    vn: int
    ks: int
    vmax: int
    vc: list = field(default_factory=list)  # L + 1 offsets; vc[L] = end of codes
    amax: int = 0
    total: int = 0
    k_scale: int = K_TENSOR

    def vc_group_bytes(self, layer: int) -> int:
        return self.head_dim * int(self.bits[layer])


def layout(n_layers: int, n_kv_heads: int, head_dim: int, capacity: int, bits, k_scale: int = K_TENSOR) -> Layout:
    bits = tuple(int(b) for b in bits)
    if len(bits) != n_layers:
        raise ValueError("one bit width per layer")
    tc = (capacity + TOKEN_ROUND - 1) // TOKEN_ROUND * TOKEN_ROUND
    L, H, d = n_layers, n_kv_heads, head_dim
    ks_bytes = {K_TENSOR: L * tc * 4, K_TOKEN: L * H * tc * 4, K_CHANNEL: L * H * d * 4}[k_scale]
    kq = 0
    vn = _align(kq + L * H * tc * d)
    ks = _align(vn + L * H * tc * 4)
    vmax = _align(ks + ks_bytes)
    vc = [_align(vmax + L * H * 4)]
    for b in bits:
        vc.append(vc[-1] + H * tc * d * b // 8)
    amax = _align(vc[-1])
    total = _align(amax + (L * H * d * 4 if k_scale == K_CHANNEL else L * 4))
    return Layout(L, H, d, capacity, tc, bits, kq, vn, ks, vmax, vc, amax, total, k_scale)


def bf16_kv_bytes(n_layers: int, n_kv_heads: int, head_dim: int, tokens: int) -> int:
    """bf16 K+V cache bytes of one agent: 2 (K and V) * tokens * Hkv * d * layers * 2 bytes.

    QKVShare blog, section 2.1 (KV cache size formula), with the hidden size
    replaced by Hkv * d for grouped-query attention.
    """
    return 2 * tokens * n_kv_heads * head_dim * n_layers * 2


class PoolImage:
    """Host model of one pool: encodes appends and writes the image bytes."""

    def __init__(self, n_layers, n_kv_heads, head_dim, capacity, bits, signs=None, k_scale=K_TENSOR,
                 corrected_norm=False):
        """signs: optional [head_dim] +1 / -1 of the randomised rotation (None: plain FWHT).
        k_scale: K_TENSOR (the pages' per-tensor scale), K_TOKEN or K_CHANNEL.
        corrected_norm: store ||v|| sqrt(d) / ||c_hat|| as the V norm (``codec.v_encode``)."""
        self.signs = None if signs is None else np.asarray(signs, dtype=np.float64)
        self.corrected_norm = bool(corrected_norm)
        self.lay = layout(n_layers, n_kv_heads, head_dim, capacity, bits, k_scale)
        L, H, d, tc = n_layers, n_kv_heads, head_dim, self.lay.tc
        self.n_tokens = np.zeros(L, dtype=np.int64)
        self.kq = np.zeros((L, H, tc, d), dtype=np.int8)
        self.vn = np.zeros((L, H, tc), dtype=np.float32)
        self.ks = np.zeros({K_TENSOR: (L, tc), K_TOKEN: (L, H, tc), K_CHANNEL: (L, H, d)}[k_scale], dtype=np.float32)
        self.vmax = np.zeros((L, H), dtype=np.float32)
        self.codes = np.zeros((L, H, tc, d), dtype=np.uint8)

    def append(self, layer_begin: int, k: np.ndarray, v: np.ndarray) -> None:
        """Quantise k, v [nl][Hkv][n][d] (fp32 values) into layers layer_begin.. ."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        nl, H, n, d = k.shape
        for j in range(nl):
            l = layer_begin + j
            t0 = int(self.n_tokens[l])
            if t0 + n > self.lay.capacity:
                raise ValueError("append beyond capacity")
            mode = self.lay.k_scale
            if mode == K_TENSOR:
                s, q = codec.k_quantize(k[j])
                self.ks[l, t0:t0 + n] = s
            elif mode == K_TOKEN:
                s, q = codec.k_quantize_per_token(k[j])
                self.ks[l, :, t0:t0 + n] = s
            else:
                if t0 == 0:  # the first append fixes the channel scales
                    self.ks[l] = codec.k_channel_scales(k[j])
                q = codec.k_quantize_per_channel(k[j], self.ks[l])
            self.kq[l, :, t0:t0 + n] = q
            nrm, codes = codec.v_encode(v[j], self.lay.bits[l], self.signs, self.corrected_norm)
            self.vn[l, :, t0:t0 + n] = nrm
            if n:
                self.vmax[l] = np.maximum(self.vmax[l], nrm.max(axis=1))
            self.codes[l, :, t0:t0 + n] = codes
            self.n_tokens[l] = t0 + n

    def packed_codes(self, layer: int) -> np.ndarray:
        """Packed code groups of one layer, [Hkv][tc/8][d * b] bytes."""
        return codec.pack_codes(self.codes[layer], self.lay.bits[layer])

    def image(self) -> np.ndarray:
        """The whole pool image as bytes; the quantiser scratch region is zero."""
        lay = self.lay
        buf = np.zeros(lay.total, dtype=np.uint8)
        buf[lay.kq:lay.kq + self.kq.nbytes] = self.kq.reshape(-1).view(np.uint8)
        buf[lay.vn:lay.vn + self.vn.nbytes] = self.vn.reshape(-1).view(np.uint8)
        buf[lay.ks:lay.ks + self.ks.nbytes] = self.ks.reshape(-1).view(np.uint8)
        buf[lay.vmax:lay.vmax + self.vmax.nbytes] = self.vmax.reshape(-1).view(np.uint8)
        for l in range(lay.n_layers):
            p = self.packed_codes(l).reshape(-1)
            buf[lay.vc[l]:lay.vc[l] + p.size] = p
        return buf

    def decoded_layer(self, layer: int, kv_head: int) -> tuple[np.ndarray, np.ndarray]:
        """(K_hat, V_hat) [T][d] in fp64 for the tokens in the pool."""
        t = int(self.n_tokens[layer])
        if self.lay.k_scale == K_TENSOR:
            sc = self.ks[layer, :t, None]
        elif self.lay.k_scale == K_TOKEN:
            sc = self.ks[layer, kv_head, :t, None]
        else:
            sc = self.ks[layer, kv_head][None, :]
        khat = sc.astype(np.float64) * self.kq[layer, kv_head, :t].astype(np.float64)
        vhat = codec.v_decode(self.vn[layer, kv_head, :t], self.codes[layer, kv_head, :t], self.lay.bits[layer],
                              self.signs)
        return khat, vhat

    def shard(self, head_begin: int, head_count: int) -> "PoolImage":
        """The pool restricted to kv heads [head_begin, head_begin + head_count)."""
        lay = self.lay
        if head_begin < 0 or head_count < 1 or head_begin + head_count > lay.n_kv_heads:
            raise ValueError("head range")
        out = PoolImage(lay.n_layers, head_count, lay.head_dim, lay.capacity, lay.bits, self.signs, lay.k_scale,
                        self.corrected_norm)
        sl = slice(head_begin, head_begin + head_count)
        out.n_tokens = self.n_tokens.copy()
        out.kq = self.kq[:, sl].copy()
        out.vn = self.vn[:, sl].copy()
        out.ks = self.ks.copy() if lay.k_scale == K_TENSOR else self.ks[:, sl].copy()
        out.vmax = self.vmax[:, sl].copy()
        out.codes = self.codes[:, sl].copy()
        return out

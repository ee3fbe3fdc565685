"""Seeded synthetic inputs for the shared compressed-KV decode path.

This module holds only shapes and random draws.  It contains none of the
method's arithmetic: no quantisation, no rotation, no attention.  The CPU
oracle's tests and the GPU path both read the arrays it makes, so they see
identical inputs.

Every slice is drawn from its own PCG64 stream, keyed by
``SeedSequence(seed, spawn_key=(tensor_id, i, j))``.  Any single (pool, layer)
or (agent, layer) slice can therefore be regenerated on its own, which is
what lets full-size parity checks recompute one sampled output at a time.

Value recipes (one per workload family), standing in for the K/V statistics of
trained models that are not available here:

* ``gauss_outlier_k``: K, V, Q ~ N(0, 1) in fp32; two K channels, chosen
  per layer, are multiplied by 8.
* ``outlier_channels``: K, V ~ N(0, 1) in bf16; per layer,
  round(1% of n_kv_heads * head_dim) (head, channel) pairs are multiplied by 10,
  chosen separately for K and V; suffix tokens share the layer's channels.
* ``lognormal_channels``: K, V = N(0, 1) * sigma with
  sigma ~ LogNormal(0, 0.5) i.i.d. per (layer, kv head, channel), separately
  for K and V; suffix tokens share sigma.

Queries are N(0, 1) in every family (fp32 or bf16 as the workload states).
bf16 values are made by round-to-nearest-even from fp32 draws.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

# Stable stream identifiers, one per named tensor.
TENSOR_IDS = {
    "k_pool": 0,
    "v_pool": 1,
    "k_mod": 2,
    "v_mod": 3,
    "sfx_k": 4,
    "sfx_v": 5,
    "q_steps": 6,
    "v_bits": 7,
    "v_signs": 8,
}


def rotation_signs(seed: int, head_dim: int, key: int = 0) -> np.ndarray:
    """[head_dim] +1 / -1 (each with probability 1/2): the sign vector of a randomised V rotation."""
    return np.where(rng_for(seed, "v_signs", key).random(head_dim) < 0.5, -1.0, 1.0)


def rng_for(seed: int, tensor: str, *key: int) -> np.random.Generator:
    """PCG64 generator for one named tensor slice."""
    ss = np.random.SeedSequence(seed, spawn_key=(TENSOR_IDS[tensor],) + tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite (the generators never draw NaN or Inf).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Tensor:
    """A drawn tensor: fp32 values plus the raw storage handed to the device.

    ``raw`` is the fp32 array itself for fp32 workloads and the uint16 bf16 bit
    pattern for bf16 workloads; ``f32`` holds exactly the stored values.
    """

    f32: np.ndarray
    raw: np.ndarray
    dtype: str  # "f32" | "bf16"


def _make(x: np.ndarray, dtype: str) -> Tensor:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return Tensor(x, x, "f32")
    bits = f32_to_bf16_bits(x)
    return Tensor(bf16_bits_to_f32(bits), bits, "bf16")


@dataclass(frozen=True)
class Workload:
    """Shapes and value recipe of one synthetic multi-agent decode workload."""

    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    pool_tokens: int  # T: tokens in each shared compressed pool
    n_agents: int
    n_pools: int  # 1 = every agent shares one pool; n_agents = one pool per agent
    steps: int  # decode steps
    sfx_mode: str  # "none" | "grow" (length s+1 at step s) | "fixed" (sfx_tokens every step)
    sfx_tokens: int  # suffix capacity per agent
    dtype: str  # storage dtype of K, V, Q: "f32" | "bf16"
    dist: str  # "gauss_outlier_k" | "outlier_channels" | "lognormal_channels"
    v_bits_mode: str  # "uniform3" | "mixed"
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def pool_of_agent(self, a: int) -> int:
        return 0 if self.n_pools == 1 else a

    def agents_of_pool(self, p: int) -> list[int]:
        return [a for a in range(self.n_agents) if self.pool_of_agent(a) == p]

    def sfx_len(self, step: int) -> int:
        if self.sfx_mode == "none":
            return 0
        if self.sfx_mode == "grow":
            return min(step + 1, self.sfx_tokens)
        return self.sfx_tokens

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # ---- channel modifiers (model statistics, shared by every pool/agent) ----
    def _channel_scale(self, which: str, layer: int) -> np.ndarray:
        """Per (kv head, channel) multiplier for K or V of one layer, [Hkv][d] fp32."""
        hkv, d = self.n_kv_heads, self.head_dim
        rng = rng_for(self.seed, "k_mod" if which == "k" else "v_mod", layer)
        s = np.ones(hkv * d, dtype=np.float32)
        if self.dist == "gauss_outlier_k":
            if which == "k":
                s[rng.choice(hkv * d, size=2, replace=False)] = 8.0
        elif self.dist == "outlier_channels":
            n_out = int(round(0.01 * hkv * d))
            s[rng.choice(hkv * d, size=n_out, replace=False)] = 10.0
        elif self.dist == "lognormal_channels":
            s = rng.lognormal(mean=0.0, sigma=0.5, size=hkv * d).astype(np.float32)
        else:
            raise ValueError(f"unknown dist {self.dist}")
        return s.reshape(hkv, d)

    def _draw(self, tensor: str, which: str, key: tuple, n_tok: int, layer: int) -> Tensor:
        rng = rng_for(self.seed, tensor, *key)
        x = rng.standard_normal((self.n_kv_heads, n_tok, self.head_dim), dtype=np.float32)
        x *= self._channel_scale(which, layer)[:, None, :]
        return _make(x, self.dtype)

    # ---- public draws ----
    def pool_k(self, pool: int, layer: int) -> Tensor:
        """Shared-context K of one pool layer, [Hkv][T][d]."""
        return self._draw("k_pool", "k", (pool, layer), self.pool_tokens, layer)

    def pool_v(self, pool: int, layer: int) -> Tensor:
        """Shared-context V of one pool layer, [Hkv][T][d]."""
        return self._draw("v_pool", "v", (pool, layer), self.pool_tokens, layer)

    def sfx_k(self, agent: int, layer: int) -> Tensor:
        """Agent-private native K of one layer, [Hkv][S_cap][d]."""
        return self._draw("sfx_k", "k", (agent, layer), self.sfx_tokens, layer)

    def sfx_v(self, agent: int, layer: int) -> Tensor:
        return self._draw("sfx_v", "v", (agent, layer), self.sfx_tokens, layer)

    def queries(self, step: int, agent: int) -> Tensor:
        """Decode queries of one agent at one step, [L][Hq][d]."""
        rng = rng_for(self.seed, "q_steps", step, agent)
        x = rng.standard_normal((self.n_layers, self.n_q_heads, self.head_dim), dtype=np.float32)
        return _make(x, self.dtype)

    def v_bits(self, pool: int) -> np.ndarray:
        """V bit-width per layer of one pool, [L] uint8 in {2, 3, 4}."""
        L = self.n_layers
        if self.v_bits_mode == "uniform3":
            return np.full(L, 3, dtype=np.uint8)
        if self.v_bits_mode != "mixed":
            raise ValueError(self.v_bits_mode)
        a = int(round(L / 3))
        b = L - 2 * a  # equal numbers of 2- and 4-bit layers: mean is exactly 3
        base = np.array([2] * a + [3] * b + [4] * a, dtype=np.uint8)
        return rng_for(self.seed, "v_bits", pool).permutation(base)


# ---- the five workloads (shapes of the models named, synthetic values) ----
TINY = Workload("tiny_L1_H1_d64_T512_A4", n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=64,
                pool_tokens=512, n_agents=4, n_pools=1, steps=1, sfx_mode="none", sfx_tokens=0,
                dtype="f32", dist="gauss_outlier_k", v_bits_mode="uniform3")
SMOLLM2 = Workload("smollm2_1.7b_L24_H32_d64_T1851_A3", n_layers=24, n_q_heads=32, n_kv_heads=32,
                   head_dim=64, pool_tokens=1851, n_agents=3, n_pools=1, steps=64, sfx_mode="grow",
                   sfx_tokens=64, dtype="bf16", dist="outlier_channels", v_bits_mode="uniform3")
LLAMA3_8B = Workload("llama3_8b_L32_Hq32_Hkv8_d128_T4096_A15", n_layers=32, n_q_heads=32, n_kv_heads=8,
                     head_dim=128, pool_tokens=4096, n_agents=15, n_pools=1, steps=128, sfx_mode="grow",
                     sfx_tokens=128, dtype="bf16", dist="lognormal_channels", v_bits_mode="uniform3")
LLAMA3_8B_LONG = Workload("llama3_8b_long_L32_Hq32_Hkv8_d128_T7194_S256_A15", n_layers=32, n_q_heads=32,
                          n_kv_heads=8, head_dim=128, pool_tokens=7194, n_agents=15, n_pools=1, steps=32,
                          sfx_mode="fixed", sfx_tokens=256, dtype="bf16", dist="lognormal_channels",
                          v_bits_mode="uniform3")
QWEN3_32B_MIXED = Workload("qwen3_32b_comix_L64_Hq64_Hkv8_d128_T8064_S128_A8", n_layers=64, n_q_heads=64,
                           n_kv_heads=8, head_dim=128, pool_tokens=8064, n_agents=8, n_pools=8, steps=16,
                           sfx_mode="fixed", sfx_tokens=128, dtype="bf16", dist="lognormal_channels",
                           v_bits_mode="mixed")

ALL = [TINY, SMOLLM2, LLAMA3_8B, LLAMA3_8B_LONG, QWEN3_32B_MIXED]
BY_NAME = {w.name: w for w in ALL}

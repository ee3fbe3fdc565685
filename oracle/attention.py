"""fp64 decode attention over a decoded shared pool plus each agent's native suffix.

PolyKV explainer, section 2.A (PooledAgent): every agent attends to the shared
pool's decoded K/V; the agent's own new tokens accumulate in its private cache.
CoMixKV news article ("incremental quantization strategy"): the most recent
states stay at native precision.  Readings (the pages state no attention
details, so standard decode attention is used):

* sigma = 1 / sqrt(d) unless given; no mask at decode (the query sees every
  pool token and every token of its own suffix);
* grouped-query attention maps q head h to kv head floor(h / G), G = Hq / Hkv
  (contiguous groups);
* o = softmax(sigma * q . [K_hat; K_sfx]) @ [V_hat; V_sfx], all in fp64;
* an agent with a private compressed segment (its own older tokens, quantized
  once when they left the native window: the incremental quantization the
  CoMixKV article describes) attends to the shared pool, then that segment,
  then its native suffix: the three token sets are concatenated.

``rotated_form`` writes the same output the way the GPU accumulates it: the
pool part of the value sum stays in the rotated, normalised domain,
acc = sum_t p_t n_t c[code_t], and one inverse transform is applied at the
end, o = (H @ acc) / d + sum_u p_u v_u.  It is used only to check that the
two forms agree (they are equal in exact arithmetic because H is linear).
"""
from __future__ import annotations

import math

import numpy as np

from . import hadamard, lloyd_max


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, sigma: float | None = None) -> np.ndarray:
    """Softmax attention of query rows q [R][d] over keys k [T][d] and values v [T][d], fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    if sigma is None:
        sigma = 1.0 / math.sqrt(d)
    s = sigma * (q @ k.T)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v


def attend_pool_and_suffix(q, khat, vhat, k_sfx=None, v_sfx=None, sigma=None) -> np.ndarray:
    """Attention of q [R][d] over the decoded pool tokens followed by native suffix tokens."""
    k = np.asarray(khat, dtype=np.float64)
    v = np.asarray(vhat, dtype=np.float64)
    if k_sfx is not None and len(k_sfx):
        k = np.concatenate([k, np.asarray(k_sfx, dtype=np.float64)], axis=0)
        v = np.concatenate([v, np.asarray(v_sfx, dtype=np.float64)], axis=0)
    return attend(q, k, v, sigma)


def rotated_form(q, k_scale, k_codes, v_norm, v_codes, bits, k_sfx=None, v_sfx=None, sigma=None):
    """Same output as ``attend_pool_and_suffix`` on the decoded pool, via one inverse FWHT."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    if sigma is None:
        sigma = 1.0 / math.sqrt(d)
    khat = np.asarray(k_scale, dtype=np.float64)[:, None] * np.asarray(k_codes, dtype=np.float64)
    cent, _ = lloyd_max.table_f32(bits)
    c = cent.astype(np.float64)[np.asarray(v_codes, dtype=np.int64)]  # [T][d]
    s_pool = sigma * (q @ khat.T)
    parts = [s_pool]
    if k_sfx is not None and len(k_sfx):
        parts.append(sigma * (q @ np.asarray(k_sfx, dtype=np.float64).T))
    s = np.concatenate(parts, axis=-1)
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=-1, keepdims=True)
    t = khat.shape[0]
    acc = (p[:, :t] * np.asarray(v_norm, dtype=np.float64)[None, :]) @ c
    h = hadamard.hadamard_matrix(d).astype(np.float64)
    o = (acc @ h) / d
    if t < s.shape[-1]:
        o = o + p[:, t:] @ np.asarray(v_sfx, dtype=np.float64)
    return o / l


def decode_call(queries, pool_of_agent, decoded, k_sfx, v_sfx, sfx_len, n_kv_heads, sigma=None,
                private=None):
    """Outputs of one decode call for every (agent, layer, q head), fp64.

    queries    [A][L][Hq][d] query values
    pool_of_agent[a]  pool id of agent a
    decoded    callable (pool, layer, kv_head) -> (K_hat [T][d], V_hat [T][d])
    k_sfx, v_sfx  callables (agent, layer) -> [Hkv][S_cap][d] native suffix values (or None)
    sfx_len[a] suffix tokens agent a attends to
    private    optional callable (agent, layer, kv_head) -> (K_hat, V_hat) of the agent's
               private segment, or None for an agent without one
    Returns [A][L][Hq][d].
    """
    q = np.asarray(queries, dtype=np.float64)
    A, L, Hq, d = q.shape
    G = Hq // n_kv_heads
    out = np.zeros_like(q)
    for a in range(A):
        for l in range(L):
            ks = vs = None
            if sfx_len[a] > 0:
                ks = k_sfx(a, l)
                vs = v_sfx(a, l)
            for g in range(n_kv_heads):
                khat, vhat = decoded(pool_of_agent[a], l, g)
                seg = private(a, l, g) if private is not None else None
                if seg is not None:
                    khat = np.concatenate([np.asarray(khat, dtype=np.float64), np.asarray(seg[0], dtype=np.float64)])
                    vhat = np.concatenate([np.asarray(vhat, dtype=np.float64), np.asarray(seg[1], dtype=np.float64)])
                kk = None if ks is None else ks[g, :sfx_len[a]]
                vv = None if vs is None else vs[g, :sfx_len[a]]
                out[a, l, g * G:(g + 1) * G] = attend_pool_and_suffix(q[a, l, g * G:(g + 1) * G], khat, vhat,
                                                                      kk, vv, sigma)
    return out


def max_rel_error(out: np.ndarray, ref: np.ndarray) -> float:
    """max over output vectors of ||out - ref||_inf / max(||ref||_inf, 1e-6)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-6)
    return float(np.max(num / den)) if num.size else 0.0

"""K and V codecs of the shared pool, in exactly specified fp32 arithmetic.

PolyKV explainer, section 2.B (asymmetric compression scheme):

* K is stored as int8 under a per-tensor linear scale ("q8_0" formula).
  Readings: symmetric, no zero point, codes in [-127, 127];
  scale s = amax / 127 (one correctly rounded fp32 division), where amax is the
  max |k| over the whole tensor quantised together (all kv heads, tokens and
  channels of one layer in one append); q = clamp(rint(k / s), -127, 127) with
  k / s one correctly rounded fp32 division and rint rounding half to even;
  amax == 0 gives s = 0 and all codes 0.  Dequantisation: k_hat = s * q.
* V is rotated by the FWHT, normalised so the rotated coordinates are
  approximately N(0, 1), and each coordinate is replaced by the index of its
  Lloyd-Max cell.  Readings: the stored per-vector norm is the plain L2 norm
  n = ||v|| (halving-tree fp32 sum, correctly rounded sqrt); y = (H v) * r with
  r = 1 / n (one correctly rounded fp32 division) and H unnormalised, so that
  sum(y^2) = d; code_i = #{j : y_i > tau_j} (strict, so a tie takes the lower
  code); n == 0 gives all codes 0.  Dequantisation (section 2.B, inverse FWHT):
  v_hat = (n / d) * H @ c[code], exact in fp64.
* CoMixKV news article ("incremental quantization strategy"; abstract): the V
  bit width is 2, 3 or 4 per (agent, layer); K stays int8.
* Randomised rotation (a codec variant measured as an ablation; the pages name
  only the plain FWHT): with a sign vector s in {+1, -1}^d, the rotation is H D
  (D = diag(s)): x is multiplied by s before the transform, and the decoded
  vector by s after the inverse transform, v_hat = s * (n / d) H c[code].  The
  norm is unchanged (squares do not see signs), and s = all +1 is the plain
  codec.  The signs are an input (chosen by the caller), not drawn here.

Code-group packing (the layout the decode kernels read).  Tokens of one
(layer, kv head) are packed in groups of 8 consecutive tokens.  A group of
d-dimensional codes at ``bits`` bits takes d * bits bytes: for each dimension
delta in natural order, one little-endian (8 * bits)-bit field holding the 8
tokens' codes, token i in bits [bits * i, bits * (i + 1)).  At 3 bits that is
8 codes in 3 bytes.  Bits of tokens that are not (yet) in the pool are zero.
"""
from __future__ import annotations

import numpy as np

from . import hadamard, lloyd_max

GROUP_TOKENS = 8


# ---------------------------------------------------------------- K codec
def k_quantize(k: np.ndarray) -> tuple[np.float32, np.ndarray]:
    """Per-tensor symmetric int8 quantisation of one K tensor (any shape, fp32 values).

    Returns (scale, codes) with codes int8 of the same shape.
    """
    k = np.asarray(k, dtype=np.float32)
    amax = np.float32(np.max(np.abs(k))) if k.size else np.float32(0.0)
    if amax == 0.0:
        return np.float32(0.0), np.zeros(k.shape, dtype=np.int8)
    s = np.float32(amax / np.float32(127.0))
    q = np.rint(k / s)  # fp32 division, then round half to even
    q = np.clip(q, -127.0, 127.0).astype(np.int8)
    return s, q


def k_quantize_per_token(k: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-token int8 quantisation of K vectors (last axis = head_dim): one scale per vector.

    A codec variant measured as an ablation (QKVShare blog, section 3.2, weighs per-tensor
    against per-token and per-channel granularity; PolyKV explainer, section 2.B, names only
    the per-tensor scale).  The q8_0 rule of ``k_quantize`` applied to each vector alone:
    s_t = fl(amax_t / 127) with amax_t = max_i |k_t,i|, q = clamp(rint(fl(k / s_t)), -127, 127),
    a zero vector gives s_t = 0 and codes 0.  Returns (scales [...], codes int8 [..., d]).
    """
    k = np.asarray(k, dtype=np.float32)
    amax = np.max(np.abs(k), axis=-1) if k.shape[-1] else np.zeros(k.shape[:-1], np.float32)
    s = (amax / np.float32(127.0)).astype(np.float32)
    nz = s > 0
    q = np.zeros(k.shape, dtype=np.float32)
    q[nz] = np.rint(k[nz] / s[nz][..., None])
    return s, np.clip(q, -127.0, 127.0).astype(np.int8)


def k_channel_scales(k: np.ndarray) -> np.ndarray:
    """Per-channel K scales of one block [..., T, d]: s_c = fl(max_t |k_t,c| / 127), shape [..., d]."""
    k = np.asarray(k, dtype=np.float32)
    amax = np.max(np.abs(k), axis=-2) if k.shape[-2] else np.zeros(k.shape[:-2] + k.shape[-1:], np.float32)
    return (amax / np.float32(127.0)).astype(np.float32)


def k_quantize_per_channel(k: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """int8 codes of K [..., T, d] under given per-channel scales [..., d] (a codec variant).

    q = clamp(rint(fl(k / s_c)), -127, 127); a channel with s_c = 0 gives codes 0.  The scales
    of a pool are taken from its first append (``k_channel_scales``) and kept: later tokens
    are coded with them and clamp at +-127, since stored codes are never re-quantised (CoMixKV
    news article, "incremental quantization strategy").
    """
    k = np.asarray(k, dtype=np.float32)
    s = np.broadcast_to(np.asarray(scales, dtype=np.float32)[..., None, :], k.shape)
    q = np.zeros(k.shape, dtype=np.float32)
    nz = s > 0
    q[nz] = np.rint(k[nz] / s[nz])
    return np.clip(q, -127.0, 127.0).astype(np.int8)


def k_dequantize(scale, q: np.ndarray) -> np.ndarray:
    """k_hat = scale * q, exact in fp64."""
    return np.float64(scale) * np.asarray(q, dtype=np.float64)


# ---------------------------------------------------------------- V codec
def v_encode(v: np.ndarray, bits: int, signs: np.ndarray | None = None,
             corrected_norm: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """Encode V vectors (last axis = head_dim) to (norms fp32, codes uint8).

    signs: optional [d] array of +1 / -1 applied to each vector before the FWHT.
    corrected_norm: store n' = ||v|| sqrt(d) / ||c_hat|| instead of ||v|| (a codec variant
    measured as an ablation), so that the decoded vector (n'/d) H c_hat has exactly the input's
    norm (||H c|| = sqrt(d) ||c||).  In fp32: cn = sqrt of the centroids' squares summed by
    the same halving tree as the norm, n' = fl(fl(n * fl(sqrt(d))) / cn); the codes are the
    plain codec's (found with 1/||v||); a zero vector keeps n' = 0.
    """
    x = np.asarray(v, dtype=np.float32)
    _, thr = lloyd_max.table_f32(bits)
    n = hadamard.norm_f32(x)
    if signs is not None:
        x = x * np.asarray(signs, dtype=np.float32)  # exact: sign flips
    z = hadamard.fwht_f32(x)
    nz = n > 0
    r = np.zeros_like(n)
    r[nz] = np.float32(1.0) / n[nz]  # fp32 division
    y = z * r[..., None]  # fp32 multiply
    codes = np.zeros(x.shape, dtype=np.uint8)
    for t in thr:
        codes += (y > t).astype(np.uint8)
    codes[~nz] = 0
    if corrected_norm:
        cent, _ = lloyd_max.table_f32(bits)
        cn = hadamard.norm_f32(cent[codes])
        sd = np.float32(np.sqrt(np.float64(x.shape[-1])))
        n = ((n * sd).astype(np.float32) / cn).astype(np.float32)
        n[~nz] = 0.0
    return n, codes


def v_decode(norm: np.ndarray, codes: np.ndarray, bits: int, signs: np.ndarray | None = None) -> np.ndarray:
    """v_hat = s * (n / d) * H @ c[code] in fp64 (inverse FWHT of the centroid vector)."""
    cent, _ = lloyd_max.table_f32(bits)
    c = cent.astype(np.float64)[np.asarray(codes, dtype=np.int64)]
    d = c.shape[-1]
    h = hadamard.hadamard_matrix(d).astype(np.float64)
    out = (np.asarray(norm, dtype=np.float64)[..., None] / d) * (c @ h)
    if signs is not None:
        out = out * np.asarray(signs, dtype=np.float64)
    return out


def signs_from_mask(mask: bytes | np.ndarray, d: int) -> np.ndarray:
    """[d] +1 / -1 from a little-endian bit mask (bit i set: dimension i negated)."""
    b = np.unpackbits(np.frombuffer(bytes(mask), dtype=np.uint8), bitorder="little")[:d]
    return np.where(b == 1, -1.0, 1.0)


# ---------------------------------------------------------------- packing
def pack_group(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack one group of codes [8][d] into d * bits bytes (layout in the module doc)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[0] != GROUP_TOKENS:
        raise ValueError("a group holds 8 tokens")
    d = codes.shape[1]
    out = bytearray()
    for delta in range(d):
        field = 0
        for i in range(GROUP_TOKENS):
            field |= int(codes[i, delta]) << (bits * i)
        out += field.to_bytes(bits, "little")
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [..., T][d] (T a multiple of 8) into [..., T/8][d * bits] bytes.

    Vectorised form of ``pack_group`` over leading axes and groups.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    *lead, t, d = codes.shape
    if t % GROUP_TOKENS:
        raise ValueError("token count must be a multiple of 8")
    g = codes.reshape(*lead, t // GROUP_TOKENS, GROUP_TOKENS, d).astype(np.uint32)
    field = np.zeros((*lead, t // GROUP_TOKENS, d), dtype=np.uint32)
    for i in range(GROUP_TOKENS):
        field |= g[..., i, :] << np.uint32(bits * i)
    le = field.astype("<u4").view(np.uint8).reshape(*lead, t // GROUP_TOKENS, d, 4)
    return np.ascontiguousarray(le[..., :bits]).reshape(*lead, t // GROUP_TOKENS, d * bits)


def unpack_codes(packed: np.ndarray, d: int, bits: int) -> np.ndarray:
    """Inverse of ``pack_codes``: [..., G][d * bits] bytes -> [..., G * 8][d] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    *lead, ng, nb = packed.shape
    if nb != d * bits:
        raise ValueError("group byte count mismatch")
    by = packed.reshape(*lead, ng, d, bits).astype(np.uint32)
    field = np.zeros((*lead, ng, d), dtype=np.uint32)
    for j in range(bits):
        field |= by[..., j] << np.uint32(8 * j)
    mask = np.uint32((1 << bits) - 1)
    out = np.stack([(field >> np.uint32(bits * i)) & mask for i in range(GROUP_TOKENS)], axis=-2)
    return out.reshape(*lead, ng * GROUP_TOKENS, d).astype(np.uint8)

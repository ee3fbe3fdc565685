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


def k_dequantize(scale, q: np.ndarray) -> np.ndarray:
    """k_hat = scale * q, exact in fp64."""
    return np.float64(scale) * np.asarray(q, dtype=np.float64)


# ---------------------------------------------------------------- V codec
def v_encode(v: np.ndarray, bits: int, signs: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Encode V vectors (last axis = head_dim) to (norms fp32, codes uint8).

    signs: optional [d] array of +1 / -1 applied to each vector before the FWHT.
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

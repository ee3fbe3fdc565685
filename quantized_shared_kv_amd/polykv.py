"""ctypes binding of libpolykv (include/polykv.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it turns torch tensors into device pointers and
dtype codes, checks shapes the C side cannot see, calls the library and raises
``PolyKVError`` on a non-zero return.  There is no fallback: if the built
library is missing, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_uint8, c_uint64, c_void_p

MAX_LAYERS = 128
PKV_F32, PKV_BF16 = 0, 1
ABI_VERSION = 106  # pkv_version() of the library these ctypes mirrors describe
KERNEL_DEFAULT, KERNEL_VALU, KERNEL_MFMA = 0, 1, 2
ERRORS = {0: "PKV_OK", -1: "PKV_EINVAL", -2: "PKV_EUNSUPPORTED", -3: "PKV_ECAPACITY", -4: "PKV_ENOSPACE",
          -5: "PKV_EHIP"}

# PKV_LIBRARY selects another build of the same library (the sanitizer build of the host code)
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib",
                                                         "libpolykv.so")


class PolyKVError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({lib().pkv_strerror(code).decode()})")


KSCALE_TENSOR, KSCALE_TOKEN, KSCALE_CHANNEL = 0, 1, 2
VNORM_PLAIN, VNORM_CORRECTED = 0, 1


class PoolConfig(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("capacity_tokens", c_int32), ("v_bits", c_uint8 * MAX_LAYERS), ("v_signs", c_uint8 * 16),
                ("k_scale", c_uint8), ("v_norm", c_uint8), ("reserved", c_uint8 * 2)]


class Pool(ctypes.Structure):
    _fields_ = [("cfg", PoolConfig), ("base", c_void_p), ("bytes", c_uint64), ("tc", c_int32),
                ("n_tokens", c_int32 * MAX_LAYERS), ("off_kq", c_uint64), ("off_vn", c_uint64),
                ("off_ks", c_uint64), ("off_vmax", c_uint64), ("off_amax", c_uint64),
                ("off_vc", c_uint64 * (MAX_LAYERS + 1))]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("n_agents", c_int32), ("n_q_heads", c_int32), ("layer_begin", c_int32),
                ("layer_count", c_int32), ("softmax_scale", c_float),
                ("agent_pool", POINTER(POINTER(Pool))), ("q", c_void_p), ("q_dtype", c_int32),
                ("sfx_k", c_void_p), ("sfx_v", c_void_p), ("sfx_dtype", c_int32), ("sfx_cap", c_int32),
                ("sfx_len", POINTER(c_int32)), ("out", c_void_p), ("kernel", c_int32), ("splits", c_int32),
                ("pool_events", POINTER(c_void_p)), ("agent_private_pool", POINTER(POINTER(Pool)))]


class ComixArgs(ctypes.Structure):
    _fields_ = [("n_agents", c_int32), ("layer_count", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("softmax_scale", c_float), ("n_recent", c_int32), ("q", c_void_p),
                ("q_dtype", c_int32), ("win_k", c_void_p), ("win_v", c_void_p), ("win_dtype", c_int32),
                ("win_cap", c_int32), ("win_len", POINTER(c_int32)), ("out", c_void_p)]


class PoolHeader(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("abi_version", c_int32), ("cfg", PoolConfig),
                ("n_tokens", c_int32 * MAX_LAYERS), ("image_bytes", c_uint64)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built: run python -m quantized_shared_kv_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.pool_bytes.argtypes = [POINTER(PoolConfig)]
        L.pool_bytes.restype = c_size_t
        L.pool_build.argtypes = [POINTER(PoolConfig), c_void_p, c_size_t, POINTER(Pool)]
        L.pool_build.restype = c_int32
        L.pool_quantize_append.argtypes = [POINTER(Pool), c_int32, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                           c_void_p]
        L.pool_quantize_append.restype = c_int32
        L.agent_decode_attention.argtypes = [POINTER(DecodeArgs), c_void_p, POINTER(c_size_t), c_void_p]
        L.agent_decode_attention.restype = c_int32
        L.agent_decode_attention_noalloc.argtypes = [POINTER(DecodeArgs), c_void_p]
        L.agent_decode_attention_noalloc.restype = c_int32
        L.pkv_noalloc_scratch_bytes.restype = c_size_t
        L.pkv_stream_read.argtypes = [c_void_p, c_size_t, c_void_p, c_void_p]
        L.pkv_stream_read.restype = c_int32
        L.pkv_stream_read_sink_words.restype = c_size_t
        L.pkv_strerror.argtypes = [c_int32]
        L.pkv_strerror.restype = ctypes.c_char_p
        L.pkv_version.restype = c_int32
        L.pkv_abi_sizeof.argtypes = [c_int32]
        L.pkv_abi_sizeof.restype = c_size_t
        L.pkv_lloyd_max_table.argtypes = [c_int32, POINTER(c_float), POINTER(c_float)]
        L.pkv_lloyd_max_table.restype = c_int32
        L.pool_export_header.argtypes = [POINTER(Pool), POINTER(PoolHeader)]
        L.pool_export_header.restype = c_int32
        L.pool_import.argtypes = [POINTER(PoolHeader), c_void_p, c_size_t, POINTER(Pool)]
        L.pool_import.restype = c_int32
        L.pool_shard.argtypes = [POINTER(Pool), c_int32, c_int32, c_void_p, c_size_t, POINTER(Pool), c_void_p]
        L.pool_shard.restype = c_int32
        L.pkv_lloyd_max_distortion.argtypes = [c_int32]
        L.pkv_lloyd_max_distortion.restype = ctypes.c_double
        L.comix_sensitivity.argtypes = [POINTER(ComixArgs), c_void_p]
        L.comix_sensitivity.restype = c_int32
        L.comix_allocate_bits.argtypes = [c_int32, POINTER(c_float), POINTER(c_uint64), POINTER(ctypes.c_double),
                                          c_uint64, POINTER(c_uint8)]
        L.comix_allocate_bits.restype = c_int32
        for i, s in enumerate((PoolConfig, Pool, DecodeArgs, ComixArgs, PoolHeader)):
            if L.pkv_abi_sizeof(i) != ctypes.sizeof(s):
                raise ImportError(f"ABI mismatch for {s.__name__}")
        if L.pkv_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {L.pkv_version()}, this binding expects {ABI_VERSION}: rebuild it")
        _LIB = L
    return _LIB


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise PolyKVError(rc, where)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_config(n_layers: int, n_kv_heads: int, head_dim: int, capacity_tokens: int, v_bits,
                v_signs=None, k_scale: int = KSCALE_TENSOR, v_norm: int = VNORM_PLAIN) -> PoolConfig:
    """v_signs: optional head_dim values, negative (or True) where the V rotation negates a coordinate.
    k_scale: KSCALE_TENSOR / KSCALE_TOKEN / KSCALE_CHANNEL; v_norm: VNORM_PLAIN / VNORM_CORRECTED."""
    cfg = PoolConfig(n_layers, n_kv_heads, head_dim, capacity_tokens)
    cfg.k_scale, cfg.v_norm = k_scale, v_norm
    vb = list(v_bits) if hasattr(v_bits, "__len__") else [int(v_bits)] * n_layers
    for i, b in enumerate(vb):
        cfg.v_bits[i] = int(b)
    if v_signs is not None:
        neg = [bool(x < 0) if not isinstance(x, bool) else x for x in v_signs]
        if len(neg) != head_dim:
            raise ValueError("one sign per head dimension")
        for i, n in enumerate(neg):
            if n:
                cfg.v_signs[i // 8] |= 1 << (i % 8)
    return cfg


def pool_bytes(cfg: PoolConfig) -> int:
    return int(lib().pool_bytes(ctypes.byref(cfg)))


def pool_build(cfg: PoolConfig, dev_ptr: int, dev_bytes: int) -> Pool:
    pool = Pool()
    _check(lib().pool_build(ctypes.byref(cfg), c_void_p(dev_ptr), dev_bytes, ctypes.byref(pool)), "pool_build")
    return pool


def pool_quantize_append(pool: Pool, layer_begin: int, k, v, stream=None) -> None:
    """k, v: device tensors [layer_count][n_kv_heads][n_tokens][head_dim], fp32 or bf16."""
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
        raise ValueError("k and v must be equal-shape 4-D tensors")
    if not (k.is_contiguous() and v.is_contiguous()) or not (k.is_cuda and v.is_cuda):
        raise ValueError("k and v must be contiguous device tensors")
    nl, hkv, n, d = k.shape
    if hkv != pool.cfg.n_kv_heads or d != pool.cfg.head_dim:
        raise ValueError("k/v shape does not match the pool")
    _check(lib().pool_quantize_append(ctypes.byref(pool), layer_begin, nl, c_void_p(k.data_ptr()),
                                      c_void_p(v.data_ptr()), _dtype_code(k), n, c_void_p(_stream_handle(stream))),
           "pool_quantize_append")


def _decode_args(pools, q, out, layer_begin, sfx_k=None, sfx_v=None, sfx_len=None, softmax_scale=0.0,
                 kernel=KERNEL_DEFAULT, splits=0, pool_events=None, private_pools=None):
    import torch

    n_agents = len(pools)
    arr = (POINTER(Pool) * max(n_agents, 1))(*[ctypes.pointer(p) for p in pools])
    lens = (c_int32 * max(n_agents, 1))(*(list(sfx_len) if sfx_len is not None else [0] * n_agents))
    if q.dim() != 4:
        raise ValueError("q must be [n_agents][layers][n_q_heads][head_dim]")
    A, lc, hq, d = q.shape
    if A != n_agents or tuple(out.shape) != (A, lc, hq, d) or not q.is_contiguous() or not out.is_contiguous():
        raise ValueError("q/out must be contiguous [n_agents][layers][n_q_heads][head_dim]")
    if out.dtype != torch.float32:
        raise ValueError("out must be float32 (the kernels write fp32 outputs)")
    _dtype_code(q)
    if not (q.is_cuda and out.is_cuda):
        raise ValueError("q and out must be device tensors")
    a = DecodeArgs()
    a.n_agents, a.n_q_heads, a.layer_begin, a.layer_count = n_agents, hq, layer_begin, lc
    a.softmax_scale = softmax_scale
    a.agent_pool = arr
    a.q = q.data_ptr()
    a.q_dtype = _dtype_code(q)
    a.out = out.data_ptr()
    if (sfx_k is None) != (sfx_v is None):
        raise ValueError("sfx_k and sfx_v are given together")
    if sfx_k is not None:
        if sfx_k.shape != sfx_v.shape or sfx_k.dim() != 5 or not sfx_k.is_contiguous() or not sfx_v.is_contiguous():
            raise ValueError("sfx_k/sfx_v must be contiguous [n_agents][layers][n_kv_heads][sfx_cap][head_dim]")
        hkv = pools[0].cfg.n_kv_heads if n_agents else sfx_k.shape[2]
        if tuple(sfx_k.shape[:3]) != (A, lc, hkv) or sfx_k.shape[4] != d:
            raise ValueError(f"sfx_k/sfx_v shape {tuple(sfx_k.shape)} does not match "
                             f"[n_agents={A}][layers={lc}][n_kv_heads={hkv}][sfx_cap][head_dim={d}]")
        if sfx_k.dtype != sfx_v.dtype:
            raise ValueError("sfx_k and sfx_v must have the same dtype")
        _dtype_code(sfx_k)
        if not (sfx_k.is_cuda and sfx_v.is_cuda):
            raise ValueError("sfx_k and sfx_v must be device tensors")
        a.sfx_k, a.sfx_v = sfx_k.data_ptr(), sfx_v.data_ptr()
        a.sfx_dtype = _dtype_code(sfx_k)
        a.sfx_cap = sfx_k.shape[3]
    a.sfx_len = lens
    a.kernel, a.splits = kernel, splits
    evs = None
    if pool_events is not None:
        evs = (c_void_p * 2)(*[e.cuda_event if hasattr(e, "cuda_event") else e for e in pool_events])
        a.pool_events = ctypes.cast(evs, POINTER(c_void_p))
    prv = None
    if private_pools is not None:
        if len(private_pools) != n_agents:
            raise ValueError("private_pools needs one entry (a Pool or None) per agent")
        prv = (POINTER(Pool) * max(n_agents, 1))(*[ctypes.pointer(p) if p is not None else None
                                                   for p in private_pools])
        a.agent_private_pool = prv
    return a, (arr, lens, evs, prv)


def agent_decode_attention(pools, q, out, layer_begin=0, sfx_k=None, sfx_v=None, sfx_len=None, workspace=None,
                           softmax_scale=0.0, kernel=KERNEL_DEFAULT, splits=0, stream=None,
                           pool_events=None, private_pools=None) -> int:
    """Enqueue one decode call.  pools: list of Pool (one per agent; the same object = shared pool).

    private_pools: optional list with one entry per agent, a Pool the agent also attends
    (its own older tokens, quantized once) or None.

    With workspace=None only the required workspace size is computed and returned.
    pool_events: optional pair of recorded torch.cuda.Event (or raw hipEvent_t handles)
    bracketing the pool kernel.  Returns the workspace bytes the call needs.
    """
    a, keep = _decode_args(pools, q, out, layer_begin, sfx_k, sfx_v, sfx_len, softmax_scale, kernel, splits,
                           pool_events, private_pools)
    size = c_size_t(0)
    if workspace is None:
        _check(lib().agent_decode_attention(ctypes.byref(a), None, ctypes.byref(size), None), "agent_decode_attention")
        return int(size.value)
    size.value = workspace.numel() * workspace.element_size()
    ws_ptr = workspace.data_ptr()
    if not ws_ptr:
        # the C call reads a NULL workspace as a size query and would enqueue nothing
        raise ValueError("workspace has no device address (a zero-size tensor); allocate at least 256 bytes")
    _check(lib().agent_decode_attention(ctypes.byref(a), c_void_p(ws_ptr), ctypes.byref(size),
                                        c_void_p(_stream_handle(stream))), "agent_decode_attention")
    del keep
    return int(size.value)


def agent_decode_attention_noalloc(pools, q, out, layer_begin=0, sfx_k=None, sfx_v=None, sfx_len=None,
                                   softmax_scale=0.0, kernel=KERNEL_DEFAULT, splits=0, stream=None,
                                   pool_events=None, private_pools=None) -> None:
    """Enqueue one decode call whose partial records use the library's per-device scratch array
    (no workspace, nothing allocated).  Arguments as agent_decode_attention."""
    a, keep = _decode_args(pools, q, out, layer_begin, sfx_k, sfx_v, sfx_len, softmax_scale, kernel, splits,
                           pool_events, private_pools)
    _check(lib().agent_decode_attention_noalloc(ctypes.byref(a), c_void_p(_stream_handle(stream))),
           "agent_decode_attention_noalloc")
    del keep


def noalloc_scratch_bytes() -> int:
    """Bytes of the per-device array agent_decode_attention_noalloc uses."""
    return int(lib().pkv_noalloc_scratch_bytes())


def stream_read(src, sink, stream=None) -> None:
    """Enqueue the streaming read of the device tensor src (its bytes) into sink (device int32/uint32,
    at least stream_read_sink_words() elements): the HBM read ceiling of the measurements."""
    if not (src.is_cuda and sink.is_cuda and src.is_contiguous()) or sink.element_size() != 4 or \
            sink.numel() < stream_read_sink_words():
        raise ValueError("src: contiguous device tensor; sink: device 32-bit tensor of stream_read_sink_words()")
    _check(lib().pkv_stream_read(c_void_p(src.data_ptr()), src.numel() * src.element_size(), c_void_p(sink.data_ptr()),
                                 c_void_p(_stream_handle(stream))), "pkv_stream_read")


def stream_read_sink_words() -> int:
    return int(lib().pkv_stream_read_sink_words())


def lloyd_max_table(bits: int):
    """The library's fp32 (centroids, thresholds) lists for `bits`."""
    c = (c_float * 16)()
    t = (c_float * 15)()
    _check(lib().pkv_lloyd_max_table(bits, c, t), "pkv_lloyd_max_table")
    return list(c[: 1 << bits]), list(t[: (1 << bits) - 1])


def lloyd_max_distortion(bits: int) -> float:
    """The library's D_b = E[(X - Q(X))^2] for N(0, 1) at `bits` (2, 3, 4)."""
    d = lib().pkv_lloyd_max_distortion(bits)
    if d < 0:
        raise PolyKVError(-2, "pkv_lloyd_max_distortion")
    return float(d)


def comix_sensitivity(q, win_k, win_v, win_len, out, softmax_scale=0.0, stream=None) -> None:
    """Enqueue the CoMixKV sensitivity estimate.

    q: [n_recent][A][L][Hq][d] (bf16 or fp32); win_k, win_v: [A][L][Hkv][cap][d] (bf16 or
    fp32, the agents' native windows); win_len: A ints; out: fp32 [A][L].
    """
    R, A, L, Hq, d = q.shape
    if not q.is_contiguous() or not out.is_contiguous() or tuple(out.shape) != (A, L) or out.dtype.itemsize != 4:
        raise ValueError("q must be contiguous [R][A][L][Hq][d]; out contiguous fp32 [A][L]")
    if win_k is None or win_v is None:
        raise ValueError("windows required")
    if not (win_k.is_contiguous() and win_v.is_contiguous()) or win_k.shape != win_v.shape or \
            win_k.dim() != 5 or tuple(win_k.shape[:2]) != (A, L) or win_k.shape[4] != d or win_k.dtype != win_v.dtype:
        raise ValueError("windows must be contiguous [A][L][Hkv][cap][d], same shape and dtype")
    if not (q.is_cuda and out.is_cuda and win_k.is_cuda and win_v.is_cuda):
        raise ValueError("q, windows and out must be device tensors")
    lens = (c_int32 * A)(*[int(x) for x in win_len])
    a = ComixArgs(A, L, Hq, int(win_k.shape[2]), d, float(softmax_scale), R, c_void_p(q.data_ptr()), _dtype_code(q),
                  c_void_p(win_k.data_ptr()), c_void_p(win_v.data_ptr()), _dtype_code(win_k), int(win_k.shape[3]),
                  lens, c_void_p(out.data_ptr()))
    _check(lib().comix_sensitivity(ctypes.byref(a), c_void_p(_stream_handle(stream))), "comix_sensitivity")


def comix_allocate_bits(sensitivity, cost, error_factor, budget: int):
    """Bits (2..4) per item; sensitivity [n] floats, cost [n][3] byte counts, error_factor [3]."""
    n = len(sensitivity)
    s = (c_float * max(n, 1))(*[float(x) for x in sensitivity])
    c = (c_uint64 * max(3 * n, 1))(*[int(x) for row in cost for x in row])
    e = (ctypes.c_double * 3)(*[float(x) for x in error_factor])
    out = (c_uint8 * max(n, 1))()
    _check(lib().comix_allocate_bits(n, s, c, e, int(budget), out), "comix_allocate_bits")
    return [int(out[i]) for i in range(n)]


def pool_export_header(pool) -> PoolHeader:
    """The handoff header of a pool (host only)."""
    h = PoolHeader()
    _check(lib().pool_export_header(ctypes.byref(pool), ctypes.byref(h)), "pool_export_header")
    return h


def pool_import(header, dev_ptr: int, dev_bytes: int):
    """Describe an image already copied to dev_ptr (host only)."""
    p = Pool()
    _check(lib().pool_import(ctypes.byref(header), c_void_p(dev_ptr), dev_bytes, ctypes.byref(p)), "pool_import")
    return p


def pool_shard(src, head_begin: int, head_count: int, dev_ptr: int, dev_bytes: int, stream=None):
    """A pool of kv heads [head_begin, head_begin + head_count) of src in the given device buffer."""
    p = Pool()
    _check(lib().pool_shard(ctypes.byref(src), head_begin, head_count, c_void_p(dev_ptr), dev_bytes, ctypes.byref(p),
                            c_void_p(_stream_handle(stream))), "pool_shard")
    return p

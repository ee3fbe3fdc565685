"""MI355X-native shared, asymmetrically compressed KV pool with fused multi-agent decode attention.

The compute path is the HIP library ``_lib/libpolykv.so`` (sources in ``csrc/``,
C ABI in ``include/polykv.h``); ``polykv`` is its ctypes binding (argument
marshalling only; torch tensors supply device memory and streams).
"""
from . import polykv  # noqa: F401

__all__ = ["polykv"]

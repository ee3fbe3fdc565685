"""CPU oracle for the shared compressed-KV decode path (test infrastructure).

A plain, slow, obviously checkable NumPy implementation of what the GPU path
computes.  It is *test infrastructure*: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it shares no code, tables or constants with that path.

Sources (the PolyKV and CoMixKV web pages; citations name page and section):

* PolyKV explainer, section 2.A (core architecture): one shared pool written
  once and read by many agents; memory independent of the agent count.
* PolyKV explainer, section 2.B (asymmetric compression scheme): K to int8 by a
  per-tensor linear scale; V by an FWHT rotation, Lloyd-Max centroids for
  N(0, 1) at 3 bits, and dequantisation by centroid lookup plus inverse FWHT.
* PolyKV explainer, section 2 (compression-ratio equation): 16 / ((8+3)/2).
* CoMixKV news article, "incremental quantization strategy": per-(agent, layer)
  2 to 4 bit widths; recent tokens stay at native precision; quantised blocks
  are never re-quantised.
* CoMixKV news article, abstract and method: online sensitivity from recent
  Q/K/V as a local attention-error bound; joint bit allocation over agents and
  layers under a shared byte budget.

Modules:

* ``hadamard``   Sylvester Hadamard matrix, fp32 stage-wise FWHT, fp32 norm.
* ``lloyd_max``  Lloyd-Max quantiser for N(0, 1) in double, rounded to fp32.
* ``codec``      K int8 codec, V rotate/normalise/code codec, code-group packing.
* ``pool_image`` byte layout of one pool and a builder that writes it.
* ``attention``  fp64 decode attention over decoded pool + native suffix.
* ``comixkv``    CoMixKV controller: local attention-error sensitivity per
  (agent, layer) and greedy joint 2/3/4-bit allocation under a byte budget.

Readings of what the pages leave open are stated in each function's docstring.
"""
from . import hadamard, lloyd_max, codec, pool_image, attention, comixkv  # noqa: F401

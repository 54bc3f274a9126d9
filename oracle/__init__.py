"""CPU oracle for the fused attention forward pass — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code that states what the HIP path computes, written
from the pages' description and nothing else:

* ``attention``  — the exact result (three-pass definition and the block-by-block
  running-softmax loop of the "Fused attention kernel" page, Implementation sketch),
  masks, varlen packing and the paged-KV gather.
* ``fp8``        — the e4m3 codec, the random-sign x Hadamard rotation and the
  block / per-tensor quantisers of the page's "8-bit forward pass" section, plus a
  float64 emulation of the quantised pipeline.
* ``backward``   — the gradients of the exact forward with respect to Q, K and V
  (the chain rule written out).
* ``int8``       — the symmetric int8 codec and quantisers of the int8 path
  (int8 Q and K, e4m3 V) and its float64 emulation.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and this
package imports nothing from the product library.
"""
from . import attention, backward, fp8, int8  # noqa: F401

"""fp64 CPU oracle for the chunk-wise causal attention round of Wave Forcing.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (``chunk_causal_dit_amd``,
``include/``) imports, links or calls this package; only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may.
It shares no code with the HIP library: inputs come from ``workloads`` (random
draws only) and everything below is written out plainly in numpy float64.

Modules
  attention  chunk-wise causal attention: per-chunk-prefix form, dense masked
             form, scalar brute force, softmax weights
  rope       3D (frame/height/width) rotary position embedding
  quant      int8 per-block quantization with a per-channel key mean
  ring       plain-list model of the history cache (append/refresh/evict)

What the method computes, and where the pages say so, is stated on each
function. Every function here is pinned by ``tests/test_oracle_pins.py``
against brute force, closed forms, library special cases or hand-derived
golden values (``tests/golden/``); none says "parity unpinned".
"""
from . import attention, quant, ring, rope  # noqa: F401

"""Plain CPU oracle for group-quantised bit-packed weight x activation products.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code, table or constant generator with
the HIP library under ``bit_packed_weight_amd/``; the two meet only in the
seeded input generators of ``synth/``.

Everything here is numpy, in fp64 for floating point (int64 for integer group
partials), written to be checked against the pages by eye:

* ``formats``   -- bit layouts of the packed weights (unpack / pack / block split)
* ``quant``     -- the per-row and per-group int8 activation quantiser
* ``reference`` -- dequantise-then-matmul definitions, int group partials,
                   act-order permutation, dtype rounding

Every function is pinned by ``-m "not gpu"`` tests against something other
than itself (brute force, closed forms, the pages' printed mappings,
invariants). Sources cited as "<page title>, <section>".
"""
from . import formats, quant, reference  # noqa: F401

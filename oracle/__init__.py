"""CPU oracle for the tensor-parallel layer shard -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its Python
binding) never imports, calls or falls back to it.  It shares no code with the HIP
path; the only common dependency is the seeded input generator in ``workloads``.

Everything is computed in float64 from the exact values of the inputs, with no
re-rounding of intermediates.  See ``tp_oracle`` for each function's source passage.
"""
from .tp_oracle import *  # noqa: F401,F403

"""MI355X-native tensor-parallel layer-shard library.

The compute lives in ``libtp_shard.so`` (hand-written HIP for gfx950, C ABI declared in
``include/tp_shard.h``).  ``tp`` is the thin ctypes binding with the same function names;
``pipeline`` composes the calls into the column/row MLP, the attention-head shard and the
whole block with the simulated ranks computed in turn.  Importing ``tp`` raises if the
library has not been built: there is no fallback path.
"""

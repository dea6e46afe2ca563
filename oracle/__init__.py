"""CPU float64 oracle of grouped-query causal KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Importable by ``tests/``, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg; never by the library.  It imports
nothing from the library and no code is shared with the GPU path.
"""
from . import bf16, int8, rope
from .attention import (attend_rows, attend_rows_scalar, decode, kv_group,
                        prefill_chunk, prefill_ragged, rel_error, stored_values)

__all__ = ["bf16", "int8", "rope", "attend_rows", "attend_rows_scalar", "decode", "kv_group",
           "prefill_chunk", "prefill_ragged", "rel_error", "stored_values"]

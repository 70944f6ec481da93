"""Shared-QK angular-LSH attention forward pass (Reformer) for MI355X / gfx950.

The compute lives in the C-ABI library `liblsh_attn.so` (hand-written HIP
kernels, declared in include/lsh_attn.h); `binding` is its thin ctypes
binding and `inputs` the seeded synthetic input generators.
"""
from .binding import (EventSet, LshError, fwd_workspace_bytes, hash_workspace_bytes,  # noqa: F401
                      lsh_chunk_attn, lsh_hash, lsh_sort, lsh_unsort_combine, reformer_lsh_attn_fwd,
                      sort_workspace_bytes)

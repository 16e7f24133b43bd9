"""Paged KV-cache attention for MI355X (gfx950): a C-ABI HIP library and its binding.

The library (``libpagedattn.so``, built by ``paged_kv_cache_463_amd.build``)
exports the entry points declared in ``include/pa.h``; this package re-exports
their thin Python wrappers. Importing the package does not load the library;
the first call does, and raises ``LibraryNotBuilt`` if it is missing.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    BlockManager,
    copy_blocks,
    swap_blocks,
    LibraryNotBuilt,
    PagedAttentionError,
    StepGraph,
    decode,
    decode_fp8,
    decode_step,
    decode_step_fp8,
    decode_splitkv,
    decode_splitkv_fp8,
    decode_splitkv_noalloc,
    NOALLOC_SCRATCH_BYTES,
    lib,
    prefill_chunked,
    prefill_chunked_fp8,
    read_kv_rows,
    reshape_and_cache,
    reshape_and_cache_fp8,
    splitkv_workspace_bytes,
)

__all__ = ["reshape_and_cache", "decode", "decode_splitkv", "splitkv_workspace_bytes",
           "reshape_and_cache_fp8", "decode_fp8", "decode_splitkv_fp8", "decode_step", "decode_step_fp8",
           "decode_splitkv_noalloc", "NOALLOC_SCRATCH_BYTES", "StepGraph",
           "prefill_chunked", "prefill_chunked_fp8", "copy_blocks", "swap_blocks", "read_kv_rows", "BlockManager", "lib", "LIB_PATH",
           "LibraryNotBuilt", "PagedAttentionError"]

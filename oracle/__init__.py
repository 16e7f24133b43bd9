"""CPU oracle for the paged KV-cache attention path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library and its Python binding
never call it, and this package imports nothing from them: the two share no
code, headers, tables or helpers. The only common ground is the seeded input
generator in ``workloads/``, which holds no attention arithmetic.

Everything here is plain NumPy in float64, written to be checked by eye against
the pages it cites:

* ``scatter``: the new token's K/V land in the slot the block manager chose
  (page "vLLM推理引擎深度解析" §三 ``append_token`` and §五, where writing the new
  K/V into the cache is left to the manager);
* ``gather`` + ``attend``: per sequence, walk the block table over
  ``ceil(L / block_size)`` logical blocks, take K and V rows from the physical
  blocks, score ``q·k / sqrt(d)``, softmax, and weight V (page
  "vLLM推理引擎深度解析" §五, ``PagedAttention.forward``);
* ``append_slot`` + ``paged_decode_step``: a whole decode step, the new token
  written at position ``L - 1`` through the table, then decode (the same
  pages' append rule and forward);
* ``decode_partials`` + ``lse_merge``: the same softmax split over token
  partitions and recombined by log-sum-exp (not on the pages; the identity is
  exact in exact arithmetic, so the merged result must equal ``paged_decode``);
* ``paged_prefill``: causal attention of a chunk of new queries over the cached
  prefix plus the chunk itself (the pages only name the chunked-prefill switch,
  page "vLLM推理引擎深度实战" §5.3; the reading is: query i of a chunk sits at
  absolute position ``L - q_len + i`` and sees keys ``0 .. that position``).

``block_manager`` (imported as a module) holds the block manager and the block
copy / swap definitions: share counts, head-of-free-list allocation, fill then
new block on append, copy-on-write of a shared block before a write (pages
"vLLM推理引擎深度解析" §三, "vLLM 原理与源码阅读" Block 管理器, "vLLM推理引擎深度实战"
§5.3); its pins are in ``tests/test_block_manager_oracle.py``.

``fp8`` (imported as a module) holds the e4m3 KV cache: the format's values,
round-to-nearest-even quantisation with one float32 scale per kv head, the
quantising cache write and decode over the dequantised cache (the pages only
list FP8 among the supported quantisation schemes, page "vLLM推理引擎深度实战",
introduction; the format is the OCP 8-bit floating point E4M3); its pins, in
``tests/test_fp8_oracle.py``, compare it with torch's float8_e4m3fn conversion,
closed forms and the 16-bit oracle.

Parity pins: every function here is pinned by tests in
``tests/test_oracle_pins.py`` against something other than itself (torch's
fp64 ``scaled_dot_product_attention``, 40-digit ``decimal`` brute force, closed
forms, invariants, golden slot positions derived from the pages' append rule),
and mutation tests plant mistakes in this oracle to show that the pins catch
them. No function is "parity unpinned".
"""
from . import block_manager  # noqa: F401
from . import fp8  # noqa: F401
from .paged_attention import (  # noqa: F401
    to_f64,
    scatter,
    gather,
    attend,
    paged_decode,
    append_slot,
    paged_decode_step,
    decode_partials,
    lse_merge,
    paged_decode_splitkv,
    paged_prefill,
)

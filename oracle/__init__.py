"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The product (the HIP
library and its Python binding) never imports, links or calls it, and this
package imports nothing from the product; the two share only the seeded input
generator ``paged_kv_cache_364_amd.workloads``, which holds none of the
method's arithmetic.

Everything is plain numpy: integer bookkeeping in Python, attention in
float64 from its definition.  Pins (tests/test_oracle_*.py) tie each
function to facts the pages or mathematics fix:

=====================  ====================================================
function               pinned by
=====================  ====================================================
allocator              worked example of block size 4 (cnblogs section 8),
                       the 1000-token / 63-block example ("08.
                       PagedAttention"), hand-built tables, invariants
                       under random operation sequences
cache.kv_write         the slot formula, bytes outside written slots intact
cache.copy_blocks      byte equality, sources read before destinations
attention.decode       hand-computed golden case, brute force on contiguous
                       K/V, closed forms (one token, equal keys, zero
                       query), GQA = MHA with repeated KV heads, invariance
                       under block relabelling
attention.prefill      row i equals decode at context P + i + 1, chunking
                       invariance, brute force
attention.brute_force  hand-computed golden case
sizes                  the pages' Llama-3.1-8B and OPT-13B arithmetic
=====================  ====================================================
"""
from . import allocator, attention, cache, runner, sizes  # noqa: F401

"""pagedkv: paged KV-cache attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libpagedkv.so`` (HIP kernels and a C++ block
allocator behind the C ABI of ``include/pagedkv.h``); this package only
marshals torch tensors and host arrays into those calls.  The library is
loaded on first use and its absence is an error.
"""
from .api import (  # noqa: F401
    copy_blocks,
    decode_workspace_size,
    kv_write,
    paged_attention_decode,
    paged_attention_decode_append,
    paged_attention_prefill,
    swap_in,
    swap_out,
)
from .allocator import BlockAllocator, OutOfBlocks  # noqa: F401
from ._native import PagedKVError  # noqa: F401

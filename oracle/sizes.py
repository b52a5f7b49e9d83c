"""KV-cache size arithmetic from the pages.

TEST INFRASTRUCTURE ONLY.

* Bytes of K and V per token across all layers:
  layers * 2 (K and V) * kv_heads * head_dim * bytes per element.
  Llama-3.1-8B (32 layers, 8 KV heads, head_dim 128, 2-byte elements) gives
  128 KiB; a 16-token block holds 2 MiB; 50 GiB of KV space is 25,600 blocks
  or 409,600 tokens.  "08. PagedAttention", section "how much waste remains",
  and its opening paragraph (about 400k tokens on one card).
* OPT-13B (40 layers, hidden 5120) gives 800 KiB per token and 1.5625 GiB for
  2048 tokens (quoted as about 800 KB and 1.6 GB).  intelliparadigm.com
  article, section 1.
* Tail waste: a sequence of n tokens in blocks of B occupies ceil(n / B)
  blocks and leaves ceil(n / B) * B - n < B slots unused.  cnblogs section 4;
  "08. PagedAttention", section "how much waste remains".
"""
from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return layers * 2 * kv_heads * head_dim * elem_bytes


def blocks_for(n_tokens: int, block_size: int) -> int:
    return -(-n_tokens // block_size)


def tail_waste(n_tokens: int, block_size: int) -> int:
    return blocks_for(n_tokens, block_size) * block_size - n_tokens

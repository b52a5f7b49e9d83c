"""Python entry points over the C ABI, taking torch tensors.

Each function checks that its tensors live on the GPU, are contiguous and
have the expected dtype, then passes raw device pointers and the current
HIP stream to the matching ``pkv_*`` call of libpagedkv.so.  Nothing is
computed here.  Names follow the C calls without their ``pkv_`` prefix.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _native as N

_DTYPES = {torch.float32: N.DTYPE_F32, torch.bfloat16: N.DTYPE_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _cache_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor):
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    return k_cache.shape  # N, Hkv, B, D


def kv_write(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
             v_cache: torch.Tensor, stream=None) -> None:
    """k_cache/v_cache[slot // B, :, slot % B, :] = k_new/v_new[t] (pkv_kv_write)."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    T = slot_mapping.numel()
    if k_new.shape != (T, H, D) or v_new.shape != (T, H, D):
        raise ValueError("k_new and v_new must be [num_tokens, num_kv_heads, head_dim]")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("new K/V must have the cache dtype")
    N.check(N.lib().pkv_kv_write(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping", torch.int32), T,
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), N_, H, B, D, _dtype_code(k_cache), _stream(stream)),
        "kv_write")


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs: torch.Tensor, stream=None) -> None:
    """Copy whole blocks src -> dst for K and V (pkv_copy_blocks); pairs int32 [n, 2]."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [num_pairs, 2]")
    N.check(N.lib().pkv_copy_blocks(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(pairs, "pairs", torch.int32), pairs.shape[0],
        N_, H, B, D, _dtype_code(k_cache), _stream(stream)), "copy_blocks")


def _pinned(t: torch.Tensor, name: str, shape, dtype) -> int:
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor (torch.empty(..., pin_memory=True))")
    if not t.is_contiguous() or tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return t.data_ptr()


def swap_out(k_cache: torch.Tensor, v_cache: torch.Tensor, block_ids: torch.Tensor, host_k: torch.Tensor,
             host_v: torch.Tensor, stream=None) -> None:
    """host_k/host_v[i] = k_cache/v_cache[block_ids[i]] (pkv_swap_out); host
    tensors pinned, [n, num_kv_heads, block_size, head_dim]."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    n = block_ids.numel()
    N.check(N.lib().pkv_swap_out(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_ids, "block_ids", torch.int32), n, N_, H, B,
        D, _dtype_code(k_cache), _pinned(host_k, "host_k", (n, H, B, D), k_cache.dtype),
        _pinned(host_v, "host_v", (n, H, B, D), k_cache.dtype), _stream(stream)), "swap_out")


def swap_in(k_cache: torch.Tensor, v_cache: torch.Tensor, block_ids: torch.Tensor, host_k: torch.Tensor,
            host_v: torch.Tensor, stream=None) -> None:
    """k_cache/v_cache[block_ids[i]] = host_k/host_v[i] (pkv_swap_in)."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    n = block_ids.numel()
    N.check(N.lib().pkv_swap_in(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_ids, "block_ids", torch.int32), n, N_, H, B,
        D, _dtype_code(k_cache), _pinned(host_k, "host_k", (n, H, B, D), k_cache.dtype),
        _pinned(host_v, "host_v", (n, H, B, D), k_cache.dtype), _stream(stream)), "swap_in")


def decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                          max_blocks_per_seq: int, dtype: torch.dtype) -> int:
    n = N.lib().pkv_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                          max_blocks_per_seq, _DTYPES[dtype])
    if n == 0:
        raise N.PagedKVError(N.PKV_ERR_UNSUPPORTED, "decode_workspace_size")
    return n


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           workspace: Optional[torch.Tensor] = None, stream=None, window: int = 0) -> torch.Tensor:
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s through the block
    tables (pkv_paged_attention_decode); with ``window`` > 0 only the last
    ``window`` tokens of each context are attended
    (pkv_paged_attention_decode_window).  ``workspace`` is a uint8 GPU
    tensor of at least decode_workspace_size(...) bytes; one is allocated
    when omitted."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    S, Hq, Dq = q.shape
    if Dq != D or out.shape != q.shape or out.dtype != q.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q/out must be [num_seqs, num_heads, head_dim] of the cache dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    mb = block_tables.shape[1]
    if workspace is None:
        workspace = torch.zeros(decode_workspace_size(S, Hq, H, D, B, mb, q.dtype), dtype=torch.uint8,
                                device=q.device)
    args = [_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables", torch.int32), mb, _dev(context_lens, "context_lens", torch.int32), S,
            Hq, H, D, B, N_]
    tail = [float(scale), _dtype_code(q), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
            _stream(stream)]
    if window and window > 0:
        N.check(N.lib().pkv_paged_attention_decode_window(*args, int(window), *tail), "paged_attention_decode_window")
    else:
        N.check(N.lib().pkv_paged_attention_decode(*args, *tail), "paged_attention_decode")
    return out


def paged_attention_decode_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float, workspace: Optional[torch.Tensor] = None,
                                  stream=None) -> torch.Tensor:
    """kv_write of each sequence's new token (k_new/v_new[s], [num_seqs,
    num_kv_heads, head_dim]) at position context_lens[s] - 1 through its
    block table, then paged_attention_decode, in one call
    (pkv_paged_attention_decode_append); bit for bit the two calls."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    S, Hq, Dq = q.shape
    if Dq != D or out.shape != q.shape or out.dtype != q.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q/out must be [num_seqs, num_heads, head_dim] of the cache dtype")
    if k_new.shape != (S, H, D) or v_new.shape != (S, H, D) or k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise ValueError("k_new/v_new must be [num_seqs, num_kv_heads, head_dim] of the cache dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    mb = block_tables.shape[1]
    if workspace is None:
        workspace = torch.zeros(decode_workspace_size(S, Hq, H, D, B, mb, q.dtype), dtype=torch.uint8,
                                device=q.device)
    N.check(N.lib().pkv_paged_attention_decode_append(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables", torch.int32), mb,
        _dev(context_lens, "context_lens", torch.int32), S, Hq, H, D, B, N_, float(scale), _dtype_code(q),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream)),
        "paged_attention_decode_append")
    return out


def paged_attention_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                                   scale: float, stream=None) -> torch.Tensor:
    """As paged_attention_decode, with the partials in the library's own
    per-GPU scratch array (pkv_paged_attention_decode_noalloc): no
    allocation anywhere, for callers that cannot allocate."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    S, Hq, Dq = q.shape
    if Dq != D or out.shape != q.shape or out.dtype != q.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q/out must be [num_seqs, num_heads, head_dim] of the cache dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    N.check(N.lib().pkv_paged_attention_decode_noalloc(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, Hq, H, D, B, N_, float(scale), _dtype_code(q),
        _stream(stream)), "paged_attention_decode_noalloc")
    return out


def decode_shared_max_members(num_heads: int, num_kv_heads: int) -> int:
    """Largest group paged_attention_decode_shared takes (pkv_decode_shared_max_members)."""
    return int(N.lib().pkv_decode_shared_max_members(int(num_heads), int(num_kv_heads)))


def paged_attention_decode_shared(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor, group_start: torch.Tensor,
                                  shared_blocks: torch.Tensor, scale: float, stream=None) -> torch.Tensor:
    """Decode of a batch whose sequences share prompt blocks, each group's
    shared blocks read once for all its members
    (pkv_paged_attention_decode_shared); group_start int32 [num_groups + 1]
    and shared_blocks int32 [num_groups] as BlockAllocator.shared_prefix_groups
    returns them, on the GPU."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    S, Hq, Dq = q.shape
    if Dq != D or out.shape != q.shape or out.dtype != q.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q/out must be [num_seqs, num_heads, head_dim] of the cache dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    G = shared_blocks.numel()
    if group_start.shape != (G + 1,):
        raise ValueError("group_start must be [num_groups + 1]")
    N.check(N.lib().pkv_paged_attention_decode_shared(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, _dev(group_start, "group_start", torch.int32),
        _dev(shared_blocks, "shared_blocks", torch.int32), G, Hq, H, D, B, N_, float(scale), _dtype_code(q),
        _stream(stream)), "paged_attention_decode_shared")
    return out


def gather_units(pool_a: torch.Tensor, pool_b: Optional[torch.Tensor], unit_ids: torch.Tensor, unit_kib: int,
                 sink: torch.Tensor, stream=None) -> None:
    """Read every listed unit of unit_kib KiB of pool_a (and pool_b) once,
    with no other arithmetic (pkv_gather_units): the bandwidth ceiling of the
    paged access pattern.  sink: int32 GPU tensor, one word per wavefront."""
    nbytes = pool_a.numel() * pool_a.element_size()
    if pool_b is not None and pool_b.numel() * pool_b.element_size() != nbytes:
        raise ValueError("pool_a and pool_b must have the same size")
    pool_units = nbytes // (int(unit_kib) * 1024)
    N.check(N.lib().pkv_gather_units(
        _dev(pool_a, "pool_a"), _dev(pool_b, "pool_b") if pool_b is not None else None,
        _dev(unit_ids, "unit_ids", torch.int32), unit_ids.numel(), int(unit_kib), pool_units,
        _dev(sink, "sink", torch.int32), sink.numel(), _stream(stream)), "gather_units")


def paged_attention_prefill(out: torch.Tensor, q: torch.Tensor, cu_q_lens: torch.Tensor, max_q_len: int,
                            k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, scale: float, stream=None) -> torch.Tensor:
    """Causal chunk attention over the cached prefix (pkv_paged_attention_prefill);
    q/out packed [total_q, num_heads, head_dim] bf16, cu_q_lens int32 [S + 1]."""
    N_, H, B, D = _cache_geometry(k_cache, v_cache)
    T, Hq, Dq = q.shape
    S = context_lens.shape[0]
    if Dq != D or out.shape != q.shape or out.dtype != q.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q/out must be [total_q, num_heads, head_dim] of the cache dtype")
    if cu_q_lens.shape != (S + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("cu_q_lens must be [num_seqs + 1], block_tables [num_seqs, max_blocks]")
    N.check(N.lib().pkv_paged_attention_prefill(
        _dev(out, "out"), _dev(q, "q"), _dev(cu_q_lens, "cu_q_lens", torch.int32), T, int(max_q_len),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1], _dev(context_lens, "context_lens", torch.int32), S, Hq, H, D, B, N_, float(scale),
        _dtype_code(q), _stream(stream)), "paged_attention_prefill")
    return out

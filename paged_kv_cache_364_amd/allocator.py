"""Python handle over the C++ block allocator of libpagedkv.so."""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import _native as N


class OutOfBlocks(N.PagedKVError):
    pass


class BlockAllocator:
    """Free list + reference counts + block tables (pkv_alloc_*).

    ``append`` returns the slot of each new token and the (src, dst) block
    copies to perform before writing them; see include/pagedkv.h for the
    policy."""

    def __init__(self, num_blocks: int, block_size: int, init_order: Optional[Sequence[int]] = None):
        L = N.lib()
        self._L = L
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if init_order is None:
            h = L.pkv_alloc_create(self.num_blocks, self.block_size, None)
        else:
            arr = np.ascontiguousarray(init_order, dtype=np.int32)
            if arr.shape != (self.num_blocks,):
                raise ValueError("init_order must have num_blocks entries")
            h = L.pkv_alloc_create(self.num_blocks, self.block_size, arr.ctypes.data_as(N.i32p))
        if not h:
            raise N.PagedKVError(N.PKV_ERR_INVALID, "pkv_alloc_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._L.pkv_alloc_destroy(h)
            self._h = None

    def add(self, seq: int) -> None:
        N.check(self._L.pkv_seq_add(self._h, int(seq)), "seq_add")

    def append(self, seq: int, n: int) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        slots = np.empty(max(int(n), 1), dtype=np.int32)
        pairs = np.empty(2, dtype=np.int32)
        nc = ctypes.c_int(0)
        st = self._L.pkv_seq_append(self._h, int(seq), int(n), slots.ctypes.data_as(N.i32p),
                                    pairs.ctypes.data_as(N.i32p), 1, ctypes.byref(nc))
        if st == N.PKV_ERR_NO_BLOCKS:
            raise OutOfBlocks(st, "seq_append")
        N.check(st, "seq_append")
        return slots[: int(n)], [(int(pairs[0]), int(pairs[1]))] if nc.value else []

    def append_tokens(self, seq: int, tokens) -> Tuple[np.ndarray, List[Tuple[int, int]], int]:
        """Append tokens with known ids, reusing cached full blocks
        (pkv_seq_append_tokens).  Returns slots (-1 where the token's K/V
        are already cached), copies, and the number of cached tokens."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = tok.shape[0]
        slots = np.empty(max(n, 1), dtype=np.int32)
        pairs = np.empty(2, dtype=np.int32)
        nc, ncached = ctypes.c_int(0), ctypes.c_int(0)
        st = self._L.pkv_seq_append_tokens(self._h, int(seq), tok.ctypes.data_as(N.i32p), n,
                                           slots.ctypes.data_as(N.i32p), ctypes.byref(ncached),
                                           pairs.ctypes.data_as(N.i32p), 1, ctypes.byref(nc))
        if st == N.PKV_ERR_NO_BLOCKS:
            raise OutOfBlocks(st, "seq_append_tokens")
        N.check(st, "seq_append_tokens")
        return slots[:n], ([(int(pairs[0]), int(pairs[1]))] if nc.value else []), int(ncached.value)

    def trim(self, seq: int, keep_from: int) -> int:
        """Release the blocks wholly before position keep_from (pkv_seq_trim);
        returns how many table entries were released."""
        x = ctypes.c_int(0)
        N.check(self._L.pkv_seq_trim(self._h, int(seq), int(keep_from), ctypes.byref(x)), "seq_trim")
        return int(x.value)

    def prefix_cache_size(self) -> int:
        x = ctypes.c_int(0)
        N.check(self._L.pkv_prefix_cache_size(self._h, ctypes.byref(x)), "prefix_cache_size")
        return int(x.value)

    def fork(self, parent: int, child: int, fork_pos: int) -> None:
        N.check(self._L.pkv_seq_fork(self._h, int(parent), int(child), int(fork_pos)), "seq_fork")

    def release(self, seq: int) -> None:
        N.check(self._L.pkv_seq_free(self._h, int(seq)), "seq_free")

    def _blocks_call(self, fn, seq: int, what: str) -> List[int]:
        n = ctypes.c_int(0)
        out = np.empty(max(self.num_blocks, 1), dtype=np.int32)
        st = fn(self._h, int(seq), out.ctypes.data_as(N.i32p), self.num_blocks, ctypes.byref(n))
        if st == N.PKV_ERR_NO_BLOCKS:
            raise OutOfBlocks(st, what)
        N.check(st, what)
        return out[: n.value].tolist()

    def swap_out(self, seq: int) -> List[int]:
        """Release the sequence's blocks (pkv_seq_swap_out); returns its
        table, the blocks whose contents go to host memory."""
        return self._blocks_call(self._L.pkv_seq_swap_out, seq, "seq_swap_out")

    def swap_in(self, seq: int) -> List[int]:
        """Fresh blocks for a swapped-out sequence (pkv_seq_swap_in); host
        buffer i goes to returned block i."""
        return self._blocks_call(self._L.pkv_seq_swap_in, seq, "seq_swap_in")

    def length(self, seq: int) -> int:
        x = ctypes.c_int64(0)
        N.check(self._L.pkv_seq_len(self._h, int(seq), ctypes.byref(x)), "seq_len")
        return int(x.value)

    def table(self, seq: int) -> List[int]:
        n = ctypes.c_int(0)
        self._L.pkv_get_block_table(self._h, int(seq), None, 0, ctypes.byref(n))
        out = np.empty(max(n.value, 1), dtype=np.int32)
        N.check(self._L.pkv_get_block_table(self._h, int(seq), out.ctypes.data_as(N.i32p), n.value,
                                            ctypes.byref(n)), "get_block_table")
        return out[: n.value].tolist()

    def block_tables(self, seqs: Sequence[int], width: int) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        t = np.empty((len(ids), max(int(width), 1)), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        N.check(self._L.pkv_build_block_tables(self._h, ids.ctypes.data_as(N.i64p), len(ids), t.shape[1],
                                               t.ctypes.data_as(N.i32p), lens.ctypes.data_as(N.i32p)),
                "build_block_tables")
        return t, lens

    def shared_prefix_groups(self, seqs: Sequence[int], max_members: int) -> Tuple[np.ndarray, np.ndarray]:
        """Groups of the batch for the shared-prefix decode
        (pkv_shared_prefix_groups): group_start [num_groups + 1] and
        shared_blocks [num_groups], both int32."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        starts = np.empty(len(ids) + 1, dtype=np.int32)
        shared = np.empty(max(len(ids), 1), dtype=np.int32)
        ng = ctypes.c_int(0)
        N.check(self._L.pkv_shared_prefix_groups(self._h, ids.ctypes.data_as(N.i64p), len(ids), int(max_members),
                                                 starts.ctypes.data_as(N.i32p), shared.ctypes.data_as(N.i32p),
                                                 ctypes.byref(ng)), "shared_prefix_groups")
        return starts[: ng.value + 1].copy(), shared[: ng.value].copy()

    def stats(self) -> N.PkvStats:
        s = N.PkvStats()
        N.check(self._L.pkv_alloc_stats(self._h, ctypes.byref(s)), "alloc_stats")
        return s

    def ref(self, block: int) -> int:
        r = ctypes.c_int(0)
        N.check(self._L.pkv_block_ref(self._h, int(block), ctypes.byref(r)), "block_ref")
        return r.value

    def free_list(self) -> List[int]:
        n = ctypes.c_int(0)
        out = np.empty(self.num_blocks, dtype=np.int32)
        N.check(self._L.pkv_free_list(self._h, out.ctypes.data_as(N.i32p), self.num_blocks, ctypes.byref(n)),
                "free_list")
        return out[: n.value].tolist()

    def num_free(self) -> int:
        return int(self.stats().num_free)

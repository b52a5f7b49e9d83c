"""Run a workload script on the CPU model: allocator, pools, then attention.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check, the benchmark's CPU
baseline).

A step runs its allocator operations in order, then performs every
copy-on-write copy they produced (reading all sources first), then writes the
K/V rows of the step's appends to their slots (intelliparadigm.com article,
section 2.3 for the copy-before-modify order; "08. PagedAttention", section
"why the name" for the slot write).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

from . import attention, cache
from .allocator import BlockAllocator


@dataclass
class OracleState:
    alloc: BlockAllocator
    k_pool: np.ndarray
    v_pool: np.ndarray
    tables: np.ndarray
    context_lens: np.ndarray
    step_slots: List[List[int]] = field(default_factory=list)
    step_copies: List[List[Tuple[int, int]]] = field(default_factory=list)


def run(wl, with_pools: bool = True) -> OracleState:
    alloc = BlockAllocator(wl.num_blocks, wl.block_size, wl.init_order)
    shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    kp = cache.new_pool(*shape, wl.dtype) if with_pools else None
    vp = cache.new_pool(*shape, wl.dtype) if with_pools else None
    all_slots, all_copies = [], []
    for st in wl.steps:
        slots, copies, ks, vs, wslots = [], [], [], [], []
        for op in st.ops:
            if op.kind == "add":
                alloc.add(op.seq)
            elif op.kind == "append":
                if op.tokens is not None:
                    sl, cp, _ = alloc.append_tokens(op.seq, op.tokens)
                else:
                    sl, cp = alloc.append(op.seq, op.n)
                slots += sl
                copies += cp
                if op.k is not None:
                    wslots += sl
                    ks.append(op.k)
                    vs.append(op.v)
            elif op.kind == "fork":
                alloc.fork(op.parent, op.seq, op.fork_pos)
            elif op.kind == "free":
                alloc.release(op.seq)
            else:
                raise ValueError(op.kind)
        if with_pools:
            cache.copy_blocks(kp, copies)
            cache.copy_blocks(vp, copies)
            if ks:
                cache.kv_write(kp, cache.as_raw(np.concatenate(ks), wl.dtype), wslots)
                cache.kv_write(vp, cache.as_raw(np.concatenate(vs), wl.dtype), wslots)
        all_slots.append(slots)
        all_copies.append(copies)
    tables, lens = alloc.block_tables(wl.batch, wl.max_blocks_per_seq)
    return OracleState(alloc, kp, vp, tables, lens, all_slots, all_copies)


def cu_lens(q_lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)


def expected(wl, st: OracleState) -> np.ndarray:
    """float64 attention output of the workload's batch."""
    if wl.kind == "decode":
        return attention.decode(wl.q, st.k_pool, st.v_pool, st.tables, st.context_lens, wl.scale, wl.dtype)
    return attention.prefill(wl.q, cu_lens(wl.q_lens), st.k_pool, st.v_pool, st.tables,
                             st.context_lens, wl.scale, wl.dtype)

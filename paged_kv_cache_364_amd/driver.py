"""Run an operation script (add / append / fork / free steps) through the
C++ allocator and the HIP kernels, and run the attention batch it ends with.

A step runs its allocator operations in order, then one ``copy_blocks`` for
all copy-on-write pairs they produced, then one ``kv_write`` for all the
tokens they appended (copy before modify: intelliparadigm.com article,
section 2.3).  Pools are allocated with torch and poisoned with quiet NaNs
so that any read of a slot that was never written shows up in the output.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import api
from .allocator import BlockAllocator

POISON = {torch.bfloat16: (torch.int16, 0x7FC0), torch.float32: (torch.int32, 0x7FC00000)}


def torch_dtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(values: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Workload raw values (uint16 bf16 bits or float32) -> GPU tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(values).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(device)


def new_pool(num_blocks, num_kv_heads, block_size, head_dim, dtype: torch.dtype, device) -> torch.Tensor:
    p = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype, device=device)
    it, bits = POISON[dtype]
    p.view(it).fill_(bits)
    return p


@dataclass
class GpuState:
    alloc: BlockAllocator
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    tables: np.ndarray
    context_lens: np.ndarray
    tables_dev: torch.Tensor
    lens_dev: torch.Tensor
    step_slots: List[List[int]] = field(default_factory=list)
    step_copies: List[list] = field(default_factory=list)


def run_script(wl, device="cuda", pools: Optional[tuple] = None) -> GpuState:
    alloc = BlockAllocator(wl.num_blocks, wl.block_size, wl.init_order)
    dt = torch_dtype(wl.dtype)
    if pools is None:
        kp = new_pool(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, dt, device)
        vp = new_pool(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, dt, device)
    else:
        kp, vp = pools
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
                sl = sl.tolist()
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
        if copies:
            pairs = torch.tensor(copies, dtype=torch.int32, device=device)
            api.copy_blocks(kp, vp, pairs)
        if ks:
            kn = to_device(np.concatenate(ks), wl.dtype, device)
            vn = to_device(np.concatenate(vs), wl.dtype, device)
            sm = torch.tensor(wslots, dtype=torch.int32, device=device)
            api.kv_write(kn, vn, sm, kp, vp)
        all_slots.append(slots)
        all_copies.append(copies)
    tables, lens = alloc.block_tables(wl.batch, wl.max_blocks_per_seq)
    return GpuState(alloc, kp, vp, tables, lens, torch.from_numpy(tables).to(device),
                    torch.from_numpy(lens).to(device), all_slots, all_copies)


def cu_lens(q_lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)


def run_attention(wl, st: GpuState, device="cuda", q: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    q = to_device(wl.q, wl.dtype, device) if q is None else q
    out = torch.empty_like(q) if out is None else out
    if wl.kind == "decode":
        api.paged_attention_decode(out, q, st.k_pool, st.v_pool, st.tables_dev, st.lens_dev, float(wl.scale),
                                   workspace=workspace)
    else:
        cu = torch.from_numpy(cu_lens(wl.q_lens)).to(device)
        api.paged_attention_prefill(out, q, cu, max(wl.q_lens), st.k_pool, st.v_pool, st.tables_dev, st.lens_dev,
                                    float(wl.scale))
    return out


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def pool_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a pool as numpy (uint16 for bf16, uint32 for fp32)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)

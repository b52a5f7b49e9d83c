"""Paged K/V pools: slot writes and whole-block copies, bit for bit.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check, the benchmark's CPU
baseline).

Pool layout (a reading; the pages do not fix one): ``[num_blocks,
num_kv_heads, block_size, head_dim]`` of raw element bits (uint16 for bf16,
float32 bits viewed as uint32 for fp32), so that a copy is a copy of bits and
NaN poison survives unchanged.

* ``kv_write``: token t goes to slot s = block * B + offset, i.e. to
  ``pool[s // B, :, s % B, :]``.  "08. PagedAttention", section "why the
  name" (slot = block_table[logical block] * block_size + offset, one small
  kernel writes each token's K/V to its slot).  A negative slot is skipped.
* ``copy_blocks``: for each (src, dst) pair the destination block becomes a
  copy of the source block, for K and V, every head and every slot
  (intelliparadigm.com article, section 2.3: allocate a new block, copy the
  original block's contents).  All sources are read before any destination
  is written.
* ``swap_out`` / ``swap_in``: whole blocks to and from a host buffer whose
  entry i is block ids[i] (intelliparadigm.com article, sections 3.1 and
  6.1: a preempted request's blocks go to CPU memory and come back).
"""
from __future__ import annotations

import numpy as np

POISON_BF16 = np.uint16(0x7FC0)
POISON_F32 = np.uint32(0x7FC00000)


def raw_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.uint32


def new_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype: str) -> np.ndarray:
    """A pool filled with quiet-NaN bit patterns."""
    fill = POISON_BF16 if dtype == "bf16" else POISON_F32
    return np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=raw_dtype(dtype))


def as_raw(values: np.ndarray, dtype: str) -> np.ndarray:
    """Workload values (uint16 bf16 bits or float32) -> raw pool bits."""
    if dtype == "bf16":
        return np.asarray(values, dtype=np.uint16)
    return np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)


def kv_write(pool: np.ndarray, new: np.ndarray, slots) -> None:
    """pool[slot // B, :, slot % B, :] = new[t] for every slot >= 0."""
    B = pool.shape[2]
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        pool[s // B, :, s % B, :] = new[t]


def copy_blocks(pool: np.ndarray, pairs) -> None:
    pairs = [(int(a), int(b)) for a, b in pairs]
    if not pairs:
        return
    src = np.array([a for a, _ in pairs])
    dst = np.array([b for _, b in pairs])
    data = pool[src].copy()  # read every source first
    pool[dst] = data


def swap_out(pool: np.ndarray, ids) -> np.ndarray:
    """Host buffer [n, H_kv, B, D]: entry i is block ids[i] of the pool."""
    out = np.empty((len(ids),) + pool.shape[1:], dtype=pool.dtype)
    for i, b in enumerate(ids):
        out[i] = pool[int(b)]
    return out


def swap_in(pool: np.ndarray, ids, host: np.ndarray) -> None:
    """Block ids[i] of the pool becomes host entry i."""
    for i, b in enumerate(ids):
        pool[int(b)] = host[i]

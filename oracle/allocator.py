"""Block allocator model (the bookkeeping half of paged KV caching).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
CPU-baseline leg of the benchmark; never by the product path.

What the pages fix, and where:

* KV memory is cut into equal physical blocks; a sequence's tokens sit in
  logical blocks [lb*B, lb*B + B) and a per-sequence block table maps logical
  block -> physical block.  cnblogs "paged attention" sections 2, 3 and 8;
  "08. PagedAttention", section "borrowing OS paging".
* Allocation is on demand: prefill takes what it needs, decode takes a new
  block only when the current one is full (block size 4: 10 tokens use
  3 blocks, the 11th and 12th still go to logical block 2, the 13th needs a
  4th block).  cnblogs section 8; "08. PagedAttention", same section.
* At request end all blocks go back to the free list and are reused at once.
  cnblogs sections 7 and 8.
* Sharing by reference counts; copy-on-write when a sequence modifies a
  shared block: allocate a new block, copy the contents, update the table,
  decrement the old block's count.  intelliparadigm.com article, section 2.3;
  "08. PagedAttention", section "what else paging solves".
* A slot is block_table[logical_block] * block_size + offset.
  "08. PagedAttention", section "why the name".

Readings where the pages are silent (one fixed policy, so two
implementations can be compared bit for bit; any free block is as good as
another):

* The free list is a LIFO stack.  Initially ``init_order[0]`` is on top.
* ``free`` releases blocks in reverse logical order, so logical block 0 ends
  on top and re-allocating the same length reproduces the same table.
* Copy-on-write happens only when the block is shared (ref count > 1) at the
  sequence's first write into it; the last holder writes in place.
* ``fork(parent, child, f)`` gives the child the first ceil(f / B) blocks of
  the parent (ref + 1 each) and length f.
* ``append`` is atomic: it first counts the blocks it needs and fails with
  no change when the free list is too short.

Swapping (preemption by swap: the intelliparadigm.com article, sections 3.1
and 6.1, moves a preempted request's blocks to CPU memory and back; "08.
PagedAttention", section "what it does not solve"):

* ``swap_out`` returns the sequence's table (the blocks whose contents must
  reach host memory) and then gives the blocks back exactly as ``release``
  does; the sequence keeps its length and holds no blocks.
* ``swap_in`` takes as many fresh blocks off the free list as it had, in
  logical order (all or nothing); host buffer i goes to the i-th of them.
* append, fork and table export refuse a swapped sequence; release drops it.

Prefix caching (cnblogs section 9: a system prompt shared by many requests
is stored once; "08. PagedAttention", section "what else paging solves":
only full blocks are shared, through reference counts):

* ``append_tokens`` names every full block of a sequence by a chained hash,
  FNV-1a 64 over (previous full block's hash as 8 little-endian bytes, 0 for
  the first block) followed by the block's token ids (4 little-endian bytes
  each).
* A block that the append covers whole reuses the cached block with the same
  hash and tokens, while every earlier new block of the append did; hits are
  decided on the cache as it stood before the append, and a hit block whose
  count is 0 comes back off the free list.  Its tokens' slots are -1: there
  is nothing to write.
* Every other block is placed as ``append`` places it.  A block the append
  filled is filed under its hash unless that hash is filed already.
* A block taken off the free list loses its cache entry: it is about to be
  overwritten.
* A plain ``append`` (or a fork inside a block) takes the sequence out of
  prefix caching for good.

Sliding-window reclamation (intelliparadigm.com article, section 5.2: old
blocks leave a sliding window and are reclaimed):

* ``trim(seq, keep_from)`` releases every block wholly before position
  keep_from, last first, as ``release`` would; its table entry becomes -1
  (a hole) and the length does not change.
* Holes are skipped wherever blocks are counted or released; a fork shares
  them as holes; swapping moves live blocks only and keeps the holes.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64 bit: for each byte, xor it in, then multiply by the prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(prev: int, tokens: Sequence[int]) -> int:
    data = prev.to_bytes(8, "little") + b"".join(int(t & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


class OutOfBlocks(Exception):
    pass


class AllocatorError(Exception):
    pass


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int, init_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocatorError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if init_order is None else [int(b) for b in init_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocatorError("init_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # top of the stack is the end of the list
        self.free: List[int] = list(reversed(order))
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.swapped: Dict[int, List[bool]] = {}  # seq -> holes of its table when swapped out
        # prefix caching
        self.cache: Dict[int, int] = {}  # block hash -> block
        self.cached_as: Dict[int, Tuple[int, Tuple[int, ...]]] = {}  # block -> (hash, token ids)
        self.tok_ok: Dict[int, bool] = {}
        self.hashes: Dict[int, List[int]] = {}  # seq -> hash of each full block
        self.pending: Dict[int, List[int]] = {}  # seq -> token ids of the partial last block

    # -- sequence lifecycle -------------------------------------------------
    def add(self, seq: int) -> None:
        if seq in self.tables:
            raise AllocatorError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0
        self.tok_ok[seq] = True
        self.hashes[seq] = []
        self.pending[seq] = []

    def _pop(self) -> int:
        b = self.free.pop()
        if b in self.cached_as:  # its contents are about to be overwritten
            h, _ = self.cached_as.pop(b)
            del self.cache[h]
        return b

    def append(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Reserve slots for ``n`` new tokens of ``seq``.  Returns the slot of
        each token and the (src, dst) block copies that must happen before
        the tokens are written."""
        if seq not in self.tables:
            raise AllocatorError(f"unknown sequence {seq}")
        if seq in self.swapped:
            raise AllocatorError(f"sequence {seq} is swapped out")
        if n < 0:
            raise AllocatorError("negative token count")
        B = self.block_size
        table = self.tables[seq]
        start = self.lens[seq]
        # count first (atomic append)
        need = 0
        have = len(table)
        seen_shared = set()
        for p in range(start, start + n):
            lb = p // B
            if lb >= len(table):
                if lb >= have:
                    need += 1
                    have += 1
            elif table[lb] < 0:
                # a hole (a block released by a trim of the sequence this one
                # was forked from) is a missing block: a write into it takes
                # a fresh one, as a write past the table does
                if lb not in seen_shared:
                    seen_shared.add(lb)
                    need += 1
            elif self.ref[table[lb]] > 1 and lb not in seen_shared:
                seen_shared.add(lb)
                need += 1
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        if n > 0:
            self.tok_ok[seq] = False
            self.pending[seq] = []
        slots: List[int] = []
        copies: List[Tuple[int, int]] = []
        for p in range(start, start + n):
            lb = p // B
            if lb == len(table):
                b = self._pop()
                self.ref[b] = 1
                table.append(b)
            elif table[lb] < 0:
                b = self._pop()
                self.ref[b] = 1
                table[lb] = b
            elif self.ref[table[lb]] > 1:
                old = table[lb]
                b = self._pop()
                copies.append((old, b))
                self.ref[old] -= 1
                self.ref[b] = 1
                table[lb] = b
            slots.append(table[lb] * B + p % B)
        self.lens[seq] = start + n
        return slots, copies

    def fork(self, parent: int, child: int, fork_pos: int) -> None:
        if parent not in self.tables:
            raise AllocatorError(f"unknown sequence {parent}")
        if child in self.tables:
            raise AllocatorError(f"sequence {child} exists")
        if parent in self.swapped:
            raise AllocatorError(f"sequence {parent} is swapped out")
        if not 0 <= fork_pos <= self.lens[parent]:
            raise AllocatorError("fork position outside the parent")
        nb = -(-fork_pos // self.block_size)
        shared = self.tables[parent][:nb]
        for b in shared:
            if b >= 0:
                self.ref[b] += 1
        self.tables[child] = list(shared)
        self.lens[child] = fork_pos
        whole = fork_pos // self.block_size
        ok = self.tok_ok[parent] and fork_pos % self.block_size == 0 and len(self.hashes[parent]) >= whole
        self.tok_ok[child] = ok
        self.hashes[child] = list(self.hashes[parent][:whole]) if ok else []
        self.pending[child] = []

    def _give_back(self, table: List[int]) -> None:
        live = [b for b in table if b >= 0]
        for b in reversed(live):
            if self.ref[b] <= 0:
                raise AllocatorError("reference count underflow")
        for b in reversed(live):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    def release(self, seq: int) -> None:
        if seq not in self.tables:
            raise AllocatorError(f"unknown sequence {seq}")
        self._give_back(self.tables[seq])
        del self.tables[seq]
        del self.lens[seq]
        self.swapped.pop(seq, None)
        for d in (self.tok_ok, self.hashes, self.pending):
            d.pop(seq, None)

    def swap_out(self, seq: int) -> List[int]:
        if seq not in self.tables:
            raise AllocatorError(f"unknown sequence {seq}")
        if seq in self.swapped:
            raise AllocatorError(f"sequence {seq} is already swapped out")
        table = list(self.tables[seq])
        self._give_back(table)
        self.tables[seq] = []
        self.swapped[seq] = [b < 0 for b in table]
        return table

    def swap_in(self, seq: int) -> List[int]:
        if seq not in self.swapped:
            raise AllocatorError(f"sequence {seq} is not swapped out")
        holes = self.swapped[seq]
        n = sum(1 for h in holes if not h)
        if n > len(self.free):
            raise OutOfBlocks(f"need {n} blocks, {len(self.free)} free")
        table = []
        for h in holes:
            if h:
                table.append(-1)
                continue
            b = self._pop()
            self.ref[b] = 1
            table.append(b)
        self.tables[seq] = table
        del self.swapped[seq]
        return list(table)

    def append_tokens(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]], int]:
        """Append tokens with known ids; returns (slots with -1 for cached
        tokens, copies, number of cached tokens)."""
        if seq not in self.tables:
            raise AllocatorError(f"unknown sequence {seq}")
        if seq in self.swapped:
            raise AllocatorError(f"sequence {seq} is swapped out")
        tokens = [int(t) for t in tokens]
        B0, t0, l0 = self.block_size, self.tables[seq], self.lens[seq]
        hole = l0 % B0 != 0 and len(t0) > l0 // B0 and t0[l0 // B0] < 0
        if not self.tok_ok[seq] or hole:  # no hash chain, or a hole where the append starts
            slots, copies = self.append(seq, len(tokens))
            return slots, copies, 0
        B = self.block_size
        table = self.tables[seq]
        start = self.lens[seq]
        n = len(tokens)
        end = start + n
        have = len(table)
        # the blocks that become full, their hashes, and the hits (decided
        # on the cache as it is now)
        filled = []  # (logical block, hash, token ids)
        hit: Dict[int, int] = {}
        cur = list(self.pending[seq])
        prev = self.hashes[seq][-1] if self.hashes[seq] else 0
        chain = True
        for p in range(start, end):
            cur.append(tokens[p - start])
            if len(cur) == B:
                lb = p // B
                h = block_hash(prev, cur)
                filled.append((lb, h, tuple(cur)))
                if lb >= have:
                    b = self.cache.get(h) if chain else None
                    if b is not None and self.cached_as[b][1] == tuple(cur):
                        hit[lb] = b
                    else:
                        chain = False
                prev = h
                cur = []
        # blocks the free list has to give
        cow = n > 0 and start // B < have and self.ref[table[start // B]] > 1
        want = -(-end // B)
        need = int(cow) + sum(1 for lb in range(have, want) if lb not in hit or self.ref[hit[lb]] == 0)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        for lb in range(have, want):
            if lb in hit and self.ref[hit[lb]] == 0:
                self.free.remove(hit[lb])
        copies: List[Tuple[int, int]] = []
        if cow:
            old = table[start // B]
            b = self._pop()
            copies.append((old, b))
            self.ref[old] -= 1
            self.ref[b] = 1
            table[start // B] = b
        for lb in range(have, want):
            if lb in hit:
                b = hit[lb]
                self.ref[b] += 1
            else:
                b = self._pop()
                self.ref[b] = 1
            table.append(b)
        slots = [-1 if (p // B) in hit else table[p // B] * B + p % B for p in range(start, end)]
        for lb, h, toks in filled:
            self.hashes[seq].append(h)
            if lb not in hit and h not in self.cache:
                self.cache[h] = table[lb]
                self.cached_as[table[lb]] = (h, toks)
        self.pending[seq] = cur
        self.lens[seq] = end
        return slots, copies, sum(1 for s in slots if s < 0)

    def trim(self, seq: int, keep_from: int) -> int:
        """Release the blocks wholly before position keep_from; returns how
        many table entries were released."""
        if seq not in self.tables:
            raise AllocatorError(f"unknown sequence {seq}")
        if seq in self.swapped:
            raise AllocatorError(f"sequence {seq} is swapped out")
        if not 0 <= keep_from <= self.lens[seq]:
            raise AllocatorError("trim position outside the sequence")
        table = self.tables[seq]
        upto = min(keep_from // self.block_size, len(table))
        victims = [lb for lb in range(upto) if table[lb] >= 0]
        self._give_back([table[lb] for lb in victims])
        for lb in victims:
            table[lb] = -1
        return len(victims)

    # -- queries ------------------------------------------------------------
    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lens[seq]

    def num_free(self) -> int:
        return len(self.free)

    def used_blocks(self) -> set:
        return {b for b in range(self.num_blocks) if self.ref[b] > 0}

    def shared_prefix_groups(self, seqs: Sequence[int], max_members: int):
        """Groups of a batch for the shared-prefix decode.  A group is a
        sequence and the ones right after it in the batch whose first table
        entry is the same physical block (forks of one prompt hold it
        together: intelliparadigm.com article, section 2.3), at most
        max_members; its shared length is the number of leading table
        entries that are the same live block in every member and lie wholly
        inside every member's context.  A one-member group shares nothing.
        Returns (group_start [num_groups + 1], shared_blocks [num_groups])."""
        B = self.block_size
        starts, shared = [], []
        i, n = 0, len(seqs)
        while i < n:
            first = self.tables[seqs[i]]
            j = i + 1
            while (j < n and j - i < max_members and first and first[0] >= 0
                   and self.tables[seqs[j]] and self.tables[seqs[j]][0] == first[0]):
                j += 1
            k = 0
            if j - i > 1:
                members = seqs[i:j]
                while (k < len(first) and first[k] >= 0
                       and all(k < len(self.tables[m]) and self.tables[m][k] == first[k]
                               and (k + 1) * B <= self.lens[m] for m in members)):
                    k += 1
            starts.append(i)
            shared.append(k)
            i = j
        starts.append(n)
        return starts, shared

    def block_tables(self, seqs: Sequence[int], width: int):
        """Padded [len(seqs), width] table (pad -1) and context lengths."""
        import numpy as np

        t = np.full((len(seqs), max(width, 1)), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            if s in self.swapped:
                raise AllocatorError(f"sequence {s} is swapped out")
            row = self.tables[s]
            if len(row) > width:
                raise AllocatorError("table wider than the padded width")
            t[i, : len(row)] = row
            lens[i] = self.lens[s]
        return t, lens

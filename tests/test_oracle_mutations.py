"""Plant a plausible mistake in the CPU oracle and show that a pin catches it.

Each test swaps one oracle function for a subtly wrong copy (on the CPU,
inside this process only) and asserts that at least one of the pins of
test_oracle_pins.py now fails.  This is what makes the pins trustworthy:
a dropped term, a wrong index or a transposed operand cannot pass them."""
import numpy as np
import pytest

import oracle
from oracle import attention
from oracle.allocator import BlockAllocator

import test_oracle_pins as P


def fails(check, *args):
    try:
        check(*args)
    except AssertionError:
        return True
    return False


def _decode_with(mapping=None, scale_mul=1.0, causal_strict=False, reverse_tokens=False):
    def decode(q, k_pool, v_pool, block_tables, context_lens, scale, dtype):
        qf = attention.to_f64(q, dtype)
        S, Hq, D = qf.shape
        Hkv = k_pool.shape[1]
        G = Hq // Hkv
        sc = float(np.float32(scale)) * scale_mul
        out = np.zeros((S, Hq, D))
        for s in range(S):
            n = int(context_lens[s])
            if n <= 0:
                continue
            K = attention.gather_sequence(k_pool, block_tables[s], n, dtype)
            V = attention.gather_sequence(v_pool, block_tables[s], n, dtype)
            if reverse_tokens:
                V = V[:, ::-1]
            for h in range(Hq):
                g = mapping(h, G, Hkv) if mapping else h // G
                x = sc * (K[g] @ qf[s, h])
                out[s, h] = attention._softmax_weighted(x, V[g])
        return out
    return decode


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(attention, "decode", _decode_with(mapping=lambda h, G, Hkv: h % Hkv))
    assert fails(P.check_gqa_equals_repeated_mha)
    assert fails(P.check_decode_vs_brute_force, P.small_decode_workload(3, G=2))


def test_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(attention, "decode", _decode_with(scale_mul=1.0 / 0.35355339))
    assert fails(P.check_decode_vs_brute_force, P.small_decode_workload(4, G=1))


def test_misaligned_values_are_caught(monkeypatch):
    monkeypatch.setattr(attention, "decode", _decode_with(reverse_tokens=True))
    assert fails(P.check_decode_vs_brute_force, P.small_decode_workload(5, G=1))


def test_wrong_gather_axis_is_caught(monkeypatch):
    def gather(pool, table_row, n, dtype):
        B = pool.shape[2]
        nb = -(-n // B)
        parts = [attention.to_f64(pool[int(b)], dtype) for b in table_row[:nb]]
        full = np.concatenate(parts, axis=1)  # [Hkv, nb*B, D]
        # heads and tokens mixed up: read rows in block-major, head-minor order
        flat = full.transpose(1, 0, 2).reshape(full.shape)
        return flat[:, :n, :]
    monkeypatch.setattr(attention, "gather_sequence", gather)
    assert fails(P.check_decode_vs_brute_force, P.small_decode_workload(6, G=1))


def test_table_ignored_is_caught(monkeypatch):
    real = attention.gather_sequence

    def gather(pool, table_row, n, dtype):
        nb = -(-n // pool.shape[2])
        return real(pool, sorted(int(b) for b in table_row[:nb]), n, dtype)
    monkeypatch.setattr(attention, "gather_sequence", gather)
    assert fails(P.check_decode_vs_brute_force, P.small_decode_workload(8, G=1, lens=(13, 9, 11, 7)))


def test_exclusive_causal_mask_is_caught(monkeypatch):
    def prefill(q, cu, k_pool, v_pool, tables, ctx, scale, dtype):
        qf = attention.to_f64(q, dtype)
        T, Hq, D = qf.shape
        G = Hq // k_pool.shape[1]
        sc = float(np.float32(scale))
        out = np.zeros((T, Hq, D))
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            n = int(ctx[s])
            P_ = n - (b - a)
            K = attention.gather_sequence(k_pool, tables[s], n, dtype)
            V = attention.gather_sequence(v_pool, tables[s], n, dtype)
            pos = P_ + np.arange(b - a)[:, None]
            allowed = np.arange(n)[None, :] < pos
            allowed[:, 0] = True
            for h in range(Hq):
                x = sc * (qf[a:b, h] @ K[h // G].T)
                out[a:b, h] = attention._softmax_weighted(np.where(allowed, x, -np.inf), V[h // G])
        return out
    monkeypatch.setattr(attention, "prefill", prefill)
    assert fails(P.check_prefill_vs_decode)


def test_free_order_mistake_is_caught(monkeypatch):
    def release(self, seq):
        for b in self.tables[seq]:  # forward order: block 0 ends at the bottom
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[seq]
        del self.lens[seq]
    monkeypatch.setattr(BlockAllocator, "release", release)
    assert fails(P.check_free_then_reuse_same_table)


def test_cow_on_unshared_block_is_caught(monkeypatch):
    real = BlockAllocator.append

    def append(self, seq, n):
        # copy the partial last block on every first write, shared or not
        B = self.block_size
        t = self.tables[seq]
        copies = []
        if n and self.lens[seq] % B and self.ref[t[-1]] >= 1:
            old = t[-1]
            b = self.free.pop()
            copies.append((old, b))
            self.ref[old] -= 1
            if self.ref[old] == 0:
                self.free.append(old)
            self.ref[b] = 1
            t[-1] = b
        slots, more = real(self, seq, n)
        return slots, copies + more
    monkeypatch.setattr(BlockAllocator, "append", append)
    assert fails(P.check_fork_cow)


def test_fork_without_refcount_is_caught(monkeypatch):
    def fork(self, parent, child, f):
        nb = -(-f // self.block_size)
        self.tables[child] = list(self.tables[parent][:nb])
        self.lens[child] = f
    monkeypatch.setattr(BlockAllocator, "fork", fork)
    assert fails(P.check_fork_cow)


def test_off_by_one_slot_is_caught(monkeypatch):
    def kv_write(pool, new, slots):
        B = pool.shape[2]
        for t, s in enumerate(slots):
            if s >= 0:
                pool[s // B, :, (s + 1) % B, :] = new[t]
    monkeypatch.setattr(oracle.cache, "kv_write", kv_write)
    assert fails(P.check_kv_write)


def test_copy_in_place_order_is_caught(monkeypatch):
    def copy_blocks(pool, pairs):
        for a, b in pairs:  # no staging: a later pair can read an overwritten source
            pool[b] = pool[a]
    monkeypatch.setattr(oracle.cache, "copy_blocks", copy_blocks)
    assert fails(P.check_copy_blocks)


def test_brute_force_transposed_is_caught(monkeypatch):
    def brute_force(q_rows, k_seq, v_seq, scale, dtype, group=1):
        return attention.brute_force.__wrapped__(q_rows, v_seq, k_seq, scale, dtype, group)
    real = attention.brute_force
    brute_force.__wrapped__ = real
    monkeypatch.setattr(attention, "brute_force", brute_force)
    assert fails(P.check_hand_golden)


def test_swap_in_order_mistake_is_caught(monkeypatch):
    real = oracle.cache.swap_in

    def reversed_swap_in(pool, ids, host):
        real(pool, list(ids)[::-1], host)

    monkeypatch.setattr(oracle.cache, "swap_in", reversed_swap_in)
    assert fails(P.check_swap_roundtrip)


def test_swap_out_keeping_blocks_is_caught(monkeypatch):
    def swap_out_without_release(self, seq):
        table = list(self.tables[seq])
        self.tables[seq] = []
        self.swapped[seq] = len(table)
        return table

    monkeypatch.setattr(BlockAllocator, "swap_out", swap_out_without_release)
    assert fails(P.check_swap_allocator)


def test_unchained_block_hash_is_caught(monkeypatch):
    import oracle.allocator as A
    real = A.block_hash
    monkeypatch.setattr(A, "block_hash", lambda prev, toks: real(0, toks))
    assert fails(P.check_prefix_cache)


def test_block_hash_over_part_of_the_block_is_caught(monkeypatch):
    """A hash that skips the chain and the block's first token."""
    import oracle.allocator as A
    real = A.block_hash
    monkeypatch.setattr(A, "block_hash", lambda prev, toks: real(0, toks[1:]))
    assert fails(P.check_prefix_cache)


def test_window_off_by_one_is_caught(monkeypatch):
    real = attention.decode

    def wider(q, k, v, t, c, scale, dtype, window=0):
        return real(q, k, v, t, c, scale, dtype, window=window + 1 if window > 0 else 0)

    monkeypatch.setattr(attention, "decode", wider)
    assert fails(P.check_window_decode)


def _to_f64_with(shift=16, as_fp16=False):
    real = attention.to_f64

    def to_f64(raw, dtype):
        if dtype != "bf16":
            return real(raw, dtype)
        u = np.asarray(raw, dtype=np.uint16)
        if as_fp16:
            return u.view(np.float16).astype(np.float64)
        return (u.astype(np.uint32) << np.uint32(shift)).view(np.float32).astype(np.float64)
    return to_f64


def test_bf16_shift_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(attention, "to_f64", _to_f64_with(shift=15))
    assert fails(P.check_bf16_decoding)


def test_bf16_read_as_fp16_is_caught(monkeypatch):
    monkeypatch.setattr(attention, "to_f64", _to_f64_with(as_fp16=True))
    assert fails(P.check_bf16_decoding)


def test_shared_prefix_past_a_member_context_is_caught(monkeypatch):
    """A grouping that shares a block some member's context ends inside."""
    def groups(self, seqs, max_members):
        starts, shared = [], []
        i, n = 0, len(seqs)
        while i < n:
            first = self.tables[seqs[i]]
            j = i + 1
            while j < n and j - i < max_members and first and self.tables[seqs[j]][:1] == first[:1]:
                j += 1
            k = 0
            if j - i > 1:
                while k < len(first) and all(k < len(self.tables[m]) and self.tables[m][k] == first[k]
                                             for m in seqs[i:j]):
                    k += 1
            starts.append(i)
            shared.append(k)
            i = j
        starts.append(n)
        return starts, shared
    monkeypatch.setattr(BlockAllocator, "shared_prefix_groups", groups)
    assert fails(P.check_shared_prefix_groups)

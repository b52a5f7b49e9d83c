"""Attention over a paged K/V cache, evaluated in float64 from its definition.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check, the benchmark's CPU
baseline).

Paging changes where K and V are stored, never the result: attention is
softmax(q K^T * scale) V over the sequence's tokens (cnblogs "paged
attention", sections 5 and 6; "08. PagedAttention", section "what it does not
solve": decode still reads the whole history, only its location changes).
So each function here follows the block table to assemble the sequence's
K and V contiguously, then applies that formula directly in float64 from the
exact stored values.  No tiling, splitting or online softmax.

Readings (the pages are silent on these):

* ``context_lens[s]`` counts every token attended, including the one this
  step wrote; a context of 0 gives an all-zero output.
* Query head h reads KV head h // (H_q / H_kv) (contiguous grouping; the
  cnblogs article, section 6, lists grouped-query attention as combinable).
* Prefill: query i of a chunk of C tokens in a sequence with context n sits
  at position n - C + i and attends keys 0..n - C + i inclusive.
* ``scale`` is used exactly as the float32 value the GPU receives.
"""
from __future__ import annotations

import math

import numpy as np


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw element bits (or float32 values) -> float64, exactly."""
    if dtype == "bf16":
        return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    a = np.asarray(raw)
    if a.dtype == np.uint32:
        a = a.view(np.float32)
    return a.astype(np.float64)


def gather_sequence(pool: np.ndarray, table_row, n: int, dtype: str) -> np.ndarray:
    """Follow the block table: logical block lb -> physical block
    table_row[lb]; return the first n tokens as float64 [num_kv_heads, n, D]."""
    B = pool.shape[2]
    nb = -(-n // B)
    blocks = [int(b) for b in table_row[:nb]]
    parts = [to_f64(pool[b], dtype) for b in blocks]  # each [Hkv, B, D]
    if not parts:
        return np.zeros((pool.shape[1], 0, pool.shape[3]))
    return np.concatenate(parts, axis=1)[:, :n, :]


def gather_range(pool: np.ndarray, table_row, lo: int, n: int, dtype: str) -> np.ndarray:
    """Tokens lo .. n-1 of a sequence, one at a time through the table
    (token t sits in physical block table_row[t // B] at offset t % B):
    float64 [num_kv_heads, n - lo, D].  Blocks before lo are never touched."""
    B = pool.shape[2]
    rows = [to_f64(pool[int(table_row[t // B]), :, t % B, :], dtype) for t in range(lo, n)]
    if not rows:
        return np.zeros((pool.shape[1], 0, pool.shape[3]))
    return np.stack(rows, axis=1)


def _softmax_weighted(scores: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax over the last axis of ``scores`` applied to rows of ``v``."""
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return (e / e.sum(axis=-1, keepdims=True)) @ v


def decode(q, k_pool, v_pool, block_tables, context_lens, scale, dtype, window: int = 0) -> np.ndarray:
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over context_lens[s]
    tokens, or over the last ``window`` of them when window > 0 (a sliding
    window: intelliparadigm.com article, section 5.2).  q: [S, Hq, D] raw;
    returns float64 [S, Hq, D]."""
    qf = to_f64(q, dtype)
    S, Hq, D = qf.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((S, Hq, D))
    for s in range(S):
        n = int(context_lens[s])
        if n <= 0:
            continue
        if window > 0:
            lo = max(0, n - window)
            K = gather_range(k_pool, block_tables[s], lo, n, dtype)
            V = gather_range(v_pool, block_tables[s], lo, n, dtype)
        else:
            K = gather_sequence(k_pool, block_tables[s], n, dtype)
            V = gather_sequence(v_pool, block_tables[s], n, dtype)
        for h in range(Hq):
            g = h // G
            x = sc * (K[g] @ qf[s, h])
            out[s, h] = _softmax_weighted(x, V[g])
    return out


def prefill(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, scale, dtype) -> np.ndarray:
    """Causal chunk attention: q packed [sum C_s, Hq, D]; query i of sequence
    s attends its first context_lens[s] - C_s + i + 1 tokens."""
    qf = to_f64(q, dtype)
    T, Hq, D = qf.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((T, Hq, D))
    S = len(cu_q_lens) - 1
    for s in range(S):
        a, b = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        C = b - a
        n = int(context_lens[s])
        if C <= 0 or n <= 0:
            continue
        P = n - C
        K = gather_sequence(k_pool, block_tables[s], n, dtype)
        V = gather_sequence(v_pool, block_tables[s], n, dtype)
        pos = P + np.arange(C)[:, None]
        allowed = np.arange(n)[None, :] <= pos  # [C, n]
        for h in range(Hq):
            g = h // G
            x = sc * (qf[a:b, h] @ K[g].T)
            x = np.where(allowed, x, -np.inf)
            out[a:b, h] = _softmax_weighted(x, V[g])
    return out


def brute_force(q_rows, k_seq, v_seq, scale, dtype, group=1) -> np.ndarray:
    """Textbook attention on never-paged, contiguous K/V, with explicit loops
    (tiny inputs only).  q_rows: [Hq, D]; k_seq, v_seq: [n, Hkv, D] raw.
    Returns float64 [Hq, D]."""
    q = to_f64(q_rows, dtype)
    k = to_f64(k_seq, dtype)
    v = to_f64(v_seq, dtype)
    Hq, D = q.shape
    n = k.shape[0]
    sc = float(np.float32(scale))
    out = np.zeros((Hq, D))
    for h in range(Hq):
        g = h // group
        scores = []
        for t in range(n):
            acc = 0.0
            for d in range(D):
                acc += q[h, d] * k[t, g, d]
            scores.append(acc * sc)
        if not scores:
            continue
        mx = max(scores)
        w = [math.exp(x - mx) for x in scores]
        tot = sum(w)
        for d in range(D):
            out[h, d] = sum(w[t] * v[t, g, d] for t in range(n)) / tot
    return out

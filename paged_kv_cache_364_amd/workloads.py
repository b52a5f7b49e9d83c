"""Seeded synthetic workloads for paged KV-cache attention.

This module only *generates inputs*: sequence lengths, the order in which
physical blocks come off the free list, allocator operation scripts
(add / append / fork / free), and random query / key / value values.  It
contains none of the arithmetic of the method itself (no slot formula, no
attention, no allocation policy); both the CPU oracle and the GPU path consume
its output and execute the scripts with their own code.

Shapes follow the pages' workloads:

* Llama-3.1-8B attention shape (32 query heads, 8 KV heads, head_dim 128),
  16-token blocks and a 25,600-block pool per layer, from "08. PagedAttention"
  (niuwancheng.cn), section "how much waste remains" (128 KiB per token over
  32 layers, 2 MiB per block, 50 GiB / 2 MiB = 25,600 blocks).
* OPT-13B attention shape (40 heads, head_dim 5120 / 40 = 128) from the
  intelliparadigm.com article, section 1 (about 800 KB of KV per token).
* The tiny block-size-4 case from the cnblogs article, section 8.

Values are standard normal in float32; bf16 workloads round them to bf16
with round-to-nearest-even and keep the raw 16-bit patterns, so both sides
read identical bits.  Draw order is fixed: (1) lengths and structure,
(2) physical placement, (3) queries, (4) cached K/V in (sequence, position)
order, (5) the new token's K/V.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_bits(x) if dtype == BF16 else x


@dataclass
class Op:
    """One allocator operation.  ``append`` carries the K/V rows it writes
    (``[n, num_kv_heads, head_dim]`` raw values) or ``None`` when the tokens'
    contents do not matter (churn fillers, whose slots stay poisoned)."""

    kind: str  # "add" | "append" | "fork" | "free"
    seq: int
    n: int = 0
    parent: int = -1
    fork_pos: int = 0
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    tokens: Optional[np.ndarray] = None  # token ids: the append goes through the prefix cache


@dataclass
class Step:
    """A batch of operations.  Executing a step means: run the allocator ops
    in order, then copy every copy-on-write pair they produced, then write
    the K/V rows of every append."""

    ops: List[Op] = field(default_factory=list)


@dataclass
class Workload:
    name: str
    kind: str  # "decode" | "prefill"
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: np.float32
    init_order: np.ndarray  # int32 permutation: order blocks leave the free list
    steps: List[Step]
    batch: List[int]  # sequence ids, in batch order
    q: np.ndarray  # decode: [S, Hq, D]; prefill: [sum C_s, Hq, D] packed
    q_lens: Optional[List[int]] = None  # prefill chunk length per sequence
    max_blocks_per_seq: int = 0
    notes: str = ""

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    def seq_tokens(self) -> dict:
        """Per-sequence contiguous K/V (token order) built from the script's
        appends and forks, independent of any paging: {seq: (K, V)} with
        K, V shaped [len, num_kv_heads, head_dim] raw values.  Tokens whose
        contents were never given (fillers) are absent from the result."""
        seqs: dict = {}
        for st in self.steps:
            for op in st.ops:
                if op.kind == "add":
                    seqs[op.seq] = ([], [])
                elif op.kind == "append":
                    if op.k is not None:
                        seqs[op.seq][0].append(op.k)
                        seqs[op.seq][1].append(op.v)
                elif op.kind == "fork":
                    pk = np.concatenate(seqs[op.parent][0]) if seqs[op.parent][0] else None
                    pv = np.concatenate(seqs[op.parent][1]) if seqs[op.parent][1] else None
                    if pk is None:
                        seqs[op.seq] = ([], [])
                    else:
                        seqs[op.seq] = ([pk[: op.fork_pos]], [pv[: op.fork_pos]])
                elif op.kind == "free":
                    seqs.pop(op.seq, None)
        out = {}
        for s, (ks, vs) in seqs.items():
            if ks:
                out[s] = (np.concatenate(ks), np.concatenate(vs))
        return out


def _scale(head_dim: int) -> np.float32:
    return np.float32(1.0 / np.sqrt(np.float64(head_dim)))


def _decode_script(rng, lens, hkv, d, dtype, seq_ids):
    """History (len-1 tokens per sequence) then one decode token each."""
    hist = [int(n) - 1 for n in lens]
    tot = sum(hist)
    kh = _values(rng, (tot, hkv, d), dtype)
    vh = _values(rng, (tot, hkv, d), dtype)
    kn = _values(rng, (len(lens), hkv, d), dtype)
    vn = _values(rng, (len(lens), hkv, d), dtype)
    pre = Step()
    off = 0
    for s, n in zip(seq_ids, hist):
        pre.ops.append(Op("add", s))
        if n > 0:
            pre.ops.append(Op("append", s, n=n, k=kh[off: off + n], v=vh[off: off + n]))
        off += n
    new = Step([Op("append", s, n=1, k=kn[i: i + 1], v=vn[i: i + 1]) for i, s in enumerate(seq_ids)])
    return [pre, new]


def decode_workload(name, seed, lens, *, num_heads, num_kv_heads, head_dim, block_size,
                    num_blocks, dtype, scale=None, churn_ops=0, max_blocks_per_seq=None,
                    notes=""):
    """Generic decode workload: one sequence per entry of ``lens`` (context
    length including the token written by this step), physical placement a
    seeded permutation of the pool, or identity order followed by seeded
    alloc/free churn when ``churn_ops`` > 0."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    steps: List[Step] = []
    if churn_ops:
        init_order = np.arange(num_blocks, dtype=np.int32)
        steps.append(_churn_step(rng, num_blocks, block_size, lens, churn_ops))
    else:
        init_order = rng.permutation(num_blocks).astype(np.int32)
    seq_ids = list(range(len(lens)))
    q = _values(rng, (len(lens), num_heads, head_dim), dtype)
    steps += _decode_script(rng, lens, num_kv_heads, head_dim, dtype, seq_ids)
    mb = max_blocks_per_seq or max(1, max(-(-n // block_size) for n in lens))
    return Workload(name, "decode", dtype, num_heads, num_kv_heads, head_dim, block_size,
                    num_blocks, np.float32(scale) if scale is not None else _scale(head_dim),
                    init_order, steps, seq_ids, q, max_blocks_per_seq=mb, notes=notes)


CHURN_SEQ_BASE = 1_000_000


def _churn_step(rng, num_blocks, block_size, lens, n_ops):
    """Seeded alloc/free churn with filler sequences that stay live.  Each op
    allocates a filler of U{1..64} blocks with probability 1/2 (skipped if it
    would leave fewer free blocks than the real batch will take), else frees a
    uniformly chosen live filler."""
    need = sum(-(-n // block_size) for n in lens)
    free = num_blocks
    live: List[tuple] = []
    nxt = CHURN_SEQ_BASE
    st = Step()
    for _ in range(n_ops):
        if rng.random() < 0.5:
            nb = int(rng.integers(1, 65))
            if free - nb >= need:
                st.ops.append(Op("add", nxt))
                st.ops.append(Op("append", nxt, n=nb * block_size))
                live.append((nxt, nb))
                free -= nb
                nxt += 1
        elif live:
            i = int(rng.integers(0, len(live)))
            s, nb = live.pop(i)
            st.ops.append(Op("free", s))
            free += nb
    return st


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

LLAMA = dict(num_heads=32, num_kv_heads=8, head_dim=128)
OPT13B = dict(num_heads=40, num_kv_heads=40, head_dim=128)


def tiny_f32_decode():
    """Tiny fp32 decode: context lengths {10, 3, 17, 1}, 2 heads, head_dim 16,
    block size 4, 32-block pool in seeded random order, scale 1/sqrt(16)."""
    return decode_workload("tiny-f32-decode", 1, [10, 3, 17, 1], num_heads=2, num_kv_heads=2,
                           head_dim=16, block_size=4, num_blocks=32, dtype=F32,
                           scale=np.float32(0.25))


def llama_decode(seed=2, num_seqs=64, lo=128, hi=2048, num_blocks=25_600, name=None, block_size=16):
    """Llama-3.1-8B-shaped decode, batch ``num_seqs``, context ~ U{lo..hi}.
    The same seed gives the same lengths and values for any block size."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=num_seqs)
    wl = decode_workload(name or f"llama31-8b-decode-b{num_seqs}", rng.integers(1 << 62), lens,
                         **LLAMA, block_size=block_size, num_blocks=num_blocks, dtype=BF16,
                         max_blocks_per_seq=-(-hi // block_size))
    return wl


def llama_decode_b64():
    return llama_decode(2, 64, 128, 2048, 25_600, "llama31-8b-decode-b64")


def ragged_lens(rng, num_seqs, median=500.0, sigma=1.0, lo=1, hi=8192):
    ln = rng.normal(np.log(median), sigma, size=num_seqs)
    return np.clip(np.rint(np.exp(ln)), lo, hi).astype(np.int64)


def ragged_decode(seed=3, num_seqs=256, num_blocks=25_600, churn_ops=2000, hi=8192, name=None):
    """Ragged long-context decode: log-normal lengths (median 500, sigma 1,
    clipped to [1, hi]) over a free list fragmented by seeded churn."""
    rng = np.random.default_rng(seed)
    lens = ragged_lens(rng, num_seqs, hi=hi)
    return decode_workload(name or f"llama31-8b-ragged-b{num_seqs}", rng.integers(1 << 62), lens,
                           **LLAMA, block_size=16, num_blocks=num_blocks, dtype=BF16,
                           churn_ops=churn_ops, max_blocks_per_seq=-(-hi // 16))


def llama_ragged_b256():
    return ragged_decode(3, 256, 25_600, 2000, 8192, "llama31-8b-ragged-b256")


PROMPT_SEQ_BASE = 10_000


def shared_prefix(seed=4, num_prompts=32, prompt_len=1024, n_branches=4, fork_lo=1000,
                  fork_hi=1023, priv_hi=256, num_blocks=25_600, name=None, fork_points=None, block_size=16,
                  heads=None):
    """Parallel sampling: each prompt is forked into ``n_branches`` branches at
    a point f drawn uniformly from fork_lo..fork_hi minus the multiples of the
    block size; the prompt is then released, so the
    branches hold the shared blocks alone.  Each branch writes p ~ U{0..priv_hi}
    private tokens, then one decode token (context f + p + 1)."""
    rng = np.random.default_rng(seed)
    bsz = block_size
    hd = dict(LLAMA) if heads is None else dict(heads)
    hkv, d = hd["num_kv_heads"], hd["head_dim"]
    if fork_points is None:
        # uniform over the fork points inside a block, so that every branch's
        # first write lands in a shared, partly filled block and forces a
        # copy (block-aligned forks are exercised with explicit fork_points)
        cands = np.array([f for f in range(fork_lo, fork_hi + 1) if f % bsz], dtype=np.int64)
        if len(cands) == 0:
            cands = np.arange(fork_lo, fork_hi + 1, dtype=np.int64)
        forks = cands[rng.integers(0, len(cands), size=num_prompts)]
    else:
        forks = np.asarray(fork_points, dtype=np.int64)
        assert len(forks) == num_prompts
    nseq = num_prompts * n_branches
    priv = rng.integers(0, priv_hi + 1, size=nseq)
    init_order = rng.permutation(num_blocks).astype(np.int32)
    q = _values(rng, (nseq, hd["num_heads"], d), BF16)
    kp = _values(rng, (num_prompts, prompt_len, hkv, d), BF16)
    vp = _values(rng, (num_prompts, prompt_len, hkv, d), BF16)
    tot = int(priv.sum())
    kx = _values(rng, (tot, hkv, d), BF16)
    vx = _values(rng, (tot, hkv, d), BF16)
    kn = _values(rng, (nseq, hkv, d), BF16)
    vn = _values(rng, (nseq, hkv, d), BF16)
    a = Step()
    for i in range(num_prompts):
        p = PROMPT_SEQ_BASE + i
        a.ops += [Op("add", p), Op("append", p, n=prompt_len, k=kp[i], v=vp[i])]
    b = Step()
    for i in range(num_prompts):
        p = PROMPT_SEQ_BASE + i
        for j in range(n_branches):
            b.ops.append(Op("fork", i * n_branches + j, parent=p, fork_pos=int(forks[i])))
        b.ops.append(Op("free", p))
    c = Step()
    off = 0
    for s in range(nseq):
        n = int(priv[s])
        if n:
            c.ops.append(Op("append", s, n=n, k=kx[off: off + n], v=vx[off: off + n]))
        off += n
    dstep = Step([Op("append", s, n=1, k=kn[s: s + 1], v=vn[s: s + 1]) for s in range(nseq)])
    mb = -(-(fork_hi + priv_hi + 1) // bsz)
    return Workload(name or f"llama31-8b-shared-prefix-{num_prompts}x{n_branches}", "decode", BF16,
                    **hd, block_size=bsz, num_blocks=num_blocks, scale=_scale(d),
                    init_order=init_order, steps=[a, b, c, dstep], batch=list(range(nseq)), q=q,
                    max_blocks_per_seq=mb)


def llama_shared_prefix_32x4():
    return shared_prefix(4, 32, 1024, 4, 1000, 1023, 256, 25_600, "llama31-8b-shared-prefix-32x4")


def prefill_workload(seed=5, num_seqs=16, prefix_hi=1536, chunk=512, num_blocks=4096,
                     heads=OPT13B, name=None, prefix_lens=None, chunk_lens=None, block_size=16):
    """Paged prefill: each sequence has a cached prefix P ~ U{0..prefix_hi}
    and a new causal query chunk of ``chunk`` tokens whose K/V are written
    first; the chunk then attends over prefix + chunk."""
    rng = np.random.default_rng(seed)
    if prefix_lens is None:
        pl = rng.integers(0, prefix_hi + 1, size=num_seqs)
    else:
        pl = np.asarray(prefix_lens, dtype=np.int64)
    cl = [chunk] * num_seqs if chunk_lens is None else [int(c) for c in chunk_lens]
    hq, hkv, d = heads["num_heads"], heads["num_kv_heads"], heads["head_dim"]
    init_order = rng.permutation(num_blocks).astype(np.int32)
    q = _values(rng, (int(sum(cl)), hq, d), BF16)
    tot = int(pl.sum())
    kh = _values(rng, (tot, hkv, d), BF16)
    vh = _values(rng, (tot, hkv, d), BF16)
    totc = int(sum(cl))
    kc = _values(rng, (totc, hkv, d), BF16)
    vc = _values(rng, (totc, hkv, d), BF16)
    a = Step()
    off = 0
    for s in range(num_seqs):
        a.ops.append(Op("add", s))
        n = int(pl[s])
        if n:
            a.ops.append(Op("append", s, n=n, k=kh[off: off + n], v=vh[off: off + n]))
        off += n
    b = Step()
    off = 0
    for s in range(num_seqs):
        n = cl[s]
        if n:
            b.ops.append(Op("append", s, n=n, k=kc[off: off + n], v=vc[off: off + n]))
        off += n
    mb = max(-(-(int(p) + c) // block_size) for p, c in zip(pl, cl)) if num_seqs else 1
    return Workload(name or f"opt13b-prefill-b{num_seqs}x{chunk}", "prefill", BF16, hq, hkv, d, block_size,
                    num_blocks, _scale(d), init_order, [a, b], list(range(num_seqs)), q,
                    q_lens=cl, max_blocks_per_seq=max(mb, 1))


def opt13b_prefill_b16x512():
    return prefill_workload(5, 16, 1536, 512, 4096, OPT13B, "opt13b-prefill-b16x512")


def shared_prompt_requests(seed=6, num_requests=16, prompt_len=1000, suffix_hi=200, num_blocks=4096,
                           block_size=16, vocab=32000, use_cache=True, name=None):
    """Requests that share a system prompt (cnblogs section 9): request r is
    the prompt followed by its own suffix of U{1..suffix_hi} tokens, then one
    decode token.  A token's K/V depend only on the token ids up to it, so
    the prompt's K/V are drawn once and every request carries the same rows
    for it.  With ``use_cache`` the appends carry token ids (prefix caching);
    without, the same script uses plain appends."""
    rng = np.random.default_rng(seed)
    hkv, d = LLAMA["num_kv_heads"], LLAMA["head_dim"]
    suffix = rng.integers(1, suffix_hi + 1, size=num_requests)
    init_order = rng.permutation(num_blocks).astype(np.int32)
    q = _values(rng, (num_requests, LLAMA["num_heads"], d), BF16)
    prompt_tok = rng.integers(0, vocab, size=prompt_len).astype(np.int32)
    kp = _values(rng, (prompt_len, hkv, d), BF16)
    vp = _values(rng, (prompt_len, hkv, d), BF16)
    tot = int(suffix.sum())
    sfx_tok = rng.integers(0, vocab, size=tot + num_requests).astype(np.int32)
    ks = _values(rng, (tot, hkv, d), BF16)
    vs = _values(rng, (tot, hkv, d), BF16)
    kn = _values(rng, (num_requests, hkv, d), BF16)
    vn = _values(rng, (num_requests, hkv, d), BF16)
    a = Step()
    off = 0
    for r in range(num_requests):
        n = int(suffix[r])
        toks = np.concatenate([prompt_tok, sfx_tok[off: off + n]])
        a.ops += [Op("add", r), Op("append", r, n=prompt_len + n, k=np.concatenate([kp, ks[off: off + n]]),
                                   v=np.concatenate([vp, vs[off: off + n]]), tokens=toks if use_cache else None)]
        off += n
    b = Step([Op("append", r, n=1, k=kn[r: r + 1], v=vn[r: r + 1],
                 tokens=sfx_tok[tot + r: tot + r + 1] if use_cache else None) for r in range(num_requests)])
    mb = -(-(prompt_len + suffix_hi + 1) // block_size)
    return Workload(name or f"llama31-8b-shared-prompt-{num_requests}x{prompt_len}", "decode", BF16, **LLAMA,
                    block_size=block_size, num_blocks=num_blocks, scale=_scale(d), init_order=init_order,
                    steps=[a, b], batch=list(range(num_requests)), q=q, max_blocks_per_seq=mb)


# the five seeded workloads, by name
WORKLOADS = {f.__name__: f for f in (tiny_f32_decode, llama_decode_b64, llama_ragged_b256, llama_shared_prefix_32x4,
                                     opt13b_prefill_b16x512)}

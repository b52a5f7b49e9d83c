"""HIP prefill (matrix-core path) against the CPU oracle: a causal query
chunk over a cached prefix, read through the block table.  bf16 inputs,
max absolute error <= 2e-2 against the float64 oracle on the same bf16
values."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import runner as oracle_runner  # noqa: E402
from paged_kv_cache_364_amd import api, driver, workloads as W  # noqa: E402

BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    yield


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(wl):
    say(f"[gpu] {wl.name}: script")
    st = driver.run_script(wl)
    ost = oracle_runner.run(wl)
    assert np.array_equal(st.tables, ost.tables) and np.array_equal(st.context_lens, ost.context_lens)
    torch.cuda.synchronize()
    assert np.array_equal(driver.pool_bits(st.k_pool), ost.k_pool), "k_cache differs"
    assert np.array_equal(driver.pool_bits(st.v_pool), ost.v_pool), "v_cache differs"
    say(f"[gpu] {wl.name}: prefill")
    out = driver.run_attention(wl, st)
    torch.cuda.synchronize()
    got = driver.out_to_f64(out)
    exp = oracle_runner.expected(wl, ost)
    assert np.isfinite(got).all(), "non-finite output"
    err = float(np.abs(got - exp).max())
    say(f"[gpu] {wl.name}: max abs err {err:.3g}")
    assert err <= BF16_TOL, err
    return st, out


def small(name, seed, prefix_lens, chunk_lens, hq, hkv, d, b, num_blocks=None):
    need = sum(-(-(p + c) // b) for p, c in zip(prefix_lens, chunk_lens))
    return W.prefill_workload(seed, len(prefix_lens), 0, 0, num_blocks or need + 8,
                              dict(num_heads=hq, num_kv_heads=hkv, head_dim=d), name,
                              prefix_lens=prefix_lens, chunk_lens=chunk_lens, block_size=b)


def test_prefill_small_mha():
    # chunks of 1, 31, 32, 33, 128, 130 and 300 rows; prefixes on and off block and tile edges
    check(small("pf-mha", 51, [0, 37, 64, 15, 0, 200, 129], [1, 31, 32, 33, 128, 130, 300], 4, 4, 128, 16))


@pytest.mark.parametrize("hq,hkv,d,b", [
    (8, 2, 128, 16), (8, 2, 64, 16), (4, 4, 64, 8), (6, 3, 128, 32), (4, 1, 128, 64), (2, 2, 64, 1),
    (8, 8, 128, 4), (8, 2, 128, 128), (4, 4, 64, 256),
])
def test_prefill_variants(hq, hkv, d, b):
    check(small(f"pf-{hq}-{hkv}-{d}-{b}", 60 + hq + d + b, [0, 5, 100, 63], [17, 64, 77, 129], hq, hkv, d, b))


def test_prefill_empty_chunks_and_single_token():
    """Chunks of zero rows, with and without a cached prefix, between others,
    and a sequence whose whole context is its chunk's single row."""
    check(small("pf-empty", 77, [10, 0, 40, 0, 7], [5, 0, 33, 1, 0], 4, 2, 64, 16))


def test_prefill_long_tables_block_size_1():
    """Block size 1 (a block holds fewer keys than one 1 KiB transfer covers,
    so every lane looks up its own block) and contexts past 1024 blocks."""
    check(small("pf-window", 91, [1100, 2500, 0], [50, 140, 1200], 4, 2, 64, 1))


@pytest.mark.parametrize("n,hq,hkv,d", [(80, 8, 2, 128), (64, 4, 4, 64)])
def test_prefill_many_items_per_workgroup(n, hq, hkv, d):
    """More (sequence, head, q tile) items than workgroups, of mixed sizes
    (one-tile items, empty second q tiles, prefixes 0..300): each workgroup
    streams several items and the transfers run across item ends.  80
    sequences take the batch order, 64 the ranked order."""
    rng = np.random.default_rng(1000 + n)
    prefix = [int(x) for x in rng.integers(0, 301, n)]
    chunk = [int(x) for x in rng.integers(1, 301, n)]
    check(small(f"pf-items-{n}", 95 + n, prefix, chunk, hq, hkv, d, 16))


def test_prefill_opt13b_full():
    """16 sequences, prefix U{0..1536}, 512-token chunk, 40 heads, head_dim 128."""
    check(W.opt13b_prefill_b16x512())


def test_prefill_rows_match_decode():
    """Row i of a prefill chunk is the decode output at context P + i + 1."""
    wl = small("pf-vs-decode", 71, [40, 0], [70, 50], 8, 2, 128, 16)
    st, out = check(wl)
    q = driver.to_device(wl.q, "bf16", "cuda")
    rows, lens, tabs = [], [], []
    cu = driver.cu_lens(wl.q_lens)
    for s in range(2):
        P = int(st.context_lens[s]) - wl.q_lens[s]
        for i in range(wl.q_lens[s]):
            rows.append(int(cu[s]) + i)
            lens.append(P + i + 1)
            tabs.append(st.tables[s])
    qd = q[rows].contiguous()
    od = torch.empty_like(qd)
    api.paged_attention_decode(od, qd, st.k_pool, st.v_pool, torch.from_numpy(np.stack(tabs)).cuda(),
                               torch.tensor(lens, dtype=torch.int32, device="cuda"), float(wl.scale))
    torch.cuda.synchronize()
    diff = (od.float() - out[rows].float()).abs().max().item()
    say(f"[gpu] prefill vs decode rows: max diff {diff:.3g}")
    assert diff <= 2 * BF16_TOL


def test_prefill_out_of_range_block_gives_nan_rows_only():
    wl = small("pf-badblock", 81, [32, 40], [32, 40], 4, 4, 128, 16)
    st = driver.run_script(wl)
    tb = st.tables_dev.clone()
    tb[1, 0] = 1 << 30  # keys 0..15 of sequence 1 unreachable
    q = driver.to_device(wl.q, "bf16", "cuda")
    out = torch.empty_like(q)
    cu = torch.from_numpy(driver.cu_lens(wl.q_lens)).cuda()
    api.paged_attention_prefill(out, q, cu, max(wl.q_lens), st.k_pool, st.v_pool, tb, st.lens_dev,
                                float(wl.scale))
    torch.cuda.synchronize()
    o = out.float()
    assert torch.isfinite(o[:32]).all()
    assert torch.isnan(o[32:]).all()


def test_prefill_ignores_table_padding():
    """Entries past a sequence's last block may hold anything (in-pool ids,
    ids outside the pool, negatives): the outputs are bitwise those of the
    table padded with -1."""
    wl = small("pf-padding", 88, [37, 5, 0], [20, 70, 33], 4, 2, 128, 16, num_blocks=64)
    st = driver.run_script(wl)
    q = driver.to_device(wl.q, "bf16", "cuda")
    cu = torch.from_numpy(driver.cu_lens(wl.q_lens)).cuda()
    scale = float(wl.scale)
    ref = torch.empty_like(q)
    api.paged_attention_prefill(ref, q, cu, max(wl.q_lens), st.k_pool, st.v_pool, st.tables_dev, st.lens_dev, scale)
    tb = st.tables_dev.clone()
    junk = torch.tensor([3, 1 << 30, -7, 63, 0, -1, 2 ** 31 - 1], dtype=torch.int32, device="cuda")
    for s in range(tb.shape[0]):
        used = -(-int(st.context_lens[s]) // wl.block_size)
        for i in range(used, tb.shape[1]):
            tb[s, i] = junk[(s + i) % junk.numel()]
    out = torch.empty_like(q)
    api.paged_attention_prefill(out, q, cu, max(wl.q_lens), st.k_pool, st.v_pool, tb, st.lens_dev, scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_prefill_out_of_range_block_after_some_rows():
    """A block outside the pool that only the later rows of a chunk reach:
    the rows before it match the oracle (the bad keys are masked for them,
    and a masked key's value row must not leak NaN), the rows from it on
    are NaN."""
    wl = small("pf-badblock-mid", 82, [0, 24], [40, 20], 4, 4, 128, 16)
    st = driver.run_script(wl)
    ost = oracle_runner.run(wl)
    exp = oracle_runner.expected(wl, ost)
    tb = st.tables_dev.clone()
    tb[0, 1] = 1 << 30  # keys 16..31 of sequence 0 unreachable
    q = driver.to_device(wl.q, "bf16", "cuda")
    out = torch.empty_like(q)
    cu = torch.from_numpy(driver.cu_lens(wl.q_lens)).cuda()
    say("[gpu] pf-badblock-mid: prefill")
    api.paged_attention_prefill(out, q, cu, max(wl.q_lens), st.k_pool, st.v_pool, tb, st.lens_dev,
                                float(wl.scale))
    torch.cuda.synchronize()
    got = driver.out_to_f64(out)
    # sequence 0 (prefix 0): rows 0..15 never attend keys 16..31
    assert np.isfinite(got[:16]).all()
    assert float(np.abs(got[:16] - exp[:16]).max()) <= BF16_TOL
    assert np.isnan(got[16:40]).all()
    # sequence 1 is untouched
    assert float(np.abs(got[40:] - exp[40:]).max()) <= BF16_TOL


def test_prefill_chunk_longer_than_max_q_len_gives_nan_rows():
    """max_q_len smaller than a chunk: the launch covers 256-row q tiles up
    to max_q_len; rows of a longer chunk past that come out NaN, every other
    row matches the oracle."""
    wl = small("pf-overflow", 83, [10, 3], [300, 40], 4, 2, 128, 16)
    st = driver.run_script(wl)
    ost = oracle_runner.run(wl)
    exp = oracle_runner.expected(wl, ost)
    q = driver.to_device(wl.q, "bf16", "cuda")
    out = torch.zeros_like(q)
    cu = torch.from_numpy(driver.cu_lens(wl.q_lens)).cuda()
    say("[gpu] pf-overflow: prefill with max_q_len 200")
    api.paged_attention_prefill(out, q, cu, 200, st.k_pool, st.v_pool, st.tables_dev, st.lens_dev,
                                float(wl.scale))
    torch.cuda.synchronize()
    got = driver.out_to_f64(out)
    assert float(np.abs(got[:256] - exp[:256]).max()) <= BF16_TOL
    assert np.isnan(got[256:300]).all()
    assert float(np.abs(got[300:] - exp[300:]).max()) <= BF16_TOL

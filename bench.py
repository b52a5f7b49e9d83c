"""Paged decode attention benchmark (Llama-3.1-8B attention shape), with a
paged prefill leg (OPT-13B shape).

Decode step = the device work of one decode step of one layer for the whole
batch: the 64 new tokens' K/V written into their slots and the decode (main
pass + log-sum-exp merge) over the paged cache, issued as one call,
``paged_attention_decode_append``, whose results are bit for bit those of
``kv_write`` then ``paged_attention_decode``; the two-call step is timed
too and reported beside it.  Block tables and slot mappings come from the
C++ block allocator and are resident on the device before timing starts.  Layers rotate over
separate per-layer pools (32 x 25,600 blocks = 50 GiB) so the 256 MB
Infinity Cache cannot hold the working set.

``value`` = KV bytes the attention must read per step (sum of context
lengths x kv heads x head_dim x 2 tensors x 2 bytes) / wall time per step.

Prefill leg: ``kv_write`` of the 16 x 512-token chunk, then
``paged_attention_prefill`` over prefix + chunk (40 layers x 4,096 blocks
rotated); reported in TFLOP/s of the causal attention's algorithmic flops.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, AMD published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD published
# HBM bytes per dispatch from rocprofv3 counters (written by
# paged_kv_cache_364_amd.profiling from two --pmc runs of this script)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_decode_llama31_8b_b64_prefill_opt13b_b16x512.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_util_prefill_opt13b_b16x512.txt")
SHARED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_decode_llama_shared_prefix_32x4.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_description(np):
    """CPU model, usable cores and the numpy / BLAS builds the oracle ran on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = ""
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()}))
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "sched_affinity": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas": blas}


def settle(torch, fn, ms, batch):
    """Run fn(i) back to back, untimed, for at least `ms` milliseconds, so
    that what is timed next runs at the clocks a busy GPU holds; returns
    the number of calls."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < ms * 1e-3:
        for _ in range(batch):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def timed_calls(torch, fn, n, warmup, stream, per_call=True):
    """Average time per call (ms) of ``fn(i)``: one pair of events, recorded
    on the stream the kernels run on, around n calls back to back (an event
    recorded between two kernels adds a gap of its own, several microseconds
    here, to every call it brackets).  With ``per_call``, a second pass with
    an event pair around each call gives the per-call times, for their
    spread only."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # one untimed call first: the GPU is busy when it reaches e0, so the host's
    # launch latency of the first timed call does not land between the events
    fn(warmup)
    e0.record(stream)
    for i in range(n):
        fn(warmup + 1 + i)
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / n
    ts = []
    if per_call:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            evs[i][0].record(stream)
            fn(warmup + 1 + n + i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in evs]
    return avg, ts


def copy_bandwidth(torch, api, dev, mib=2048):
    """Bandwidth of a plain copy on this device: copy_blocks moving ``mib``
    MiB (read) + ``mib`` MiB (write) between disjoint halves of a pool, each
    call on fresh blocks so caches do not hold them.  GB/s of read+write."""
    Hkv, B, D = 8, 16, 128
    pair_bytes = 2 * Hkv * B * D * 2
    n = mib * 1024 * 1024 // pair_bytes
    rounds = 4
    k = torch.empty((2 * n * rounds, Hkv, B, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    k.view(torch.int16).fill_(1)
    v.view(torch.int16).fill_(1)
    pairs = []
    for r in range(rounds):
        base = 2 * n * r
        pairs.append(torch.stack([torch.arange(base, base + n), torch.arange(base + n, base + 2 * n)], 1)
                     .to(torch.int32).to(dev).contiguous())
    stream = torch.cuda.current_stream()
    avg, _ = timed_calls(torch, lambda i: api.copy_blocks(k, v, pairs[i % rounds]), rounds * 2, rounds, stream)
    del k, v
    torch.cuda.empty_cache()
    return 2 * n * pair_bytes / (avg * 1e-3) / 1e9


def prefill_leg(args, torch, np, api, driver, workloads, dev):
    wl = workloads.opt13b_prefill_b16x512()
    st = driver.run_script(wl, device=dev)
    torch.cuda.synchronize()
    S, Hq, Hkv, D, B = len(wl.batch), wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    ctx = st.context_lens.astype(np.int64)
    C = np.array(wl.q_lens, dtype=np.int64)
    P = ctx - C
    pairs = int((C * P + C * (C + 1) // 2).sum()) * Hq
    flops = 4 * D * pairs
    kv_bytes = int(ctx.sum()) * Hkv * D * 2 * 2
    qo_bytes = 2 * int(C.sum()) * Hq * D * 2
    L = max(1, args.prefill_layers)
    kps, vps = [st.k_pool], [st.v_pool]
    for _ in range(1, L):
        kps.append(st.k_pool.clone())
        vps.append(st.v_pool.clone())
    q = driver.to_device(wl.q, wl.dtype, dev)
    out = torch.empty_like(q)
    cu = torch.from_numpy(driver.cu_lens(wl.q_lens)).to(dev)
    chunk = wl.steps[-1]
    kn = driver.to_device(np.concatenate([op.k for op in chunk.ops]), wl.dtype, dev)
    vn = driver.to_device(np.concatenate([op.v for op in chunk.ops]), wl.dtype, dev)
    slots = torch.tensor(st.step_slots[-1], dtype=torch.int32, device=dev)
    scale = float(wl.scale)
    stream = torch.cuda.current_stream()

    def prefill(i):
        li = i % L
        api.paged_attention_prefill(out, q, cu, max(wl.q_lens), kps[li], vps[li], st.tables_dev, st.lens_dev, scale)

    def write(i):
        li = i % L
        api.kv_write(kn, vn, slots, kps[li], vps[li])

    # The clocks climb while the GPU is busy: 40 calls timed right after the
    # setup (and 40 warmup calls) run several percent slower than the same
    # calls after ~100 ms of back-to-back work.  Both are reported; the
    # roofline takes the settled figure.
    cold_ms, _ = timed_calls(torch, prefill, args.prefill_steps, max(args.warmup, 40), stream, per_call=False)
    n_settle = settle(torch, prefill, args.settle_ms, 8)
    pf_ms, pf_all = timed_calls(torch, prefill, args.prefill_steps, args.warmup, stream)
    kw_ms, _ = timed_calls(torch, write, args.prefill_steps, args.warmup, stream)
    tflops = flops / (pf_ms * 1e-3) / 1e12
    log(f"prefill {wl.name}: {pf_ms * 1e3:.1f} us avg, {tflops:.1f} TFLOP/s; kv_write of the chunk "
        f"{kw_ms * 1e3:.1f} us")
    kname = f"prefill_kernel<{D}>"  # the instantiation this shape runs
    traffic = None
    mfma = {"mfma_util_pct": None, "executed_gflop": None}
    try:
        from paged_kv_cache_364_amd import profiling

        tb = profiling.traffic_bytes(profiling.read_traffic(TRAFFIC_FILE), [kname])
        traffic = int(round(tb)) if tb is not None else None
        # matrix-core counters of the same kernel, if taken from these sources
        e = profiling.read_traffic(MFMA_FILE).get("kernels", {}).get(kname)
        if e is not None and e.get("sources_sha256") == profiling.sources_sha(e["group"]):
            mfma = {"mfma_util_pct": round(e["mfma_util_pct"], 2), "executed_gflop": round(e["bf16_flops"] / 1e9, 3)}
    except Exception:
        traffic = None
    res = {
        "workload": wl.name, "num_seqs": S, "chunk": int(C[0]), "prefix_lens": "uniform 0..1536 (seed 5)",
        "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": B, "layers_rotated": L,
        "prefill_us_avg": round(pf_ms * 1e3, 2),
        "prefill_us_avg_unsettled": round(cold_ms * 1e3, 2),
        "settle": {"ms": args.settle_ms, "calls": n_settle,
                   "note": "untimed calls between the unsettled and the settled measurement"},
        "prefill_us_per_call_events": {"median": round(float(np.median(pf_all)) * 1e3, 2),
                                       "p10": round(float(np.percentile(pf_all, 10)) * 1e3, 2),
                                       "p90": round(float(np.percentile(pf_all, 90)) * 1e3, 2)},
        "kv_write_chunk_us_avg": round(kw_ms * 1e3, 2),
        "tflops": round(tflops, 2), "algorithmic_gflop": round(flops / 1e9, 3),
        "min_hbm_bytes": kv_bytes + qo_bytes,
        "hbm_gbps_at_min_bytes": round((kv_bytes + qo_bytes) / (pf_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch"},
        "rocprof_mfma": mfma,
    }
    del kps, vps
    return res, (wl, st, out)


def swap_leg(torch, api, dev, n_blocks=4096):
    """Swap-out and swap-in of n whole Llama-shape blocks (64 KiB of K + V
    each) between a pool and pinned host memory, against a plain DMA copy of
    the same bytes to and from pinned memory."""
    Hkv, B, D = 8, 16, 128
    k = torch.empty((4 * n_blocks, Hkv, B, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    k.view(torch.int16).fill_(5)
    v.view(torch.int16).fill_(6)
    ids = torch.randperm(4 * n_blocks, device=dev)[:n_blocks].to(torch.int32).contiguous()
    hk = torch.empty((n_blocks, Hkv, B, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    stream = torch.cuda.current_stream()
    nbytes = 2 * hk.numel() * 2
    out_ms, _ = timed_calls(torch, lambda i: api.swap_out(k, v, ids, hk, hv), 5, 2, stream)
    in_ms, _ = timed_calls(torch, lambda i: api.swap_in(k, v, ids, hk, hv), 5, 2, stream)
    dk = torch.empty((n_blocks, Hkv, B, D), dtype=torch.bfloat16, device=dev)
    d2h_ms, _ = timed_calls(torch, lambda i: (hk.copy_(dk, non_blocking=True), hv.copy_(dk, non_blocking=True)),
                            5, 2, stream)
    h2d_ms, _ = timed_calls(torch, lambda i: (dk.copy_(hk, non_blocking=True), dk.copy_(hv, non_blocking=True)),
                            5, 2, stream)
    torch.cuda.synchronize()
    res = {"blocks": n_blocks, "bytes": nbytes,
           "swap_out_gbps": round(nbytes / (out_ms * 1e-3) / 1e9, 2),
           "swap_in_gbps": round(nbytes / (in_ms * 1e-3) / 1e9, 2),
           "dma_d2h_gbps": round(nbytes / (d2h_ms * 1e-3) / 1e9, 2),
           "dma_h2d_gbps": round(nbytes / (h2d_ms * 1e-3) / 1e9, 2)}
    log(f"swap: {res}")
    del k, v, dk
    torch.cuda.empty_cache()
    return res


def prefix_cache_leg(torch, np, api, driver, workloads, dev, steps, warmup):
    """32 requests sharing a 1,024-token system prompt (plus U{1..256}
    own tokens each), allocated with and without the prefix cache: blocks
    held, K/V rows written, and the decode time over each batch."""
    res = {}
    stream = torch.cuda.current_stream()
    for use in (True, False):
        wl = workloads.shared_prompt_requests(6, 32, 1024, 256, 25_600, use_cache=use)
        st = driver.run_script(wl, device=dev)
        q = driver.to_device(wl.q, wl.dtype, dev)
        out = torch.empty_like(q)
        ws = torch.zeros(api.decode_workspace_size(len(wl.batch), wl.num_heads, wl.num_kv_heads, wl.head_dim,
                                                   wl.block_size, wl.max_blocks_per_seq, q.dtype),
                         dtype=torch.uint8, device=dev)

        def decode(i):
            api.paged_attention_decode(out, q, st.k_pool, st.v_pool, st.tables_dev, st.lens_dev, float(wl.scale),
                                       workspace=ws)

        ms, _ = timed_calls(torch, decode, steps, warmup, stream)
        key = "with_cache" if use else "without_cache"
        res[key] = {"blocks_held": int(st.alloc.stats().num_used),
                    "kv_rows_written": int(sum(1 for x in st.step_slots[0] if x >= 0)),
                    "decode_us_avg": round(ms * 1e3, 2)}
        del st
        torch.cuda.empty_cache()
    res["workload"] = "32 requests x (1,024-token shared prompt + U{1..256}), Llama-3.1-8B shape, B=16 (seed 6)"
    log(f"prefix cache: {res}")
    return res


def window_leg(torch, np, api, driver, workloads, dev, steps, warmup, window=512):
    """The Llama-3.1-8B batch of 64 sequences with a sliding window of `window` tokens: blocks
    wholly before each window released (pkv_seq_trim), decode over the
    trimmed tables; GB/s over the K/V bytes the window holds."""
    wl = workloads.llama_decode_b64()
    st = driver.run_script(wl, device=dev)
    a = st.alloc
    used_before = a.stats().num_used
    freed = sum(a.trim(s, max(0, a.length(s) - window)) for s in wl.batch)
    tables, lens = a.block_tables(wl.batch, wl.max_blocks_per_seq)
    tables_dev, lens_dev = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    q = driver.to_device(wl.q, wl.dtype, dev)
    out = torch.empty_like(q)
    ws = torch.zeros(api.decode_workspace_size(len(wl.batch), wl.num_heads, wl.num_kv_heads, wl.head_dim,
                                               wl.block_size, wl.max_blocks_per_seq, q.dtype),
                     dtype=torch.uint8, device=dev)

    def decode(i):
        api.paged_attention_decode(out, q, st.k_pool, st.v_pool, tables_dev, lens_dev, float(wl.scale),
                                   workspace=ws, window=window)

    ms, _ = timed_calls(torch, decode, steps, warmup, stream=torch.cuda.current_stream())
    kv = int(np.minimum(lens.astype(np.int64), window).sum()) * wl.num_kv_heads * wl.head_dim * 2 * 2
    res = {"window": window, "blocks_released": int(freed), "blocks_held": int(a.stats().num_used),
           "blocks_held_full": int(used_before), "decode_us_avg": round(ms * 1e3, 2),
           "window_kv_gbps": round(kv / (ms * 1e-3) / 1e9, 1),
           "note": "one layer, not rotated: the window's K/V may sit in the Infinity Cache"}
    log(f"sliding window: {res}")
    del st
    torch.cuda.empty_cache()
    return res


def unique_kv_tokens(np, tables, lens, B):
    """Tokens held by distinct physical blocks: a block shared by several
    tables counts once, with the most positions any of them uses."""
    held = {}
    for t, n in zip(tables, lens):
        for lb in range((int(n) + B - 1) // B):
            b = int(t[lb])
            held[b] = max(held.get(b, 0), min(B, int(n) - lb * B))
    return sum(held.values())


def calibration_copy(torch, api, dev, mib, Hkv=8, B=16, D=128):
    """One copy_blocks launch of known size, for scaling HBM byte counters:
    n source blocks -> n destination blocks of 64 KiB (K + V), so n * 64 KiB
    are read and written."""
    n = max(1, mib * 1024 * 1024 // (2 * Hkv * B * D * 2))
    ck = torch.zeros((2 * n, Hkv, B, D), dtype=torch.bfloat16, device=dev)
    cv = torch.zeros_like(ck)
    pairs = torch.stack([torch.arange(n), torch.arange(n, 2 * n)], 1).to(torch.int32).to(dev).contiguous()
    torch.cuda.synchronize()
    api.copy_blocks(ck, cv, pairs)
    torch.cuda.synchronize()
    log(f"calibration copy: {n} block pairs, {2 * n * Hkv * B * D * 2} bytes read and written")
    del ck, cv


def other_batch_legs(torch, np, api, driver, workloads, dev, steps, warmup, layers=4, only=None):
    """Decode on the other Llama-3.1-8B-shape batches: 256 log-normal
    contexts over a churned free list, and 32 prompts forked into 4 branches
    that share their prompt blocks.  Each rotates `layers` copies of its
    pools so that the working set exceeds the Infinity Cache."""
    res = {}
    stream = torch.cuda.current_stream()
    for build, desc in ((workloads.llama_ragged_b256, "256 contexts, log-normal (median 500, sigma 1, clip 1..8192), "
                                            "churned free list (seed 3)"),
                        (workloads.llama_shared_prefix_32x4, "32 prompts x 1,024 tokens forked into 4 branches at U{1000..1023} minus 1008 (never on a block edge), "
                                            "U{0..256} private tokens each (seed 4)")):
        if only is not None and build.__name__ != only:
            continue
        wl = build()
        st = driver.run_script(wl, device=dev)
        torch.cuda.synchronize()
        S, Hq, Hkv, D, B = len(wl.batch), wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
        lens = st.context_lens.astype(np.int64)
        kv_bytes = int(lens.sum()) * Hkv * D * 2 * 2
        uniq_bytes = unique_kv_tokens(np, st.tables, lens, B) * Hkv * D * 2 * 2
        kps, vps = [st.k_pool], [st.v_pool]
        for _ in range(1, layers):
            kps.append(st.k_pool.clone())
            vps.append(st.v_pool.clone())
        q = driver.to_device(wl.q, wl.dtype, dev)
        out = torch.empty_like(q)
        ws = torch.zeros(api.decode_workspace_size(S, Hq, Hkv, D, B, wl.max_blocks_per_seq, q.dtype),
                         dtype=torch.uint8, device=dev)

        def decode(i):
            api.paged_attention_decode(out, q, kps[i % layers], vps[i % layers], st.tables_dev, st.lens_dev,
                                       float(wl.scale), workspace=ws)

        ms, all_ms = timed_calls(torch, decode, steps, warmup, stream)
        shared = None
        if build is workloads.llama_shared_prefix_32x4:
            # the same batch through the shared-prefix decode: each prompt's
            # shared blocks read once for its branches
            gs, sb = st.alloc.shared_prefix_groups(wl.batch, api.decode_shared_max_members(Hq, Hkv))
            gsd, sbd = torch.from_numpy(gs).to(dev), torch.from_numpy(sb).to(dev)

            def decode_shared(i):
                api.paged_attention_decode_shared(out, q, kps[i % layers], vps[i % layers], st.tables_dev,
                                                  st.lens_dev, gsd, sbd, float(wl.scale))

            sms, _ = timed_calls(torch, decode_shared, steps, warmup, stream, per_call=False)
            shared = {"call": "paged_attention_decode_shared", "groups": int(len(sb)),
                      "shared_blocks_per_group": [int(sb.min()), int(sb.max())],
                      "decode_us_avg": round(sms * 1e3, 2),
                      "kv_gbps_unique": round(uniq_bytes / (sms * 1e-3) / 1e9, 1),
                      "pct_hbm_peak_unique": round(100 * uniq_bytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                      "seqs_per_s_per_layer": round(S / (sms * 1e-3), 1)}
            from paged_kv_cache_364_amd import profiling
            tb = profiling.traffic_bytes(profiling.read_traffic(SHARED_TRAFFIC_FILE), ["decode_shared_kernel<128>"])
            shared["traffic"] = int(round(tb)) if tb is not None else None
            shared["traffic_over_unique"] = round(tb / uniq_bytes, 4) if tb is not None else None
        r = {"workload": wl.name, "batch": desc, "num_seqs": S, "sum_context": int(lens.sum()),
             "layers_rotated": layers, "decode_us_avg": round(ms * 1e3, 2),
             "decode_us_per_call_events_median": round(float(np.median(all_ms)) * 1e3, 2),
             "kv_bytes_logical": kv_bytes, "kv_gbps_logical": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
             "kv_bytes_unique": uniq_bytes, "kv_gbps_unique": round(uniq_bytes / (ms * 1e-3) / 1e9, 1),
             "pct_hbm_peak_unique": round(100 * uniq_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
             "seqs_per_s_per_layer": round(S / (ms * 1e-3), 1)}
        if shared is not None:
            r["plain_call"] = "paged_attention_decode (every branch streams its prefix)"
            r["shared_prefix_decode"] = shared
        log(f"{wl.name}: {r}")
        res[wl.name] = r
        del st, kps, vps, q, out, ws
        torch.cuda.empty_cache()
    return res


def gather_ceiling_leg(torch, np, api, kps, vps, tables, lens, B, steps, warmup):
    """Bandwidth ceiling of the paged access pattern on this device: the
    same pools, rotated the same way, read by a kernel that only loads
    (pkv_gather_units).  Three unit lists:
      - decode_units: the (block, kv head) slices the decode reads, K and V,
        from the batch's own tables (4 KiB each at the Llama shape);
      - random_4k: as many random 4 KiB (block, kv head) slices;
      - random_32k: random whole blocks (all kv heads, 32 KiB per tensor),
        the same bytes in 8x longer contiguous runs.
    GB/s counts the bytes the units hold."""
    Nb, Hkv, Bb, D = kps[0].shape
    slice_kib = Bb * D * kps[0].element_size() // 1024
    blk_kib = Hkv * slice_kib
    rng = np.random.default_rng(12)
    units = []
    for t, n in zip(tables, lens):
        for lb in range((int(n) + B - 1) // B):
            b = int(t[lb])
            units.extend(b * Hkv + h for h in range(Hkv))
    n4 = len(units)
    lists = {
        "decode_units": (np.array(units, dtype=np.int32), slice_kib),
        "random_4k": (rng.choice(Nb * Hkv, size=n4, replace=False).astype(np.int32), slice_kib),
        "random_32k": (rng.choice(Nb, size=max(1, n4 // Hkv), replace=False).astype(np.int32), blk_kib),
    }
    sink = torch.zeros(8192, dtype=torch.int32, device=kps[0].device)
    stream = torch.cuda.current_stream()
    L = len(kps)
    res = {}
    for name, (ids, kib) in lists.items():
        idt = torch.from_numpy(ids).to(kps[0].device)
        nbytes = 2 * len(ids) * kib * 1024

        def read(i):
            api.gather_units(kps[i % L], vps[i % L], idt, kib, sink)

        ms, _ = timed_calls(torch, read, steps, warmup, stream, per_call=False)
        res[name] = {"unit_kib": kib, "units_per_pool": int(len(ids)), "bytes": nbytes,
                     "us_avg": round(ms * 1e3, 2), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)}
        log(f"gather {name}: {res[name]}")
    res["note"] = ("read-only kernel over the decode's own pools, layers rotated as for the decode; K and V "
                   "units both read")
    return res


def block_sweep(args, torch, np, api, driver, workloads, dev):
    """Decode at the Llama-3.1-8B shape for several block sizes with the same
    lengths and values (seed 2) and the same pool capacity (409,600 tokens
    per layer): kernel time, KV GB/s and the share of allocated slots that
    hold tokens (the tail waste of the last block)."""
    rows = []
    stream = torch.cuda.current_stream()
    for B in args.block_sweep:
        wl = workloads.llama_decode(2, 64, 128, 2048, 409_600 // B, f"llama31-8b-decode-b64-B{B}", block_size=B)
        st = driver.run_script(wl, device=dev)
        torch.cuda.synchronize()
        S, Hq, Hkv, D = len(wl.batch), wl.num_heads, wl.num_kv_heads, wl.head_dim
        ctx = st.context_lens.astype(np.int64)
        kv_bytes = int(ctx.sum()) * Hkv * D * 2 * 2
        L = max(1, args.layers)
        kps, vps = [st.k_pool], [st.v_pool]
        for _ in range(1, L):
            kps.append(st.k_pool.clone())
            vps.append(st.v_pool.clone())
        q = driver.to_device(wl.q, wl.dtype, dev)
        out = torch.empty_like(q)
        ws = torch.zeros(api.decode_workspace_size(S, Hq, Hkv, D, B, wl.max_blocks_per_seq, q.dtype),
                         dtype=torch.uint8, device=dev)

        def decode(i):
            api.paged_attention_decode(out, q, kps[i % L], vps[i % L], st.tables_dev, st.lens_dev,
                                       float(wl.scale), workspace=ws)

        ms, _ = timed_calls(torch, decode, args.steps, args.warmup, stream)
        slots = int(((ctx + B - 1) // B * B).sum())
        rows.append({"block_size": B, "decode_us_avg": round(ms * 1e3, 2),
                     "kv_gbps": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
                     "useful_slot_ratio": round(int(ctx.sum()) / slots, 5),
                     "waste_slots_per_seq": round((slots - int(ctx.sum())) / S, 2),
                     "table_entries_per_seq": wl.max_blocks_per_seq})
        log(f"block size {B}: {rows[-1]}")
        del kps, vps, st
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="run the step (and the prefill) untimed this long before their warmup")
    ap.add_argument("--prefill-steps", type=int, default=40)
    ap.add_argument("--prefill-layers", type=int, default=40)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-copy-bandwidth", action="store_true")
    ap.add_argument("--no-swap", action="store_true")
    ap.add_argument("--no-prefix-cache", action="store_true")
    ap.add_argument("--no-window", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the ragged and shared-prefix decode batches")
    ap.add_argument("--no-gather-ceiling", action="store_true")
    ap.add_argument("--no-block-sweep", action="store_true")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-sweep", type=int, nargs="*", default=None,
                    help="instead of the benchmark, time decode at the Llama shape for these block sizes")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before timing, copy this many MiB once with copy_blocks (a plain copy of known size, "
                         "for scaling HBM byte counters)")
    ap.add_argument("--other-batch", choices=["llama_ragged_b256", "llama_shared_prefix_32x4"], default=None,
                    help="instead of the benchmark, time the decode of this batch only (to profile it)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "pagedkv runs on one GPU only; --gpus must be 1 (the kernels have no "
                                   "multi-GPU path)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_364_amd import api, driver, profiling, workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.other_batch is not None:
        if args.calibrate_copy_mib > 0:
            calibration_copy(torch, api, dev, args.calibrate_copy_mib)
        rows = other_batch_legs(torch, np, api, driver, workloads, dev, args.steps, args.warmup,
                                only=args.other_batch)
        print(json.dumps(rows), flush=True)
        return
    if args.block_sweep is not None:
        sizes = args.block_sweep or [8, 16, 32, 64, 128, 256]
        args.block_sweep = sizes
        rows = block_sweep(args, torch, np, api, driver, workloads, dev)
        print(json.dumps({"block_sweep": rows, "workload": "llama31-8b-decode-b64 (seed 2), 409,600-token pool per "
                          f"layer, {max(1, args.layers)} layers rotated", "steps": args.steps}), flush=True)
        return
    t0 = time.time()
    wl = workloads.llama_decode_b64()
    log(f"workload {wl.name} generated in {time.time() - t0:.1f}s")
    st = driver.run_script(wl, device=dev)
    torch.cuda.synchronize()
    S, Hq, Hkv, D, B = len(wl.batch), wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    sum_ctx = int(st.context_lens.sum())
    kv_bytes = sum_ctx * Hkv * D * 2 * 2
    qo_bytes = 2 * S * Hq * D * 2
    log(f"S={S} sum_ctx={sum_ctx} KV bytes/step={kv_bytes / 1e6:.1f} MB")

    # per-layer pools (layer 0 = the oracle-checked data; the others copies)
    L = max(1, args.layers)
    kps, vps = [st.k_pool], [st.v_pool]
    for _ in range(1, L):
        kps.append(st.k_pool.clone())
        vps.append(st.v_pool.clone())
    torch.cuda.synchronize()
    q = driver.to_device(wl.q, wl.dtype, dev)
    out = torch.empty_like(q)
    dec = wl.steps[-1]  # the decode token of every sequence
    kn = driver.to_device(np.concatenate([op.k for op in dec.ops]), wl.dtype, dev)
    vn = driver.to_device(np.concatenate([op.v for op in dec.ops]), wl.dtype, dev)
    slots = torch.tensor(st.step_slots[-1], dtype=torch.int32, device=dev)
    ws = torch.zeros(api.decode_workspace_size(S, Hq, Hkv, D, B, wl.max_blocks_per_seq, q.dtype),
                     dtype=torch.uint8, device=dev)
    scale = float(wl.scale)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy_mib > 0:
        calibration_copy(torch, api, dev, args.calibrate_copy_mib)

    def append_decode(i):
        li = i % L
        api.paged_attention_decode_append(out, q, kn, vn, kps[li], vps[li], st.tables_dev, st.lens_dev, scale,
                                          workspace=ws)

    def decode(i):
        li = i % L
        api.paged_attention_decode(out, q, kps[li], vps[li], st.tables_dev, st.lens_dev, scale, workspace=ws)

    def write(i):
        li = i % L
        api.kv_write(kn, vn, slots, kps[li], vps[li])

    def two_calls(i):
        write(i)
        decode(i)

    # the step: each sequence's new token written through its block table and
    # the decode over the whole context, in one call (bitwise the same as
    # kv_write then paged_attention_decode)
    step = append_decode

    # Settle: the step runs back to back, untimed, for --settle-ms before
    # the warmup steps.  The first milliseconds of back-to-back work after the
    # setup run 1.5-3 us per step slower than the rest (the clocks climb while
    # the GPU is busy), which a short timed region would otherwise measure.
    n_settle = settle(torch, step, args.settle_ms, 50)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    # timed region: K whole steps back to back, wall clock between two
    # synchronisations, nothing else enqueued inside it
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_per_step = t_total * 1e3 / K
    # the same step as two calls, timed the same way
    for i in range(args.warmup):
        two_calls(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        two_calls(args.warmup + i)
    torch.cuda.synchronize()
    ms_two = (time.perf_counter() - t_start) * 1e3 / K
    # per-call durations: K calls back to back between one pair of events on
    # the kernels' stream (the step's call, then the plain decode, then
    # kv_write)
    dec_avg, dec_ms = timed_calls(torch, append_decode, K, 5, stream)
    dec_ms = np.array(dec_ms)
    plain_avg, _ = timed_calls(torch, decode, K, 5, stream, per_call=False)
    kvw_avg, _ = timed_calls(torch, write, K, 5, stream, per_call=False)
    log(f"append+decode avg {dec_avg * 1e3:.1f} us (per-call events: median {np.median(dec_ms) * 1e3:.1f}, "
        f"p10 {np.percentile(dec_ms, 10) * 1e3:.1f}, p90 {np.percentile(dec_ms, 90) * 1e3:.1f}); "
        f"plain decode avg {plain_avg * 1e3:.1f} us; kv_write avg {kvw_avg * 1e3:.1f} us; "
        f"wall {ms_per_step * 1e3:.1f} us/step ({ms_two * 1e3:.1f} as two calls)")

    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    new_bytes = 2 * S * Hkv * D * 2 * 2  # the new rows read and stored, K and V
    achieved = (kv_bytes + qo_bytes + new_bytes) / (dec_avg * 1e-3) / 1e9
    plain_achieved = (kv_bytes + qo_bytes) / (plain_avg * 1e-3) / 1e9
    tb = profiling.traffic_bytes(profiling.read_traffic(TRAFFIC_FILE),
                                 ["decode_main<bf16_t, 128, 4, true>", "decode_merge<bf16_t, 128, 4>"])

    result = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + seqs/s/layer, Llama-3.1-8B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "settle": {"ms": args.settle_ms, "steps": n_settle,
                   "note": "untimed steps before the warmup, so that the timed region starts at steady state"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": S, "context_lens": "uniform 128..2048 (seed 2)",
                   "sum_context": sum_ctx, "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": B, "pool_blocks_per_layer": wl.num_blocks, "layers_rotated": L,
                   "step": "kv_write + paged_attention_decode, one layer, as one call "
                           "(paged_attention_decode_append)", "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "useful_kv_ratio": round(sum_ctx / float(((st.context_lens.astype(np.int64) + B - 1) // B * B).sum()), 5),
        "seqs_per_s_per_layer": round(S / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "decode_us_avg": round(dec_avg * 1e3, 2),
        "two_call_step": {"calls": "kv_write, then paged_attention_decode", "ms_per_step": round(ms_two, 5),
                          "value": round(kv_bytes / (ms_two * 1e-3) / 1e9, 2)},
        "plain_decode": {"call": "paged_attention_decode (decode_main + decode_merge)",
                         "us_avg": round(plain_avg * 1e3, 2), "achieved": round(plain_achieved, 2),
                         "frac": round(plain_achieved / HBM_PEAK_GBPS, 4)},
        "decode_us_per_call_events": {"median": round(float(np.median(dec_ms)) * 1e3, 2),
                                      "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                                      "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
                                      "note": "an event pair around each call; each event adds its own gap"},
        "kv_write_us_avg": round(kvw_avg * 1e3, 2),
        "kv_write_us_in_two_call_step": round((ms_two - plain_avg) * 1e3, 2),
        "kv_write_note": "alone, back to back, the 64-token write is bound by the host's launch rate; "
                         "kv_write_us_in_two_call_step = two-call wall per step - plain decode average",
        "roofline": {"bound": "hbm", "kernel": "paged_attention_decode_append = decode_main (append variant) + "
                                               "decode_merge",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": int(round(tb)) if tb is not None else None, "traffic_unit": "bytes per launch"},
    }
    if not args.no_gather_ceiling:
        gc = gather_ceiling_leg(torch, np, api, kps, vps, st.tables, st.context_lens, B, 100, 10)
        result["gather_ceiling"] = gc
        result["roofline"]["frac_of_gather_ceiling"] = round(achieved / gc["decode_units"]["gbps"], 4)
    got_decode = driver.out_to_f64(out)
    del kps, vps
    torch.cuda.empty_cache()

    if not args.no_copy_bandwidth:
        cbw = copy_bandwidth(torch, api, dev)
        result["copy_kernel_gbps"] = round(cbw, 1)
        result["roofline"]["frac_of_copy_kernel"] = round(achieved / cbw, 4)
        log(f"copy_blocks bandwidth (read + write) {cbw:.0f} GB/s")

    if not args.no_swap:
        result["swap"] = swap_leg(torch, api, dev)
    if not args.no_window:
        result["sliding_window"] = window_leg(torch, np, api, driver, workloads, dev, 50, 5)
    if not args.no_prefix_cache:
        result["prefix_cache"] = prefix_cache_leg(torch, np, api, driver, workloads, dev, 50, 5)
    if not args.no_configs:
        result["other_batches"] = other_batch_legs(torch, np, api, driver, workloads, dev, 50, 5)

    if not args.no_block_sweep:
        class SweepArgs:
            block_sweep = [8, 16, 32, 64, 128, 256]
            layers = 8
            steps = 50
            warmup = 5
        rows = block_sweep(SweepArgs, torch, np, api, driver, workloads, dev)
        result["block_sweep"] = {"rows": rows, "workload": "llama31-8b-decode-b64 lengths and values (seed 2), "
                                 "409,600-token pool per layer, 8 layers rotated, decode only",
                                 "steps": SweepArgs.steps}

    pf = None
    if not args.no_prefill:
        pf, pf_state = prefill_leg(args, torch, np, api, driver, workloads, dev)
        result["prefill"] = pf

    if not args.no_cpu_baseline:
        from oracle import runner as oracle_runner

        ost = oracle_runner.run(wl)
        runs, t_cpu = 0, 0.0
        exp = None
        while runs == 0 or t_cpu < args.cpu_baseline_seconds:
            t1 = time.perf_counter()
            exp = oracle_runner.expected(wl, ost)
            t_cpu += time.perf_counter() - t1
            runs += 1
        err = float(np.abs(got_decode - exp).max())
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            cores = 1
        result["cpu_baseline"] = {
            "value": round(kv_bytes * runs / t_cpu / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"the full {wl.name} batch (layer 0, {sum_ctx} context tokens) {runs} times in "
                      f"{t_cpu:.1f}s; numpy float64 on {platform.machine()}, os.cpu_count={os.cpu_count()}, "
                      f"BLAS threads={cores}",
            "seqs_per_s_per_layer": round(S * runs / t_cpu, 1),
            "host": host_description(np)}
        result["parity_max_abs_err_vs_oracle"] = err
        log(f"oracle {t_cpu / runs:.2f}s per batch, decode parity max abs err {err:.3g}")
        if pf is not None:
            pwl, pst, pout = pf_state
            post = oracle_runner.run(pwl)
            t1 = time.perf_counter()
            pexp = oracle_runner.expected(pwl, post)
            pf["cpu_oracle_s"] = round(time.perf_counter() - t1, 3)
            pf["cpu_oracle_tflops"] = round(pf["algorithmic_gflop"] / pf["cpu_oracle_s"] / 1e3, 5)
            pf["parity_max_abs_err_vs_oracle"] = float(np.abs(driver.out_to_f64(pout) - pexp).max())
            log(f"prefill parity max abs err {pf['parity_max_abs_err_vs_oracle']:.3g}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

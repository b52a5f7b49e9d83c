"""Paged decode attention benchmark (Llama-3.1-8B attention shape).

One step = the device work of one decode step for one layer of the batch:
``kv_write`` of the batch's new tokens into their slots, then
``paged_attention_decode`` (main pass + log-sum-exp merge) over the paged
cache.  Layers rotate over separate per-layer pools (32 x 25,600 blocks,
50 GiB in all) so the 256 MB Infinity Cache cannot hold the working set.

Prints one JSON line.  ``value`` is KV bytes the attention must read per
step (sum of context lengths x kv heads x head_dim x 2 tensors x 2 bytes)
divided by the measured time per step.
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before timing, copy this many MiB once with copy_blocks (a plain copy of known size, "
                         "for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_364_amd import api, driver, workloads

    dev = "cuda:0"
    torch.cuda.set_device(0)
    t0 = time.time()
    wl = workloads.config2()
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
    ws = torch.empty(api.decode_workspace_size(S, Hq, Hkv, D, B, wl.max_blocks_per_seq, q.dtype),
                     dtype=torch.uint8, device=dev)
    scale = float(wl.scale)

    def step(i, ev=None):
        li = i % L
        if ev is not None:
            ev[0].record()
        api.kv_write(kn, vn, slots, kps[li], vps[li])
        if ev is not None:
            ev[1].record()
        api.paged_attention_decode(out, q, kps[li], vps[li], st.tables_dev, st.lens_dev, scale, workspace=ws)
        if ev is not None:
            ev[2].record()

    if args.calibrate_copy_mib > 0:
        # n source blocks -> n destination blocks of 64 KiB (K + V): n * 64 KiB read and written
        n = max(1, args.calibrate_copy_mib * 1024 * 1024 // (2 * Hkv * B * D * 2))
        ck = torch.zeros((2 * n, Hkv, B, D), dtype=q.dtype, device=dev)
        cv = torch.zeros_like(ck)
        pairs = torch.stack([torch.arange(n), torch.arange(n, 2 * n)], 1).to(torch.int32).to(dev).contiguous()
        torch.cuda.synchronize()
        api.copy_blocks(ck, cv, pairs)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} block pairs, {2 * n * Hkv * B * D * 2} bytes read and written")
        del ck, cv

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    kvw_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    ms_per_step = t_total * 1e3 / K
    dec_avg = float(dec_ms.mean())
    log(f"decode avg {dec_avg * 1e3:.1f} us (p10 {np.percentile(dec_ms, 10) * 1e3:.1f}, "
        f"p90 {np.percentile(dec_ms, 90) * 1e3:.1f}); kv_write avg {kvw_ms.mean() * 1e3:.1f} us; "
        f"wall {ms_per_step * 1e3:.1f} us/step")

    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = (kv_bytes + qo_bytes) / (dec_avg * 1e-3) / 1e9

    # parity of the last output (layer data are identical copies of layer 0)
    result = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + seqs/s/layer, Llama-3.1-8B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": S, "context_lens": "uniform 128..2048 (seed 2)",
                   "sum_context": sum_ctx, "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": B, "pool_blocks_per_layer": wl.num_blocks, "layers_rotated": L,
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "seqs_per_s_per_layer": round(S / (ms_per_step * 1e-3), 1),
        "decode_us_avg": round(dec_avg * 1e3, 2),
        "decode_us_p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
        "decode_us_p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2),
        "kv_write_us_avg": round(float(kvw_ms.mean()) * 1e3, 2),
        "roofline": {"bound": "hbm", "kernel": "paged_attention_decode (decode_main + decode_merge)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None},
    }

    if not args.no_cpu_baseline:
        from oracle import runner as oracle_runner

        ost = oracle_runner.run(wl)
        got = driver.out_to_f64(out)
        runs, t_cpu = 0, 0.0
        exp = None
        while runs == 0 or t_cpu < args.cpu_baseline_seconds:
            t1 = time.perf_counter()
            exp = oracle_runner.expected(wl, ost)
            t_cpu += time.perf_counter() - t1
            runs += 1
        err = float(np.abs(got - exp).max())
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            cores = 1
        result["cpu_baseline"] = {
            "value": round(kv_bytes * runs / t_cpu / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"full {wl.name} batch (layer 0), {runs} runs, {t_cpu:.1f}s; numpy fp64 on "
                      f"{platform.processor() or platform.machine()}, os.cpu_count={os.cpu_count()}"}
        result["parity_max_abs_err_vs_oracle"] = err
        log(f"oracle {t_cpu / runs:.2f}s per batch, parity max abs err {err:.3g}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

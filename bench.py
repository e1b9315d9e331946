"""Benchmark of the paged KV-cache hot path on one MI355X.

One step = the whole path over one Llama-8B-shaped decode batch: kv_append of one new
token per request (64 tokens, bf16, 8 kv heads of 128) into a paged pool (block size 16),
then paged_decode of one query token per request (32 q heads, GQA 4) over the updated
context (513..4097 tokens, U{512..4096} cached + 1), split-K partitions merged by
log-sum-exp.  Inputs are synthetic, seeded, already resident in HBM.

Four per-layer pools (same shapes and block tables, different data) are used in rotation,
one per step, as in a multi-layer decode: between two reads of a pool ~1.8 GB of other
KV data is read, so the 256 MB Infinity Cache cannot hold it and the timed reads come
from HBM.

Prints ONE JSON line.  value = algorithmic bytes of the step / step time (GB/s).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
N_LAYERS = 4


def algorithmic_bytes(wl):
    """Bytes the method must move, per step (the design doc states the same formulas)."""
    H, D, B, Hq = wl.num_kv_heads, wl.head_dim, wl.batch, wl.num_q_heads
    esz = 2
    ctx = wl.ctx_after.long()
    kv = int(ctx.sum()) * H * D * esz * 2                  # K and V rows of every live token
    qo = 2 * B * Hq * D * esz                              # q read + out written
    bt = int(((ctx + wl.block_size - 1) // wl.block_size).sum()) * 4 + B * 4
    decode = kv + qo + bt
    append = B * H * D * esz * 2 * 2 + B * 8              # read new K,V + write rows + slots
    return decode, append, kv


def cpu_baseline(wl, hk_bits, hv_bits, budget_s=12.0, max_reps=5):
    """The oracle as it stands, on host cores, over the same workload (append + decode)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    nk = wl.new_k.detach().contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    nv = wl.new_v.detach().contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    q = wl.q.float().cpu().numpy()
    slots = wl.slot_mapping.numpy()
    reps, t_total = 0, 0.0
    while reps < max_reps and t_total < budget_s:
        k, v = hk_bits.copy(), hv_bits.copy()
        t0 = time.perf_counter()
        oracle.append_ref(nk, nv, slots, k, v, oracle.CacheSpec("same", "bf16"), wl.block_size)
        oracle.paged_decode_ref(q, oracle.PoolView("same", k, dtype="bf16"),
                                oracle.PoolView("same", v, dtype="bf16"), wl.block_tables.numpy(),
                                wl.ctx_after.numpy(), wl.block_size, wl.num_kv_heads, wl.sm_scale)
        t_total += time.perf_counter() - t0
        reps += 1
    dec, app, _ = algorithmic_bytes(wl)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": (dec + app) * reps / t_total / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the full workload (64 requests: append + decode, float64 numpy), "
                      f"{reps} rep(s), {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no "
              "multi-GPU component to measure.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import paged_kv_cache_45_amd as P
    from paged_kv_cache_45_amd import workloads as W

    torch.cuda.set_device(0)
    P.load_library()
    layers = []
    for i in range(N_LAYERS):
        wl = W.llama8b_decode("cuda", data_seed=W.BASE_SEED + 2 + 1000 * i, poison=(i == 0))
        layers.append(wl)
    wl0 = layers[0]
    host_k = wl0.k_pool.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
    host_v = wl0.v_pool.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
    B, Hq, D = wl0.batch, wl0.num_q_heads, wl0.head_dim
    maxctx = max(w.max_context_len for w in layers)
    dev = [dict(bt=w.block_tables.cuda(), ctx=w.ctx_after.cuda(), slots=w.slot_mapping.cuda(),
                out=torch.empty_like(w.q),
                ws=P.decode_workspace(B, Hq, wl0.num_kv_heads, D, maxctx, args.partition_size))
           for w in layers]
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        w, d = layers[i % N_LAYERS], dev[i % N_LAYERS]
        if ev is not None:
            ev[0].record(stream)
        P.kv_append(w.new_k, w.new_v, d["slots"], w.k_pool, w.v_pool)
        if ev is not None:
            ev[1].record(stream)
        P.paged_decode(w.q, w.k_pool, w.v_pool, d["bt"], d["ctx"], w.max_context_len, w.sm_scale,
                       partition_size=args.partition_size, workspace=d["ws"], out=d["out"])
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # per-kernel durations with events on the launch stream (a separate pass of K steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    app_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    for d in dev:
        assert torch.isfinite(d["out"].float()).all(), "non-finite decode output"

    dec_b, app_b, kv_b = algorithmic_bytes(wl0)
    dec_bytes_all = np.mean([algorithmic_bytes(w)[0] for w in layers])
    value = (dec_bytes_all + app_b) / (ms_per_step * 1e-3) / 1e9
    dec_avg_s = dec_ms.mean() * 1e-3
    achieved = dec_bytes_all / dec_avg_s / 1e9
    traffic = None
    rec = {
        "metric": "paged decode KV GB/s (% of HBM peak) + append tokens/s, Llama-8B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama8b-decode-step", "batch": B, "num_q_heads": Hq,
                   "num_kv_heads": wl0.num_kv_heads, "head_dim": D, "block_size": wl0.block_size,
                   "context": "U{512..4096} cached + 1 appended", "layers_rotated": N_LAYERS,
                   "partition_size": args.partition_size or "auto"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_us_median": round(float(np.median(dec_ms)) * 1e3, 2),
        "decode_us_p20_p80": [round(float(np.quantile(dec_ms, 0.2)) * 1e3, 2),
                              round(float(np.quantile(dec_ms, 0.8)) * 1e3, 2)],
        "append_us_median": round(float(np.median(app_ms)) * 1e3, 2),
        "append_tokens_per_s": round(B / (float(np.median(app_ms)) * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "paged_decode (decode_kernel + merge_kernel)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl0, host_k, host_v)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

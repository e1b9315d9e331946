"""Benchmark of the paged KV-cache hot path on one MI355X.

Default workload (the headline): one step = the whole path over one Llama-8B-shaped decode
batch: the append of one new token per request (64 tokens, bf16, 8 kv heads of 128) into a
paged pool (block size 16), then the decode of one query token per request (32 q heads,
GQA 4) over the updated context (513..4097 tokens, U{512..4096} cached + 1), split-K
ranges merged by log-sum-exp.  The step is one paged_decode_append launch (the decode's
workgroups write the new tokens), or with --separate-append kv_append then paged_decode.
Inputs are synthetic, seeded, already resident in HBM.

Four per-layer pools (same shapes and block tables, different data) are used in rotation,
one per step, as in a multi-layer decode: between two reads of a pool ~1.8 GB of other
KV data is read, so the 256 MB Infinity Cache cannot hold it and the timed reads come
from HBM.

Prints ONE JSON line.  value = algorithmic bytes of the step / step time (GB/s).

Other workloads (--workload), each one JSON line of the same form, for the measurements
of the remaining shapes:
  mixed-append-fp8   8 prompts U{128..2048} + 56 decode tokens, 10% padding slots, bf16 ->
                     fp8 e4m3fn cache with per-row scales, block size 32 (tokens/s)
  long-context       B=8, 64/8 heads, block size 64, contexts U{32k..128k}, partitions of
                     512 tokens (KV GB/s)
  packed3-decode     B=32, 32/8 heads, 3-bit cache with fp16 (scale, zero), block size 16,
                     contexts U{1k..16k}, fp16 query (KV GB/s)
  pack3-exhaustive   pack3 + unpack3 over all 2^24 octets, with the bijection check
  fp8-decode         the Llama-8B decode shape over fp8 e4m3fn pools with per-row fp32 scales
  e5m2-decode        the same over fp8 e5m2 pools
  int8-decode        the same over int8 pools
  fp8-tensor-scale-decode  the fp8 e4m3fn pools with one caller-given scale per pool
  contiguous-decode  the Llama-8B decode shape over a contiguous [B, Hkv, 4096, D] cache
                     (KV GB/s; the pools hold half the bytes of the bf16 ones)
  dual-stacked-decode  the Llama-8B decode shape over the dual-stacked block layout
                     [num_blocks, 2, num_kv_heads, block_size, head_dim], as strided views (KV GB/s)
  copy-calibration   a plain device copy of 1 GiB, the reference for HBM byte counters
  add-calibration    torch's elementwise add with the mixed fp8 append's traffic (64.26 MB,
                     two bytes read per byte written): what a plain streaming kernel reaches
                     at that size

--pad-frac sets the mixed append's share of padding slots (default 0.10), for the check
that the bytes it fetches follow the valid tokens.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
N_LAYERS = 4
METRIC = "paged decode KV GB/s (% of HBM peak) + append tokens/s, Llama-8B shape"
DECODE_SOURCES = ("paged_kv_cache_45_amd/csrc/decode.hip", "paged_kv_cache_45_amd/csrc/decode_kernel.cuh",
                  "paged_kv_cache_45_amd/csrc/append_rows.cuh",
                  "paged_kv_cache_45_amd/csrc/decode_same_d128.hip", "paged_kv_cache_45_amd/csrc/common.cuh",
                  "paged_kv_cache_45_amd/csrc/launch.h", "paged_kv_cache_45_amd/csrc/api.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama8b_hbm_traffic.md")


# ----------------------------------------------------------------------------------------
# algorithmic bytes (the bytes the method must move; the same formulas are stated with the
# kernels' roofline figures in the design notes)
# ----------------------------------------------------------------------------------------
def decode_bytes(wl, kv_bytes_per_token_head):
    """K/V of every live token + q read + out written + the block-table entries used."""
    H, D, B, Hq = wl.num_kv_heads, wl.head_dim, wl.batch, wl.num_q_heads
    ctx = wl.ctx_after.long()
    kv = int(ctx.sum()) * H * kv_bytes_per_token_head
    qo = 2 * B * Hq * D * 2
    bt = int(((ctx + wl.block_size - 1) // wl.block_size).sum()) * 4 + B * 4
    return kv + qo + bt, kv


def algorithmic_bytes(wl):
    """Llama-8B step: (decode bytes, append bytes, KV bytes)."""
    H, D, B = wl.num_kv_heads, wl.head_dim, wl.batch
    dec, kv = decode_bytes(wl, 2 * D * 2)
    append = B * H * D * 2 * 2 * 2 + B * 8                # read new K,V + write rows + slots
    return dec, append, kv


def sources_sha256():
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(entry_point):
    """HBM bytes per launch of `entry_point` from the committed counter summary, or None when
    there is none or the decode sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    for m in re.finditer(r"^traffic-record: (\{.*\})$", text, re.M):
        rec = json.loads(m.group(1))
        if rec.get("entry_point") == entry_point and rec.get("sources_sha256") == sources_sha256():
            return int(rec["hbm_bytes_per_launch"])
    return None


# per-call statistics (the roofline figure among them) take the median of at least this many
# event-timed calls, whatever --steps is, so that one slow call does not move them
N_EVENT_CALLS = 100


def event_times_ms(fn, n, stream):
    """Durations of n calls of fn(i), each bracketed by events on `stream`."""
    import numpy as np
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def graph_call_times_ms(calls, reps):
    """Per-call durations of a short, launch-bound entry point: the calls are captured into
    one HIP graph (they allocate nothing and record no memset) and the graph is replayed
    `reps` times, each replay bracketed by events; returns replay time / len(calls)."""
    import numpy as np
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):               # warm-up outside the capture
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    ms = event_times_ms(lambda _: g.replay(), reps, stream)
    return ms / len(calls), g


def call_times_ms(fn, args, stream):
    """Durations of max(N_EVENT_CALLS, --steps) calls of fn(i), each bracketed by events."""
    return event_times_ms(fn, max(N_EVENT_CALLS, args.steps), stream)


def stats_us(ms):
    import numpy as np
    return {"median": round(float(np.median(ms)) * 1e3, 2),
            "p20_p80": [round(float(np.quantile(ms, 0.2)) * 1e3, 2),
                        round(float(np.quantile(ms, 0.8)) * 1e3, 2)],
            "mean": round(float(ms.mean()) * 1e3, 2), "calls": int(len(ms))}


def base_record(args, metric, value, unit, ms_per_step, dtype, config, higher=True):
    return {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": higher, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": config}


def hbm_roofline(kernel, alg_bytes, ms, traffic=None, timing="event-timed calls"):
    """Roofline record of one entry point from its timed calls `ms` (milliseconds): the
    achieved rate is the algorithmic bytes over the median call duration; the mean and the
    20th/80th percentiles are reported beside it."""
    import numpy as np
    med_s = float(np.median(ms)) * 1e-3
    achieved = alg_bytes / med_s / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": int(alg_bytes),
            "statistic": f"median of {len(ms)} {timing}",
            "frac_of_mean": round(alg_bytes / (float(ms.mean()) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "frac_p20_p80": [round(alg_bytes / (float(np.quantile(ms, q)) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                             for q in (0.8, 0.2)]}


# ----------------------------------------------------------------------------------------
# the oracle baseline (host cores): the oracle as it stands, timed with perf_counter around the
# oracle call only (host copies and data preparation excluded), repeated until a time budget
# ----------------------------------------------------------------------------------------
def blas_threads():
    from threadpoolctl import threadpool_info
    return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))


def time_oracle(run_once, budget_s, max_reps=50):
    """(reps, seconds): run_once() repeated until `budget_s` seconds of it (at least once)."""
    reps, t_total = 0, 0.0
    while reps < max_reps and (reps == 0 or t_total < budget_s):
        t0 = time.perf_counter()
        run_once()
        t_total += time.perf_counter() - t0
        reps += 1
    return reps, t_total


def cpu_baseline(wl, hk_bits, hv_bits, budget_s=12.0, max_reps=50):
    """Llama-8B step: the oracle's append + float64 decode over the whole workload."""
    import numpy as np
    import torch
    import oracle

    nk = wl.new_k.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    nv = wl.new_v.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    q = wl.q.float().cpu().numpy()
    slots = wl.slot_mapping.numpy()
    state = {}

    def prepare():
        state["k"], state["v"] = hk_bits.copy(), hv_bits.copy()

    def run():
        oracle.append_ref(nk, nv, slots, state["k"], state["v"], oracle.CacheSpec("same", "bf16"),
                          wl.block_size)
        oracle.paged_decode_ref(q, oracle.PoolView("same", state["k"], dtype="bf16"),
                                oracle.PoolView("same", state["v"], dtype="bf16"), wl.block_tables.numpy(),
                                wl.ctx_after.numpy(), wl.block_size, wl.num_kv_heads, wl.sm_scale)

    reps, t_total = 0, 0.0
    while reps < max_reps and (reps == 0 or t_total < budget_s):
        prepare()                                   # fresh pools, outside the timed region
        r, t = time_oracle(run, 0.0, 1)
        reps, t_total = reps + r, t_total + t
    dec, app, _ = algorithmic_bytes(wl)
    return {"value": (dec + app) * reps / t_total / 1e9, "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"the full workload (64 requests: append + decode, float64 numpy), "
                      f"{reps} rep(s), {t_total:.1f} s"}


def _host_codes(t, kind):
    """Device pool (or view) rows -> the numpy array the oracle's PoolView reads."""
    import numpy as np
    import torch
    t = t.contiguous()
    if kind == "same":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if kind == "u3":
        return t.cpu().numpy().view(np.uint32)
    return t.view(torch.uint8).cpu().numpy()


def decode_cpu_baseline(q, kc, vc, km, vm, kind, dtype, block_tables, ctx, block_size, num_kv_heads,
                        sm_scale, reqs, row_bytes, budget_s=8.0, scale_strides=None):
    """The oracle's float64 paged decode over requests `reqs` of a decode workload: their
    blocks of each device pool are gathered into compact host pools (outside the timed
    region) and the oracle decodes them through a renumbered block table.  Reported rate:
    the sample's algorithmic bytes (its tokens' K/V rows of `row_bytes` per kv head, q, out
    and table entries) per second."""
    import numpy as np
    import torch
    import oracle

    bt, ctx = block_tables.cpu(), ctx.cpu()
    ids, rows_bt, lens = [], [], []
    off = 0
    for b in reqs:
        L = int(ctx[b])
        nblk = -(-L // block_size)
        ids.append(bt[b, :nblk].long())
        rows_bt.append(list(range(off, off + nblk)))
        lens.append(L)
        off += nblk
    maxblk = max(1, max(len(r) for r in rows_bt))
    table = np.zeros((len(reqs), maxblk), dtype=np.int32)
    for j, r in enumerate(rows_bt):
        table[j, :len(r)] = r
    sel = torch.cat(ids).to(kc.device) if off else torch.zeros(0, dtype=torch.long, device=kc.device)
    hk, hv = _host_codes(kc[sel], kind), _host_codes(vc[sel], kind)
    mk = mv = None
    if km is not None:
        if scale_strides is not None:                 # caller-given scales: read flat, as given
            mk, mv = km.cpu().numpy(), vm.cpu().numpy()
        else:
            mk, mv = km[sel].cpu().numpy(), vm[sel].cpu().numpy()
    head_dim = q.shape[-1]
    kp = oracle.PoolView(kind, hk, mk, dtype=dtype, head_dim=head_dim, scale_strides=scale_strides)
    vp = oracle.PoolView(kind, hv, mv, dtype=dtype, head_dim=head_dim, scale_strides=scale_strides)
    qh = q[torch.tensor(list(reqs), device=q.device)].float().cpu().numpy()
    lens = np.array(lens, dtype=np.int32)

    def run():
        oracle.paged_decode_ref(qh, kp, vp, table, lens, block_size, num_kv_heads, sm_scale)

    reps, t_total = time_oracle(run, budget_s)
    Hq, D = q.shape[1], q.shape[2]
    nbytes = (int(lens.sum()) * num_kv_heads * row_bytes + 2 * len(reqs) * Hq * D * 2
              + 4 * int(sum(len(r) for r in rows_bt)) + 4 * len(reqs))
    return {"value": nbytes * reps / t_total / 1e9, "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{len(reqs)} of {q.shape[0]} requests ({int(lens.sum())} context tokens, "
                      f"float64 numpy decode), {reps} rep(s), {t_total:.1f} s"}


# ----------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------
def run_llama8b(args, P, W):
    import numpy as np
    import torch
    layers = [W.llama8b_decode("cuda", data_seed=W.BASE_SEED + 2 + 1000 * i, poison=(i == 0))
              for i in range(N_LAYERS)]
    wl0 = layers[0]
    host_k = host_v = None
    if not args.no_cpu_baseline:
        host_k = wl0.k_pool.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
        host_v = wl0.v_pool.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).copy()
    B, Hq, D = wl0.batch, wl0.num_q_heads, wl0.head_dim
    maxctx = max(w.max_context_len for w in layers)
    dev = [dict(bt=w.block_tables.cuda(), ctx=w.ctx_after.cuda(), slots=w.slot_mapping.cuda(),
                out=torch.empty_like(w.q),
                ws=P.decode_workspace(B, Hq, wl0.num_kv_heads, D, maxctx, args.partition_size))
           for w in layers]
    stream = torch.cuda.current_stream()

    def append(i):
        w, d = layers[i % N_LAYERS], dev[i % N_LAYERS]
        P.kv_append(w.new_k, w.new_v, d["slots"], w.k_pool, w.v_pool)

    def decode(i):
        w, d = layers[i % N_LAYERS], dev[i % N_LAYERS]
        P.paged_decode(w.q, w.k_pool, w.v_pool, d["bt"], d["ctx"], w.max_context_len, w.sm_scale,
                       partition_size=args.partition_size, workspace=d["ws"], out=d["out"])

    def fused(i):
        w, d = layers[i % N_LAYERS], dev[i % N_LAYERS]
        P.paged_decode_append(w.q, w.new_k, w.new_v, w.k_pool, w.v_pool, d["bt"], d["ctx"], w.max_context_len,
                              w.sm_scale, partition_size=args.partition_size, workspace=d["ws"], out=d["out"])

    # the step: one paged_decode_append launch (the new tokens appended by the decode's own
    # workgroups), or with --separate-append kv_append then paged_decode
    def step(i):
        if args.separate_append:
            append(i)
            decode(i)
        else:
            fused(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The steps of the four layers are captured in one HIP graph, as a serving loop would run
    # them (the library allocates nothing and records no memset); the timed region replays it.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(N_LAYERS):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(N_LAYERS):
            step(i)
    replays, rest = divmod(args.steps, N_LAYERS)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        graph.replay()
    for i in range(rest):                      # exactly args.steps steps
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # The replayed steps must give what eager calls give, up to the decode's summation order: the
    # order of a row's sums depends on timing, and each result is within the attention tolerance
    # (2e-3 plus half a bf16 unit in the last place at the value) of the exact one, so two of
    # them differ by at most twice that.
    graph_out = [d["out"].clone() for d in dev]
    for i in range(N_LAYERS):
        step(i)
    torch.cuda.synchronize()
    for d, g in zip(dev, graph_out):
        e, r = d["out"].float(), g.float()
        half_ulp = torch.exp2(torch.floor(torch.log2(e.abs().clamp_min(2.0 ** -126))) - 8)
        assert bool(((e - r).abs() <= 2 * (2e-3 + half_ulp)).all()), "graph replay differs from eager"

    # per-entry-point durations with events on the launch stream
    step_ms = None if args.separate_append else call_times_ms(fused, args, stream)
    dec_ms = call_times_ms(decode, args, stream)
    app_ms, _ = graph_call_times_ms([lambda i=i: append(i) for i in range(N_LAYERS)],
                                    max(1, args.steps // N_LAYERS))
    for d in dev:
        assert torch.isfinite(d["out"].float()).all(), "non-finite decode output"

    _, app_b, _ = algorithmic_bytes(wl0)
    dec_bytes_all = float(np.mean([algorithmic_bytes(w)[0] for w in layers]))
    value = (dec_bytes_all + app_b) / (ms_per_step * 1e-3) / 1e9
    config = {"workload": "llama8b-decode-step", "batch": B, "num_q_heads": Hq,
              "num_kv_heads": wl0.num_kv_heads, "head_dim": D, "block_size": wl0.block_size,
              "context": "U{512..4096} cached + 1 appended", "layers_rotated": N_LAYERS,
              "partition_size": args.partition_size or "auto",
              "step": "kv_append + paged_decode" if args.separate_append else "paged_decode_append",
              "launch": "one HIP graph of the four layers' steps, replayed"}
    rec = base_record(args, METRIC, value, "GB/s", ms_per_step, "bf16", config)
    ds, aps = stats_us(dec_ms), stats_us(app_ms)
    rec.update({
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_us": ds, "decode_us_median": ds["median"], "decode_us_p20_p80": ds["p20_p80"],
        "decode_timing": "paged_decode alone (over the appended pools), event-timed calls",
        "append_us_median": aps["median"],
        "append_tokens_per_s": round(B / (aps["median"] * 1e-6), 1),
        "append_timing": "kv_append alone, graph replay of the 4 per-layer appends (launch-bound)",
    })
    if args.separate_append:
        rec["roofline"] = hbm_roofline("paged_decode (decode_kernel + merge)", dec_bytes_all,
                                       dec_ms, recorded_traffic("paged_decode"))
    else:
        rec["step_us"] = stats_us(step_ms)
        rec["roofline"] = hbm_roofline("paged_decode_append (decode_kernel with the step's append + merge)",
                                       dec_bytes_all + app_b, step_ms, recorded_traffic("paged_decode_append"))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl0, host_k, host_v)
    return rec


def run_mixed_append(args, P, W):
    """kv_append of a mixed prefill + decode batch into an fp8 e4m3fn cache; 8 input/pool
    copies in rotation so that neither the inputs nor the pool stay in the Infinity Cache."""
    import torch
    n_copies = 8
    wl = W.mixed_append("cuda", pad_frac=args.pad_frac)
    T = wl.slot_mapping.numel()
    valid = int((wl.slot_mapping >= 0).sum())
    H, D, BS, NB = wl.num_kv_heads, wl.head_dim, wl.block_size, wl.num_blocks
    sets = []
    for i in range(n_copies):
        kc = torch.zeros((NB, BS, H, D), dtype=torch.uint8, device="cuda")
        sets.append(dict(k=wl.new_k.clone(), v=wl.new_v.clone(), slots=wl.slot_mapping.cuda(),
                         kc=kc, vc=torch.zeros_like(kc),
                         km=torch.zeros((NB, BS, H), dtype=torch.float32, device="cuda"),
                         vm=torch.zeros((NB, BS, H), dtype=torch.float32, device="cuda")))
    stream = torch.cuda.current_stream()

    def call(i):
        s = sets[i % n_copies]
        P.kv_append(s["k"], s["v"], s["slots"], s["kc"], s["vc"], s["km"], s["vm"],
                    cache_dtype="fp8")

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    eager = {k: sets[0][k].clone() for k in ("kc", "vc", "km", "vm")}
    ms, g = graph_call_times_ms([lambda i=i: call(i) for i in range(n_copies)],
                                max(N_EVENT_CALLS, args.steps // n_copies))
    for k in eager:                            # one more replay into cleared pools
        sets[0][k].zero_()
    g.replay()
    torch.cuda.synchronize()
    for k in eager:
        assert torch.equal(sets[0][k], eager[k]), f"graph replay differs from eager append ({k})"
    alg = valid * (2 * H * D * 2 + 2 * H * D + 2 * H * 4) + T * 8
    st = stats_us(ms)
    config = {"workload": "mixed-prefill-decode-append-fp8", "tokens": T, "valid_tokens": valid,
              "pad_frac": args.pad_frac,
              "num_kv_heads": H, "head_dim": D, "block_size": BS, "input": "bf16",
              "cache": "fp8 e4m3fn + fp32 per-row scale", "copies_rotated": n_copies}
    rec = base_record(args, "append tokens/s (mixed prefill + decode, fp8 cache)",
                      valid / (st["median"] * 1e-6), "tokens/s", ms_per_step, "f32", config)
    rec.update({"append_us": st, "timing": f"graph replay of the {n_copies} rotated calls",
                "roofline": hbm_roofline("append_kernel (fp8)", alg, ms, timing="per call from graph replays of the 8 rotated calls")})
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = append_cpu_baseline(wl, valid)
    return rec


def append_cpu_baseline(wl, valid, budget_s=8.0):
    """The oracle's fp8 append (per-row absmax scale, fp32 quotient, RNE e4m3fn codes) of the
    whole mixed batch into host pools."""
    import numpy as np
    import torch
    import oracle
    nk = wl.new_k.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    nv = wl.new_v.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    slots = wl.slot_mapping.cpu().numpy()
    NB, BS, H, D = wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim
    kc, vc = np.zeros((NB, BS, H, D), np.uint8), np.zeros((NB, BS, H, D), np.uint8)
    km, vm = np.zeros((NB, BS, H), np.float32), np.zeros((NB, BS, H), np.float32)

    def run():
        oracle.append_ref(nk, nv, slots, kc, vc, oracle.CacheSpec("fp8", "bf16"), BS, km, vm)

    reps, t_total = time_oracle(run, budget_s)
    return {"value": valid * reps / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the full batch ({slots.size} tokens, {valid} valid; a per-token Python "
                      f"loop over numpy row quantisers), {reps} rep(s), {t_total:.1f} s"}


def run_long_context(args, P, W):
    import torch
    wl = W.long_context("cuda")
    bt, ctx = wl.block_tables.cuda(), wl.ctx_after.cuda()
    ps = args.partition_size or 512
    ws = P.decode_workspace(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                            wl.max_context_len, ps)
    out = torch.empty_like(wl.q)
    stream = torch.cuda.current_stream()

    def call(i):
        P.paged_decode(wl.q, wl.k_pool, wl.v_pool, bt, ctx, wl.max_context_len, wl.sm_scale,
                       partition_size=ps, workspace=ws, out=out)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = call_times_ms(call, args, stream)
    assert torch.isfinite(out.float()).all()
    alg, kv = decode_bytes(wl, 2 * wl.head_dim * 2)
    st = stats_us(ms)
    config = {"workload": "long-context-split-k-decode", "batch": wl.batch,
              "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
              "head_dim": wl.head_dim, "block_size": wl.block_size, "context": "U{32768..131072}",
              "partition_size": ps, "kv_bytes": kv}
    rec = base_record(args, "paged decode KV GB/s (long context, split-K)",
                      alg / (st["median"] * 1e-6) / 1e9, "GB/s", ms_per_step, "bf16", config)
    rec.update({"decode_us": st, "roofline": hbm_roofline("paged_decode (decode_kernel + merge)",
                                                          alg, ms)})
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = decode_cpu_baseline(
            wl.q, wl.k_pool, wl.v_pool, None, None, "same", "bf16", wl.block_tables, wl.ctx_after,
            wl.block_size, wl.num_kv_heads, wl.sm_scale, [0, 1], 2 * wl.head_dim * 2)
    return rec


def run_packed3(args, P, W):
    """3-bit decode; the u3 pools (~232 MB each) are built through the u3 append and four
    copies are used in rotation so that the Infinity Cache does not hold the one read."""
    import torch
    n_copies = 4
    wl = W.packed3_decode("cuda")
    NB, BS, H, D = wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim
    slots = wl.slot_mapping.cuda()
    pools = []
    for i in range(n_copies):
        kc = torch.zeros((NB, BS, H, D * 3 // 32), dtype=torch.int32, device="cuda")
        vc = torch.zeros_like(kc)
        km = torch.zeros((NB, BS, H, 2), dtype=torch.float16, device="cuda")
        vm = torch.zeros_like(km)
        P.kv_append(wl.new_k, wl.new_v, slots, kc, vc, km, vm, cache_dtype="u3")
        pools.append((kc, vc, km, vm))
    torch.cuda.synchronize()
    n_tok = wl.new_k.shape[0]
    wl.new_k = wl.new_v = None                 # raw rows no longer needed
    bt, ctx = wl.block_tables.cuda(), wl.ctx_after.cuda()
    maxctx = int(wl.ctx_after.max())
    ps = args.partition_size
    ws = P.decode_workspace(wl.batch, wl.num_q_heads, H, D, maxctx, ps)
    out = torch.empty_like(wl.q)
    stream = torch.cuda.current_stream()

    def call(i):
        kc, vc, km, vm = pools[i % n_copies]
        P.paged_decode(wl.q, kc, vc, bt, ctx, maxctx, wl.sm_scale, k_meta=km, v_meta=vm,
                       partition_size=ps, workspace=ws, out=out, cache_dtype="u3")

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = call_times_ms(call, args, stream)
    assert torch.isfinite(out.float()).all()
    alg, kv = decode_bytes(wl, 2 * (D * 3 // 8 + 4))     # 48 B codes + 4 B (s, z), K and V
    st = stats_us(ms)
    config = {"workload": "packed3-decode", "batch": wl.batch, "num_q_heads": wl.num_q_heads,
              "num_kv_heads": H, "head_dim": D, "block_size": BS, "context": "U{1024..16384}",
              "cache": "3-bit affine, fp16 (scale, zero) per row", "query": "fp16",
              "tokens": n_tok, "kv_bytes": kv, "copies_rotated": n_copies,
              "partition_size": ps or "auto"}
    rec = base_record(args, "paged decode KV GB/s (3-bit packed cache)",
                      alg / (st["median"] * 1e-6) / 1e9, "GB/s", ms_per_step, "f16", config)
    rec.update({"decode_us": st, "roofline": hbm_roofline("paged_decode (decode_kernel u3 + merge)",
                                                          alg, ms)})
    if not args.no_cpu_baseline:
        kc, vc, km, vm = pools[0]
        rec["cpu_baseline"] = decode_cpu_baseline(
            wl.q, kc, vc, km, vm, "u3", "f16", wl.block_tables, wl.ctx_after, BS, H, wl.sm_scale,
            list(range(8)), 2 * (D * 3 // 8 + 4))
    return rec


BYTE_CACHES = {"fp8": ("fp8-decode", "fp8 e4m3fn"), "e5m2": ("e5m2-decode", "fp8 e5m2"),
               "i8": ("int8-decode", "int8")}
TOP = {"fp8": 448.0, "e5m2": 57344.0, "i8": 127.0}


def run_fp8_decode(args, P, W, kind="fp8", per_tensor=False):
    """paged_decode at the Llama-8B shape over byte-code pools (fp8 e4m3fn, fp8 e5m2 or int8,
    one fp32 scale per row), quantised from four bf16 layer pools through kv_append and read in
    rotation.  per_tensor: one caller-given scale per pool (kv_append_scaled /
    paged_decode_scaled) instead of one scale per row."""
    import torch
    name, label = BYTE_CACHES[kind]
    if per_tensor:
        name = name.replace("-decode", "-tensor-scale-decode")
    strides = (0, 0, 0) if per_tensor else None
    pools = []
    for i in range(N_LAYERS):
        wl = W.llama8b_decode("cuda", data_seed=W.BASE_SEED + 2 + 1000 * i, poison=False)
        NB, BS, H, D = wl.k_pool.shape
        kc = torch.empty((NB, BS, H, D), dtype=torch.uint8, device="cuda")
        vc = torch.empty_like(kc)
        if per_tensor:
            km = (wl.k_pool.abs().max().float() / TOP[kind]).reshape(1)
            vm = (wl.v_pool.abs().max().float() / TOP[kind]).reshape(1)
        else:
            km = torch.empty((NB, BS, H), dtype=torch.float32, device="cuda")
            vm = torch.empty_like(km)
        slots = torch.arange(NB * BS, dtype=torch.int64, device="cuda")
        P.kv_append(wl.k_pool.reshape(NB * BS, H, D), wl.v_pool.reshape(NB * BS, H, D), slots,
                    kc, vc, km, vm, cache_dtype=kind, scale_strides=strides)
        torch.cuda.synchronize()
        wl.k_pool = wl.v_pool = None               # the bf16 pools are no longer needed
        pools.append((wl, kc, vc, km, vm))
    wl0 = pools[0][0]
    B, Hq, H, D = wl0.batch, wl0.num_q_heads, wl0.num_kv_heads, wl0.head_dim
    maxctx = max(int(p[0].ctx_before.max()) for p in pools)
    dev = [dict(bt=w.block_tables.cuda(), ctx=w.ctx_before.cuda(), out=torch.empty_like(w.q)) for w, *_ in pools]
    ws = P.decode_workspace(B, Hq, H, D, maxctx, args.partition_size)
    stream = torch.cuda.current_stream()

    def call(i):
        w, kc, vc, km, vm = pools[i % N_LAYERS]
        d = dev[i % N_LAYERS]
        P.paged_decode(w.q, kc, vc, d["bt"], d["ctx"], int(w.ctx_before.max()), w.sm_scale,
                       k_meta=km, v_meta=vm, partition_size=args.partition_size, workspace=ws,
                       out=d["out"], cache_dtype=kind, scale_strides=strides)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = call_times_ms(call, args, stream)
    for d in dev:
        assert torch.isfinite(d["out"].float()).all(), "non-finite decode output"
    algs = []
    for w, *_ in pools:
        w.ctx_after = w.ctx_before                 # decode only: the pools hold ctx_before tokens
        # D codes + one fp32 scale per row, K and V (a per-tensor scale is one value per call)
        algs.append(decode_bytes(w, 2 * D if per_tensor else 2 * (D + 4))[0])
    alg = float(sum(algs) / len(algs))
    st = stats_us(ms)
    tokens = int(sum(int(w.ctx_before.sum()) for w, *_ in pools) / N_LAYERS)
    config = {"workload": name, "batch": B, "num_q_heads": Hq, "num_kv_heads": H,
              "head_dim": D, "block_size": wl0.block_size, "context": "U{512..4096}",
              "cache": f"{label} + fp32 {'per-tensor' if per_tensor else 'per-row'} scale", "query": "bf16",
              "layers_rotated": N_LAYERS, "partition_size": args.partition_size or "auto"}
    rec = base_record(args, f"paged decode KV GB/s ({label} cache{', per-tensor scale' if per_tensor else ''})",
                      alg / (st["median"] * 1e-6) / 1e9, "GB/s", ms_per_step, "bf16", config)
    rec.update({"decode_us": st, "context_tokens_per_s": round(tokens / (st["median"] * 1e-6), 1),
                "roofline": hbm_roofline(f"paged_decode (decode_kernel {kind} + merge)", alg, ms)})
    if not args.no_cpu_baseline:
        w, kc, vc, km, vm = pools[0]
        rec["cpu_baseline"] = decode_cpu_baseline(
            w.q, kc, vc, km, vm, kind, "bf16", w.block_tables, w.ctx_before, w.block_size,
            w.num_kv_heads, w.sm_scale, list(range(16)), 2 * D if per_tensor else 2 * (D + 4),
            scale_strides=strides)
    return rec


def run_contiguous(args, P, W):
    """paged_decode at the Llama-8B shape over the contiguous cache [batch, num_kv_heads,
    max_seq_len = 4352, head_dim] (room for the longest context, 4097 tokens, in whole 16-token
    blocks), read through a virtual block table (virtual block b * Hkv * S / 16 + j = tokens
    16 j .. 16 j + 15 of request b, block stride 16 D, head stride S D); four layer caches in
    rotation."""
    import torch
    S, VBS = 4352, 16
    layers = []
    for i in range(N_LAYERS):
        wl = W.llama8b_decode("cuda", data_seed=W.BASE_SEED + 2 + 1000 * i, poison=False)
        NB, BS, H, D = wl.k_pool.shape
        B = wl.batch
        caches = []
        for pool in (wl.k_pool, wl.v_pool):
            c = torch.zeros((B, H, S, D), dtype=wl.dtype, device="cuda")
            for b, blks in enumerate(wl.blocks_of):
                assert len(blks) * BS <= S, "context longer than the contiguous cache"
                rows = pool[torch.tensor(blks, device="cuda")].reshape(len(blks) * BS, H, D)
                c[b, :, :rows.shape[0]] = rows.permute(1, 0, 2)
            caches.append(c)
        torch.cuda.synchronize()
        wl.k_pool = wl.v_pool = None
        nbv = (B - 1) * H * S // VBS + S // VBS
        views = [torch.as_strided(c, (nbv, VBS, H, D), (VBS * D, D, S * D, 1)) for c in caches]
        table = (torch.arange(B, dtype=torch.int32)[:, None] * (H * S // VBS)
                 + torch.arange(S // VBS, dtype=torch.int32)[None, :]).cuda()
        layers.append((wl, caches, views, table, wl.ctx_before.cuda(), torch.empty_like(wl.q)))
    wl0 = layers[0][0]
    B, Hq, H, D = wl0.batch, wl0.num_q_heads, wl0.num_kv_heads, wl0.head_dim
    maxctx = max(int(l[0].ctx_before.max()) for l in layers)
    ws = P.decode_workspace(B, Hq, H, D, maxctx, args.partition_size)
    stream = torch.cuda.current_stream()

    def call(i):
        w, _, views, table, ctx, out = layers[i % N_LAYERS]
        P.paged_decode(w.q, views[0], views[1], table, ctx, int(w.ctx_before.max()), w.sm_scale,
                       partition_size=args.partition_size, workspace=ws, out=out)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = call_times_ms(call, args, stream)
    for l in layers:
        assert torch.isfinite(l[5].float()).all(), "non-finite decode output"
    algs = []
    for l in layers:
        w = l[0]
        w.ctx_after = w.ctx_before
        algs.append(decode_bytes(w, 2 * D * 2)[0])
    alg = float(sum(algs) / len(algs))
    st = stats_us(ms)
    config = {"workload": "contiguous-decode", "batch": B, "num_q_heads": Hq, "num_kv_heads": H,
              "head_dim": D, "max_seq_len": S, "context": "U{512..4096}",
              "layout": "[batch, num_kv_heads, max_seq_len, head_dim], virtual 16-token blocks",
              "layers_rotated": N_LAYERS, "partition_size": args.partition_size or "auto"}
    rec = base_record(args, "paged decode KV GB/s (contiguous cache)",
                      alg / (st["median"] * 1e-6) / 1e9, "GB/s", ms_per_step, "bf16", config)
    rec.update({"decode_us": st, "roofline": hbm_roofline("paged_decode (decode_kernel + merge)", alg,
                                                          ms)})
    if not args.no_cpu_baseline:
        w, _, views, table, ctx, _ = layers[0]
        rec["cpu_baseline"] = decode_cpu_baseline(
            w.q, views[0], views[1], None, None, "same", "bf16", table, ctx, VBS, H, w.sm_scale,
            list(range(16)), 2 * D * 2)
    return rec


def run_dual_stacked(args, P, W):
    """paged_decode at the Llama-8B shape over the dual-stacked block layout
    [num_blocks, 2, num_kv_heads, block_size, head_dim] (K and V of a block in one buffer,
    head-major inside the block), passed as two strided views; four layer pools in rotation."""
    import torch
    layers = []
    for i in range(N_LAYERS):
        wl = W.llama8b_decode("cuda", data_seed=W.BASE_SEED + 2 + 1000 * i, poison=False)
        NB, BS, H, D = wl.k_pool.shape
        buf = torch.empty((NB, 2, H, BS, D), dtype=wl.dtype, device="cuda")
        kc, vc = buf[:, 0].permute(0, 2, 1, 3), buf[:, 1].permute(0, 2, 1, 3)
        kc.copy_(wl.k_pool)
        vc.copy_(wl.v_pool)
        torch.cuda.synchronize()
        wl.k_pool = wl.v_pool = None
        layers.append((wl, buf, kc, vc, wl.block_tables.cuda(), wl.ctx_before.cuda(), torch.empty_like(wl.q)))
    wl0 = layers[0][0]
    B, Hq, H, D = wl0.batch, wl0.num_q_heads, wl0.num_kv_heads, wl0.head_dim
    maxctx = max(int(l[0].ctx_before.max()) for l in layers)
    ws = P.decode_workspace(B, Hq, H, D, maxctx, args.partition_size)
    stream = torch.cuda.current_stream()

    def call(i):
        w, _, kc, vc, bt, ctx, out = layers[i % N_LAYERS]
        P.paged_decode(w.q, kc, vc, bt, ctx, int(w.ctx_before.max()), w.sm_scale,
                       partition_size=args.partition_size, workspace=ws, out=out)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = call_times_ms(call, args, stream)
    for l in layers:
        assert torch.isfinite(l[6].float()).all(), "non-finite decode output"
    algs = []
    for l in layers:
        w = l[0]
        w.ctx_after = w.ctx_before
        algs.append(decode_bytes(w, 2 * D * 2)[0])
    alg = float(sum(algs) / len(algs))
    st = stats_us(ms)
    config = {"workload": "dual-stacked-decode", "batch": B, "num_q_heads": Hq, "num_kv_heads": H,
              "head_dim": D, "block_size": wl0.block_size, "context": "U{512..4096}",
              "layout": "[num_blocks, 2, num_kv_heads, block_size, head_dim]", "layers_rotated": N_LAYERS,
              "partition_size": args.partition_size or "auto"}
    rec = base_record(args, "paged decode KV GB/s (dual-stacked block layout)",
                      alg / (st["median"] * 1e-6) / 1e9, "GB/s", ms_per_step, "bf16", config)
    rec.update({"decode_us": st, "roofline": hbm_roofline("paged_decode (decode_kernel + merge)", alg,
                                                          ms)})
    if not args.no_cpu_baseline:
        w, _, kc, vc, bt, ctx, _ = layers[0]
        rec["cpu_baseline"] = decode_cpu_baseline(
            w.q, kc, vc, None, None, "same", "bf16", bt, ctx, w.block_size, H, w.sm_scale,
            list(range(16)), 2 * D * 2)
    return rec


def run_pack3_exhaustive(args, P, W):
    """pack3 + unpack3 over every 24-bit octet: values v_j(i) = (i >> 3j) & 7 must pack to
    the three little-endian bytes of i, and unpack back."""
    import torch
    n_oct = 1 << 24
    i = torch.arange(n_oct, dtype=torch.int32, device="cuda")
    values = torch.stack([((i >> (3 * j)) & 7).to(torch.uint8) for j in range(8)], dim=1).reshape(-1)
    want_packed = torch.stack([((i >> (8 * j)) & 255).to(torch.uint8) for j in range(3)], dim=1).reshape(-1)
    del i
    packed = torch.empty(3 * n_oct, dtype=torch.uint8, device="cuda")
    back = torch.empty_like(values)
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        P.pack3(values, packed)
        P.unpack3(packed, values.numel(), back)
    torch.cuda.synchronize()
    pk = call_times_ms(lambda _: P.pack3(values, packed), args, stream)
    up = call_times_ms(lambda _: P.unpack3(packed, values.numel(), back), args, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    P.pack3(values, packed)
    P.unpack3(packed, values.numel(), back)
    ok = bool(torch.equal(packed, want_packed)) and bool(torch.equal(back, values))
    torch.cuda.synchronize()
    e2e_ms = (time.perf_counter() - t0) * 1e3
    assert ok, "exhaustive pack3/unpack3 check failed"
    ps, us = stats_us(pk), stats_us(up)
    nbytes = values.numel() + packed.numel()
    config = {"workload": "pack3-exhaustive-2^24", "octets": n_oct, "values_bytes": values.numel(),
              "packed_bytes": packed.numel()}
    rec = base_record(args, "exhaustive 2^24 pack3/unpack3 check time", e2e_ms, "ms", e2e_ms, "u8",
                      config, higher=False)
    rec.update({"pack3_us": ps, "unpack3_us": us, "check_passed": ok,
                "roofline": hbm_roofline("unpack3_kernel", nbytes, up),
                "pages_figures": {"cpu_exhaustive_s": 0.91, "gpu_exhaustive_ms": 1982.2,
                                  "hardware": "RTX 3060 Laptop GPU (Triton 3.2.0) and its host CPU"}})
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = pack3_cpu_baseline(values, want_packed)
    return rec


def pack3_cpu_baseline(values, want_packed):
    """The oracle's vectorised pack3 then unpack3 over all 2^24 octets on one core, with both
    comparisons (the form of the 3-bit page's CPU exhaustive check)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    vh, wh = values.cpu().numpy(), want_packed.cpu().numpy()
    with threadpool_limits(1):
        t0 = time.perf_counter()
        pk = oracle.pack3(vh)
        back = oracle.unpack3(pk)
        ok = bool(np.array_equal(pk, wh)) and bool(np.array_equal(back, vh))
        t = time.perf_counter() - t0
    assert ok, "the oracle's exhaustive pack3/unpack3 check failed"
    return {"value": round(t * 1e3, 1), "unit": "ms", "cores": 1, "kind": "oracle",
            "sample": "all 2^24 octets, pack3 then unpack3 of the packed bytes, both compared "
                      "(vectorised numpy, one thread), 1 rep"}


def run_add_calibration(args, P, W):
    """torch.add(a, b, out=c) over bf16 tensors whose traffic matches the mixed fp8 append's
    algorithmic bytes (two thirds read, one third written), 8 sets in rotation: the rate a
    plain streaming kernel reaches at that size, beside the append's."""
    import torch
    total = 64263976
    n = total // 3 // 2
    sets = [tuple(torch.randn(n, device="cuda", dtype=torch.bfloat16) for _ in range(3)) for _ in range(8)]
    stream = torch.cuda.current_stream()

    def call(i):
        a, b, c = sets[i % 8]
        torch.add(a, b, out=c)

    for i in range(max(1, args.warmup)):
        call(i)
    ms = call_times_ms(call, args, stream)
    st = stats_us(ms)
    config = {"workload": "add-calibration", "bytes_read": 4 * n, "bytes_written": 2 * n, "sets_rotated": 8}
    rec = base_record(args, "elementwise add GB/s (read + write)", 6 * n / (st["median"] * 1e-6) / 1e9,
                      "GB/s", st["median"] * 1e-3, "bf16", config)
    rec.update({"add_us": st, "timing": "event-timed eager calls",
                "roofline": hbm_roofline("torch add", 6 * n, ms)})
    return rec


def run_copy_calibration(args, P, W):
    """A plain device-to-device copy of 1 GiB (torch's copy kernel): the known-size
    transfer that the HBM byte counters of the decode kernel are scaled by."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        dst.copy_(src)
    ms = call_times_ms(lambda _: dst.copy_(src), args, stream)
    st = stats_us(ms)
    config = {"workload": "copy-calibration", "bytes_read": n, "bytes_written": n}
    rec = base_record(args, "device copy GB/s (read + write)", 2 * n / (st["median"] * 1e-6) / 1e9,
                      "GB/s", st["median"] * 1e-3, "u8", config)
    rec["copy_us"] = st
    if not args.no_cpu_baseline:
        import numpy as np
        a = np.ones(1 << 28, dtype=np.uint8)
        b = np.empty_like(a)
        reps, t = time_oracle(lambda: np.copyto(b, a), 2.0)
        rec["cpu_baseline"] = {"value": 2 * a.size * reps / t / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "host copy",
                               "sample": f"numpy copy of 256 MiB (the calibration has no oracle), {reps} rep(s)"}
    return rec


WORKLOADS = {"llama8b-decode-step": run_llama8b, "mixed-append-fp8": run_mixed_append,
             "long-context": run_long_context, "packed3-decode": run_packed3,
             "pack3-exhaustive": run_pack3_exhaustive, "copy-calibration": run_copy_calibration,
             "add-calibration": run_add_calibration,
             "fp8-decode": run_fp8_decode, "dual-stacked-decode": run_dual_stacked,
             "e5m2-decode": lambda a, P, W: run_fp8_decode(a, P, W, "e5m2"),
             "int8-decode": lambda a, P, W: run_fp8_decode(a, P, W, "i8"),
             "fp8-tensor-scale-decode": lambda a, P, W: run_fp8_decode(a, P, W, "fp8", True),
             "contiguous-decode": run_contiguous}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pad-frac", type=float, default=0.10)
    ap.add_argument("--separate-append", action="store_true",
                    help="Llama-8B step as kv_append then paged_decode instead of one paged_decode_append")
    ap.add_argument("--workload", default="llama8b-decode-step", choices=sorted(WORKLOADS))
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no "
              "multi-GPU component to measure.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_45_amd as P
    from paged_kv_cache_45_amd import workloads as W

    torch.cuda.set_device(0)
    P.load_library()
    rec = WORKLOADS[args.workload](args, P, W)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

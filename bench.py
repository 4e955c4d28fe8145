"""Benchmark of one stratified sparse decode step (one attention layer).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1m|128k|32k|batched]

A step is one ssa_decode call over the whole layer: scores, top-k, tail
sampling, gather attention and merge, with inputs already resident in HBM.
Prints one JSON line: KV-tokens/s/layer (sum of sequence lengths / step
time), the indexer's roofline against MI355X's 8 TB/s HBM peak (HIP events
around the indexer launch inside the timed region), per-stage times from a
separate event-bracketed pass, per-step medians with and without a 512 MiB
cache-evicting read before each step, the 128K workload, and variants of the main
workload: a top-p capped deterministic stratum, early stopping over it, split
keys (on the device and with the rest of the keys and the values in pinned
host memory) with the cache append, and multi-token decode with shared and
per-query selections; then the CPU oracle timed on a bounded sample of the
same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-decode KV-tokens/s/layer + HBM GB/s vs peak at L=128K and L=1M"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
INDEXER_SOURCES = [os.path.join(ROOT, "long_context_sparse_approx_amd", "csrc", f)
                   for f in ("indexer.hip", "ssa_device.h")]

WORKLOADS = {
    "1m": "1M-token decode: B=1, 32 q / 8 kv heads, d=128, L=1048576, bf16 paged KV "
          "(16-token blocks, shuffled), RoPE theta=1e6, 256 planted keys per kv head, "
          "50x budget = top-k 10486 + sampled 10486, split-K over 256 chunks",
    "128k": "128K decode, batch 4: 32 q / 8 kv heads, d=128, L=131072 each, heavy-tailed keys "
            "(90% N(0,1), 10% N(0,9)), 50x budget = top-k 1311 + sampled 1310",
    "32k": "32K decode: B=1, 32 q / 8 kv heads, d=128, L=32768, 64 planted keys per kv head, "
           "50x budget = top-k 328 + sampled 327",
    "batched": "batched paged decode: B=32, L log-uniform in [8192, 131072], 32 q / 8 kv heads, "
               "d=128, per-sequence 50x budget split top-k/sampled, seeds 1000+b",
}


class Hip:
    """hipEvent helpers from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.h.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, e):
        self.h.hipEventDestroy(ctypes.c_void_p(e))


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per indexer launch from the committed rocprofv3 counter
    summary, or None if there is none or the kernel changed since."""
    path = os.path.join(PROFILES, f"indexer_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^kernel_source_sha256_16:\s*(\S+)", text, re.M)
    t = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m or not t or m.group(1) != source_digest(INDEXER_SOURCES):
        return None
    return float(t.group(1))


def split_keys(wl, host):
    """(k_dom, k_rest, v) of the workload's cache in the split key layout,
    cut with torch slicing; with ``host`` the rest of the keys and the values
    live in pinned host memory."""
    import torch

    lo, hi = 2 * wl.pair_begin, 2 * (wl.pair_begin + wl.pair_count)
    k_dom = wl.k_cache[..., lo:hi].contiguous()
    k_rest = torch.cat([wl.k_cache[..., :lo], wl.k_cache[..., hi:]], dim=-1).contiguous()
    v = wl.v_cache
    if host:
        k_rest, v = k_rest.cpu().pin_memory(), v.cpu().pin_memory()
    return k_dom, k_rest, v


def run_gpu(args, name, steps, warmup, with_stage_events=True, top_p=None, wl=None,
            num_queries=1, query_group=1, early_stop=0.0, keys="whole", refine=0,
            ceilings=False):
    """Times `steps` decode steps (after `warmup` untimed ones) of a workload.
    ``top_p`` (a float) caps every sequence's deterministic stratum at the
    top-p prefix; ``wl`` reuses an already generated workload; with
    ``num_queries`` T > 1 each step carries T query positions per sequence,
    ``query_group`` of them sharing one selection.  ``keys`` = "split" runs
    over split keys on the device, "split_host" with the rest of the keys and
    the values in pinned host memory."""
    import torch

    from long_context_sparse_approx_amd import ssa, synth

    dev = "cuda:0"
    t_gen = time.perf_counter()
    if wl is None:
        wl = synth.make_workload(name, dev, num_queries=num_queries)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    tp = None if top_p is None else torch.full((wl.B,), top_p, dtype=torch.float32, device=dev)
    split = keys != "whole"
    p = ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                       pair_begin=wl.pair_begin, pair_count=wl.pair_count,
                       query_group=query_group, early_stop=early_stop,
                       key_layout=ssa.SSA_KEYS_SPLIT if split else ssa.SSA_KEYS_WHOLE,
                       max_topk=int(wl.topk.max()), refine=refine)
    ws = ssa.alloc_workspace(p, dev)
    out = torch.empty(wl.q.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    tail = (wl.block_table, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    if split:
        k_dom, k_rest, v_split = split_keys(wl, keys == "split_host")
        call = (p, wl.q, k_dom, k_rest, v_split) + tail
        step = ssa.decode_split
    else:
        call = (p, wl.q, wl.k_cache, wl.v_cache) + tail
        step = ssa.decode
    for _ in range(warmup):
        step(*call, out=out, workspace=ws, stream=stream, top_p=tp)
    torch.cuda.synchronize()

    hip = Hip()
    nst = len(ssa.STAGES)
    ix = ssa.STAGES.index("index")

    def event_arrays(n, stages):
        arrs = []
        for _ in range(n):
            evs = [None] * (2 * nst)
            for k in stages:
                evs[2 * k], evs[2 * k + 1] = hip.event(), hip.event()
            arrs.append((ctypes.c_void_p * (2 * nst))(*evs))
        return arrs

    def timed_loop(arrs, graphs=None, every=1):
        # arrs[i // every] brackets step i when i % every == 0.
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if graphs is not None:
                graphs[i % len(graphs)].replay()
            else:
                ev = arrs[i // every] if arrs and i % every == 0 else None
                step(*call, out=out, workspace=ws, stream=stream, top_p=tp,
                     events=ctypes.addressof(ev) if ev is not None else None)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    # Timed region: K whole steps; on every `event_every`-th of them HIP events
    # bracket the indexer launch (on the decode stream), for its roofline.  An
    # event record costs the GPU about 5 us between two kernels, so bracketing
    # every step would add about 11 us to each.
    every = max(1, args.event_every)
    n_ev = (steps + every - 1) // every
    graphs = None
    if args.graph and not split:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ssa.decode(*call, out=out, workspace=ws, stream=torch.cuda.current_stream(),
                       top_p=tp)
        graphs = [g]
        for _ in range(warmup):
            g.replay()
        idx_arrs = None
    else:
        idx_arrs = event_arrays(n_ev, [ix])
    ms_step = timed_loop(idx_arrs, graphs, every)
    idx_ms = None
    if idx_arrs:
        idx_ms = sum(hip.elapsed_ms(a[2 * ix], a[2 * ix + 1]) for a in idx_arrs) / n_ev
    # Separate pass (not the timed region): every stage bracketed by events.
    stage_ms = {s: 0.0 for s in ssa.STAGES}
    gpu_ms = 0.0
    if with_stage_events:
        all_arrs = event_arrays(steps, range(nst))
        timed_loop(all_arrs)
        for arr in all_arrs:
            for k, s in enumerate(ssa.STAGES):
                stage_ms[s] += hip.elapsed_ms(arr[2 * k], arr[2 * k + 1]) / steps
            gpu_ms += hip.elapsed_ms(arr[0], arr[2 * nst - 1]) / steps
        for arr in all_arrs:
            for e in arr:
                hip.destroy(e)
    for arr in idx_arrs or []:
        hip.destroy(arr[2 * ix])
        hip.destroy(arr[2 * ix + 1])
    # Per-step medians (events from the first stage's start to the last
    # stage's end), cold: a 512 MiB buffer read before every step evicts L2
    # and the 256 MiB Infinity Cache (a read leaves no dirty lines whose
    # write-back would land inside the step); warm: the same steps back to back.
    cache = None
    if args.cold_steps > 0 and graphs is None:
        scrub = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
        scrub_sum = torch.empty((), dtype=torch.float32, device=dev)
        arrs = event_arrays(args.cold_steps, [0, nst - 1])

        def per_step_median_us(cold):
            torch.cuda.synchronize()
            for arr in arrs:
                if cold:
                    torch.sum(scrub, dim=0, out=scrub_sum)
                step(*call, out=out, workspace=ws, stream=stream, top_p=tp,
                     events=ctypes.addressof(arr))
            torch.cuda.synchronize()
            ts = sorted(hip.elapsed_ms(a[0], a[2 * nst - 1]) for a in arrs)
            return round(ts[len(ts) // 2] * 1e3, 2)

        cache = dict(steps=args.cold_steps, scrub_mib=512,
                     cold_median_us=per_step_median_us(True),
                     warm_median_us=per_step_median_us(False))
        for arr in arrs:
            hip.destroy(arr[0])
            hip.destroy(arr[2 * nst - 1])
        del scrub, scrub_sum
    del graphs

    # Selected-set sizes of this step (deterministic: same kernels, same inputs).
    sc = ssa.score(p, wl.q, call[2], wl.block_table, wl.seq_lens, workspace=ws)
    _, _, cnt, _ = ssa.select(p, sc, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed,
                              workspace=ws, top_p=tp, q=wl.q, k_cache=call[2],
                              k_rest=call[3] if split else None, block_table=wl.block_table)
    cnt = cnt.sum(dim=2).cpu()
    n_det, n_smp = int(cnt[..., 0].sum()), int(cnt[..., 1].sum())
    del sc
    torch.cuda.synchronize()

    tokens = float(sum(wl.lens))
    d = wl.d
    groups = ssa.num_groups(p)
    idx_bytes = tokens * wl.Hkv * groups * (2 * wl.pair_count * 2)  # K pair subset per group
    gather_bytes = (n_det + n_smp) * 2.0 * d * 2                # K and V rows
    score_bytes = tokens * wl.Hkv * 4 * 4                       # 1 write + 3 reads
    if split:
        del call, k_dom, k_rest, v_split
    ceil = measure_ceilings(wl, idx_bytes, 2 * (n_det + n_smp)) if ceilings else None
    res = dict(wl=wl, p=p, ms_step=ms_step, idx_ms=idx_ms, gpu_ms=gpu_ms, stage_ms=stage_ms,
               ceilings=ceil,
               tokens=tokens,
               idx_bytes=idx_bytes, gather_bytes=gather_bytes, score_bytes=score_bytes,
               n_det=n_det, n_smp=n_smp, t_gen=t_gen, cache=cache)
    return res


def append_bench(wl, steps, warmup):
    """Cache append in the split key layout: a bulk fill of every token of the
    workload (HBM-bound: each token's key and value rows read once and written
    once) and a one-token append per sequence, as in every decode step."""
    import torch

    from long_context_sparse_approx_amd import ssa

    dev = "cuda:0"
    B, Hkv, d = wl.B, wl.Hkv, wl.d
    T = max(wl.lens)
    assert B == 1, "bulk fill measured on one sequence"
    pos = torch.arange(T, device=dev)
    rows = wl.block_table[0, (pos // 16).long()].long()
    slot = (pos % 16).long()
    k_new = wl.k_cache[rows, :, slot, :].unsqueeze(0).contiguous()  # [1, T, Hkv, d]
    v_new = wl.v_cache[rows, :, slot, :].unsqueeze(0).contiguous()
    del rows, slot, pos
    p = ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                       pair_begin=wl.pair_begin, pair_count=wl.pair_count,
                       key_layout=ssa.SSA_KEYS_SPLIT)
    pc2 = 2 * wl.pair_count
    nblk = wl.k_cache.shape[0]
    k_dom = torch.empty((nblk, Hkv, 16, pc2), dtype=torch.bfloat16, device=dev)
    k_rest = torch.empty((nblk, Hkv, 16, d - pc2), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(wl.v_cache)

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    bulk_ms = timed(lambda: ssa.append_kv(p, k_new, v_new, wl.block_table, wl.seq_lens, k_dom,
                                          k_rest, v), max(3, steps // 5))
    ok = (torch.equal(k_dom, wl.k_cache[..., 2 * wl.pair_begin:2 * wl.pair_begin + pc2])
          and torch.equal(v, wl.v_cache))
    # One-token appends back to back: the time per call is the host's launch
    # rate (the kernel itself runs for about 2 us).
    one_k, one_v = k_new[:, -1:].contiguous(), v_new[:, -1:].contiguous()
    one_ms = timed(lambda: ssa.append_kv(p, one_k, one_v, wl.block_table, wl.seq_lens, k_dom,
                                         k_rest, v), steps)
    nbytes = 2.0 * T * Hkv * (2 * d * 2)  # key + value rows, read once and written once
    gbps = nbytes / (bulk_ms * 1e-3) / 1e9
    del k_new, v_new, k_dom, k_rest, v
    torch.cuda.empty_cache()
    return dict(bulk_tokens=T, bulk_ms=round(bulk_ms, 4), bulk_bytes=nbytes,
                bulk_gbps=round(gbps, 1), bulk_frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4),
                bulk_rebuilds_cache_bitwise=bool(ok),
                one_token_call_us=round(one_ms * 1e3, 2))


def unit_host_inputs(wl, b, h):
    """Host copies of one (sequence, kv head): q group, the head's cache slab
    [nblk, 1, 16, d] and the block-table row (exact bf16 values as float32)."""
    G = wl.Hq // wl.Hkv
    qg = wl.q[b, h * G:(h + 1) * G].float().cpu().numpy().astype("float64")
    kc = wl.k_cache[:, h:h + 1].float().cpu().numpy()
    vc = wl.v_cache[:, h:h + 1].float().cpu().numpy()
    bt = wl.block_table[b].cpu().numpy().astype("int64")
    return qg, kc, vc, bt


def cpu_baseline(wl, budget_s=15.0):
    """The oracle as it stands, on a bounded sample of the workload's units."""
    import numpy as np

    from threadpoolctl import threadpool_limits

    from oracle import ssa_oracle as orc
    # The oracle is plain numpy: sorts, Philox, the specified exp and the row
    # gathers run on one thread; its two small matrix products are held to
    # one BLAS thread too, so the core count below is the one it used.
    limiter = threadpool_limits(limits=1)
    scale = 1.0 / math.sqrt(wl.d)
    units = [(b, h) for b in range(wl.B) for h in range(wl.Hkv)]
    done, tokens, elapsed = 0, 0, 0.0
    for b, h in units:
        qg, kc, vc, bt = unit_host_inputs(wl, b, h)
        L = wl.lens[b]
        t0 = time.perf_counter()
        K = orc.gather_rows(kc, bt, 0, L)
        V = orc.gather_rows(vc, bt, 0, L)
        s = orc.approx_scores(qg, K, wl.pair_begin, wl.pair_count, scale).astype(np.float32)
        sel = orc.select_unit(s, int(wl.topk[b]), int(wl.sample_budget[b]),
                              int(wl.seed[b]) & 0xFFFFFFFFFFFFFFFF, b, h)
        orc.attend_unit(qg, K, V, sel["S"], sel["R"], sel["pi_R"], scale)
        elapsed += time.perf_counter() - t0
        done += 1
        tokens += L
        del K, V, kc, vc
        if elapsed >= budget_s:
            break
    limiter.unregister()
    # One unit is one kv head of one sequence; a layer has Hkv heads per token.
    value = tokens / wl.Hkv / elapsed
    return dict(value=value, unit="KV-tokens/s/layer", cores=1, kind="oracle",
                host_cores=len(os.sched_getaffinity(0)),
                sample=f"{done} of {len(units)} (sequence, kv head) units of the same workload, "
                       f"{tokens} token-heads in {elapsed:.1f} s on one thread (numpy, BLAS "
                       f"limited to 1 thread); layer rate = token-heads / {wl.Hkv} / time")


def measure_ceilings(wl, stream_bytes, gather_rows, reps=7):
    """What HBM delivers on this device for the step's two bandwidth-bound
    access patterns, with the library's measurement kernels: a contiguous read
    of the indexer's byte count (from the key cache), and a gather of the
    attention's K+V row count of d*2-byte rows scattered uniformly over the
    value cache (seeded ids).  Each rep runs after a 512 MiB read that evicts
    L2 and the Infinity Cache; medians of the reps, from HIP events on the
    stream the kernels run on."""
    import torch

    from long_context_sparse_approx_amd import ssa

    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    sink = torch.zeros(ssa.MEASURE_SINK_WORDS, dtype=torch.int32, device=dev)
    scrub = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    scrub_sum = torch.empty((), dtype=torch.float32, device=dev)
    row_bytes = wl.d * 2
    num_rows = wl.v_cache.numel() * 2 // row_bytes
    g = torch.Generator(device=dev).manual_seed(20260)
    rows = torch.randint(0, num_rows, (int(gather_rows),), generator=g, device=dev,
                         dtype=torch.int32)
    nbytes = min(int(stream_bytes), wl.k_cache.numel() * 2) // 16 * 16

    def timed(launch):
        ts = []
        for _ in range(reps + 1):
            torch.sum(scrub, dim=0, out=scrub_sum)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    us_s = timed(lambda: ssa.measure_stream(wl.k_cache, nbytes, sink, stream))
    us_g = timed(lambda: ssa.measure_gather(wl.v_cache, row_bytes, rows, sink, stream))
    del scrub, scrub_sum, rows
    return dict(
        stream_read=dict(bytes=nbytes, us=round(us_s, 2), gbps=round(nbytes / us_s / 1e3, 1)),
        row_gather=dict(rows=int(gather_rows), row_bytes=row_bytes,
                        bytes=int(gather_rows) * row_bytes, us=round(us_g, 2),
                        gbps=round(int(gather_rows) * row_bytes / us_g / 1e3, 1)),
        reps=reps, evict_mib=512)


def summarize(res, workload):
    st = res["stage_ms"]
    roof = None
    if res["idx_ms"]:
        achieved = res["idx_bytes"] / (res["idx_ms"] * 1e-3) / 1e9
        traffic = measured_traffic(workload)
        roof = dict(bound="hbm", kernel="indexer", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBPS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBPS, 4),
                    traffic=traffic,
                    algorithmic_bytes_per_launch=res["idx_bytes"],
                    launch_us=round(res["idx_ms"] * 1e3, 2),
                    # the same launch's rate in measured HBM bytes (read + written)
                    measured_gbps=(round(traffic / (res["idx_ms"] * 1e-3) / 1e9, 1)
                                   if traffic else None))
    step_s = res["ms_step"] * 1e-3
    algo_total = res["idx_bytes"] + res["gather_bytes"]
    # The two HBM-bound kernels together (the path's >= 70% target): their
    # algorithmic bytes over their summed event times from the breakdown pass.
    pair_s = (st["index"] + st["attend"]) * 1e-3
    index_gather = None
    if pair_s > 0:
        gbps = algo_total / pair_s / 1e9
        index_gather = dict(bytes=algo_total, us=round(pair_s * 1e6, 2), gbps=round(gbps, 1),
                            frac=round(gbps / HBM_PEAK_GBPS, 4))
    ceil = res.get("ceilings")
    if roof and ceil:
        roof["measured_ceiling"] = dict(pattern="contiguous read", gbps=ceil["stream_read"]["gbps"])
        roof["frac_of_measured_ceiling"] = round(roof["achieved"] / ceil["stream_read"]["gbps"], 4)
    attention = None
    if st["attend"] > 0:
        gbps = res["gather_bytes"] / (st["attend"] * 1e-3) / 1e9
        attention = dict(bytes=res["gather_bytes"], us=round(st["attend"] * 1e3, 2),
                         gbps=round(gbps, 1), frac=round(gbps / HBM_PEAK_GBPS, 4))
        if ceil:
            attention["measured_ceiling"] = dict(pattern="scattered row gather",
                                                 gbps=ceil["row_gather"]["gbps"])
            attention["frac_of_measured_ceiling"] = round(gbps / ceil["row_gather"]["gbps"], 4)
    cold = None
    if res["cache"]:
        c = res["cache"]
        cold = dict(value=res["tokens"] / (c["cold_median_us"] * 1e-6),
                    us=c["cold_median_us"],
                    hbm_frac_algorithmic=round(algo_total / (c["cold_median_us"] * 1e-6) / 1e9
                                               / HBM_PEAK_GBPS, 4))
    return dict(index_gather=index_gather, cold=cold, attention=attention, ceilings=ceil,
        value=res["tokens"] / step_s, ms_per_step=res["ms_step"], roofline=roof,
        stages_us={k: round(v * 1e3, 2) for k, v in st.items()},
        gpu_step_us=round(res["gpu_ms"] * 1e3, 2),
        hbm_gbps_algorithmic_step=round(algo_total / step_s / 1e9, 1),
        hbm_frac_algorithmic_step=round(algo_total / step_s / 1e9 / HBM_PEAK_GBPS, 4),
        gather_gbps_algorithmic=(round(res["gather_bytes"] / (st["attend"] * 1e-3) / 1e9, 1)
                                 if st["attend"] > 0 else None),
        selected=dict(deterministic=res["n_det"], sampled=res["n_smp"]),
    )


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="1m", choices=sorted(WORKLOADS))
    ap.add_argument("--also", default="128k", help="comma list of extra workloads, or 'none'")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-stage-events", action="store_true",
                    help="skip the separate per-stage breakdown pass")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (no indexer events)")
    ap.add_argument("--top-p", type=float, default=0.02,
                    help="also time the main workload with this top-p stratum cap (0 = skip)")
    ap.add_argument("--early-stop", type=float, default=0.01,
                    help="also time the main workload with this early-stopping threshold "
                         "(0 = skip)")
    ap.add_argument("--multi", type=int, default=4,
                    help="also time the main workload with this many query positions per "
                         "step, one shared selection vs one per query (0 = skip)")
    ap.add_argument("--no-split-keys", dest="split_keys", action="store_false",
                    help="skip the split-key (device and host-offloaded) and append timings")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="per-step medians over this many steps with and without a 512 MiB "
                         "cache-evicting read before each (0 = skip)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="bracket the indexer with HIP events on every N-th timed step")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip timing the measurement kernels (contiguous read and row gather "
                         "of the step's byte and row counts)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("steps must be >= 1 and warmup >= 0")

    import torch
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)  # an elementwise kernel: n bytes read, n bytes written
        torch.cuda.synchronize()
        print(f"copy calibration: {n} bytes read + {n} bytes written per launch", file=sys.stderr)
        del a, b

    res = run_gpu(args, args.workload, args.steps, args.warmup, not args.no_stage_events,
                  ceilings=not args.no_ceilings)
    main_sum = summarize(res, args.workload)
    also = {}
    for name in [w for w in args.also.split(",") if w and w not in ("none", args.workload)]:
        r2 = run_gpu(args, name, args.steps, args.warmup, not args.no_stage_events,
                     ceilings=not args.no_ceilings)
        s2 = summarize(r2, name)
        also[name] = dict(workload=WORKLOADS[name], value=s2["value"], unit="KV-tokens/s/layer",
                          ms_per_step=s2["ms_per_step"], roofline=s2["roofline"],
                          stages_us=s2["stages_us"],
                          hbm_gbps_algorithmic_step=s2["hbm_gbps_algorithmic_step"],
                          hbm_frac_algorithmic_step=s2["hbm_frac_algorithmic_step"],
                          index_gather=s2["index_gather"],
                          attention=s2["attention"], ceilings=s2["ceilings"],
                          value_cache_flushed=s2["cold"],
                          per_step_cache=r2["cache"])
        del r2
        torch.cuda.empty_cache()
    variants = {}
    if args.top_p > 0:
        r3 = run_gpu(args, args.workload, args.steps, args.warmup, not args.no_stage_events,
                     top_p=args.top_p, wl=res["wl"])
        s3 = summarize(r3, args.workload)
        variants["top_p"] = dict(
            policy=f"deterministic stratum = min(top-k, top-p {args.top_p} prefix); "
                   "same budget m for the tail",
            value=s3["value"], unit="KV-tokens/s/layer", ms_per_step=s3["ms_per_step"],
            stages_us=s3["stages_us"], selected=s3["selected"])
        del r3
    if args.early_stop > 0:
        r5 = run_gpu(args, args.workload, args.steps, args.warmup, not args.no_stage_events,
                     wl=res["wl"], early_stop=args.early_stop)
        s5 = summarize(r5, args.workload)
        variants["early_stop"] = dict(
            policy=f"deterministic stratum visited in 64-token blocks of its order, stopping "
                   f"after the first block at which every query head's gain in exact "
                   f"attention mass is below {args.early_stop} of its mass so far; same tail "
                   "sample",
            value=s5["value"], unit="KV-tokens/s/layer", ms_per_step=s5["ms_per_step"],
            stages_us=s5["stages_us"], selected=s5["selected"])
        del r5
    if args.split_keys:
        sk = dict(policy="FASA-M layout: the scored RoPE pairs of every key in one array (the "
                         "indexer reads only it), the other dims in another; attention "
                         "reads the selected rows of both",
                  resident_bytes_per_token_head=dict(
                      whole=4 * res["wl"].d,
                      split_host=4 * res["wl"].pair_count),
                  unit="KV-tokens/s/layer")
        for keys in ("split", "split_host"):
            r6 = run_gpu(args, args.workload, args.steps if keys == "split" else 5,
                         args.warmup if keys == "split" else 1, not args.no_stage_events,
                         wl=res["wl"], keys=keys)
            s6 = summarize(r6, args.workload)
            sk[keys] = dict(value=s6["value"], ms_per_step=s6["ms_per_step"],
                            stages_us=s6["stages_us"],
                            indexer_gbps=s6["roofline"]["achieved"] if s6["roofline"] else None)
            del r6
            torch.cuda.empty_cache()
        sk["append"] = append_bench(res["wl"], args.steps, args.warmup)
        variants["split_keys"] = sk
    if args.multi > 1:
        T = args.multi
        mq = dict(queries_per_step=T,
                  policy="T query positions per sequence (the last T cache positions); a group "
                         "of g consecutive queries is scored once with its mean query; reuse: "
                         "the group's one selection serves every query within its causal "
                         "span; refine_2: every query re-ranks the group's 2 x top-k "
                         "candidates by its own score and samples the rest with its own "
                         "normaliser; group_1: one selection per query",
                  unit="query-KV-tokens/s/layer")
        wl_m = None
        for key, g, r in ((f"group_{T}", T, 0), (f"group_{T}_refine_2", T, 2), ("group_1", 1, 0)):
            r4 = run_gpu(args, args.workload, args.steps, args.warmup, not args.no_stage_events,
                         wl=wl_m, num_queries=T, query_group=g, refine=r)
            wl_m = r4["wl"]
            s4 = summarize(r4, args.workload)
            mq[key] = dict(value=T * s4["value"], ms_per_step=s4["ms_per_step"],
                           stages_us=s4["stages_us"], selected=s4["selected"])
            del r4
        del wl_m
        torch.cuda.empty_cache()
        variants["multi_query"] = mq
    cpu = None if args.no_cpu else cpu_baseline(res["wl"], args.cpu_budget)
    wl = res["wl"]
    line = {
        "metric": METRIC,
        "value": main_sum["value"],
        "unit": "KV-tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_sum["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "batch": wl.B,
                   "seq_len": wl.max_seq_len, "kv_tokens": int(res["tokens"]),
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.d,
                   "scored_pairs": wl.pair_count, "splits": "one per 4096-token chunk",
                   "parallelism": "none (one GPU)"},
        "roofline": main_sum["roofline"],
        "cpu_baseline": cpu,
        "stages_us": main_sum["stages_us"],
        "gpu_step_us": main_sum["gpu_step_us"],
        "per_step_cache": res["cache"],
        "value_cache_flushed": main_sum["cold"],
        "index_gather": main_sum["index_gather"],
        "attention": main_sum["attention"],
        "ceilings": main_sum["ceilings"],
        "hbm_gbps_algorithmic_step": main_sum["hbm_gbps_algorithmic_step"],
        "hbm_frac_algorithmic_step": main_sum["hbm_frac_algorithmic_step"],
        "gather_gbps_algorithmic": main_sum["gather_gbps_algorithmic"],
        "selected": main_sum["selected"],
        "also": also,
        "variants": variants,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

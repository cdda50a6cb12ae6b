#!/usr/bin/env python3
"""Benchmark: one decode iteration of one layer over a paged KV cache on one MI355X.

A step is the whole hot path for one layer: kv_append of each sequence's new
token into its page, then paged decode attention over every cached token
(split ranges merged by log-sum-exp).  Inputs are seeded synthetic data
already resident in HBM.  Consecutive steps rotate over ``--layers`` copies of
the cache (one per layer, as in a model), so no step finds its K/V in the
256 MB last-level cache left warm by the step before.

Prints one JSON line:
  value   = algorithmic HBM bytes of a step / wall time per step (GB/s),
  roofline.achieved = algorithmic bytes of one decode_step launch / its mean
            duration (HIP events on the launch stream around the K timed
            steps, divided by K),
  cpu_baseline = the fp64 CPU oracle on this host (append + decode, full batch).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, 8 TB/s
METRIC = "paged decode attention: KV HBM GB/s (fraction of peak) + seqs/s per layer"
CSRC = os.path.join(ROOT, "paged_kv_attention_decode_amd", "csrc")
# device sources a kernel's machine code comes from (a stored counter profile
# counts only while they are unchanged; the host-side launch structures in
# pkv_internal.h are left out)
DECODE_SRCS = ("pkv_kernels.hip", "pkv_device.h")
PREFILL_SRCS = ("pkv_prefill.hip", "pkv_device.h")
WORKLOADS = ["llama3_8b_bf16", "inflight_bf16", "long_splitkv_bf16", "fp8_kv", "inflight_fp8", "int8_kv",
             "inflight_int8", "int4_kv", "inflight_int4", "tiny_fp32", "chunked_prefill_bf16",
             "chunked_prefill_fp8"]
PREFILL_METRIC = "paged chunked prefill attention: TFLOP/s (causal pairs, algorithmic)"
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA peak
SCALED = ("fp8", "i8", "i4")    # caches of one byte or less, with per-(page, kv head) scales
ELEM_BITS = {"f32": 32, "bf16": 16, "fp8": 8, "i8": 8, "i4": 4}


def kernel_hash(srcs=DECODE_SRCS) -> str:
    h = hashlib.sha256()
    for name in srcs:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 10; 60 for the chunked-prefill workloads, whose "
                         "MFMA-bound kernel runs faster over its first ~30 ms of back-to-back steps as "
                         "the clocks rise)")
    ap.add_argument("--workload", default=None, choices=WORKLOADS,
                    help="one workload only (default: llama3_8b_bf16, plus the --also workloads nested)")
    ap.add_argument("--also", nargs="*", default=["inflight_bf16"], choices=WORKLOADS,
                    help="decode workloads measured after the default one and nested in its line")
    ap.add_argument("--layers", type=int, default=0, help="cache copies to rotate over (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    args.workload_given = args.workload is not None
    if args.workload is None:
        args.workload = "llama3_8b_bf16"
    if args.warmup is None:
        args.warmup = 60 if args.workload.startswith("chunked_prefill") else 10
    return args


def quantises_on_write(wl) -> bool:
    """One-byte cache fed with wider new rows: the step appends through
    kv_append_fp8 / kv_append_int8 (quantise on write)."""
    return wl.kv_dtype in SCALED and wl.new_dtype not in (None, wl.kv_dtype)


def decode_fn(pkv, kv_dtype):
    return {"fp8": pkv.paged_attn_decode_fp8, "i8": pkv.paged_attn_decode_int8,
            "i4": pkv.paged_attn_decode_int4}[kv_dtype]


def append_quant_fn(pkv, kv_dtype):
    return {"fp8": pkv.kv_append_fp8, "i8": pkv.kv_append_int8, "i4": pkv.kv_append_int4}[kv_dtype]


def alg_bytes(wl, seq_lens):
    """Bytes the method must move: (decode bytes, append bytes) for one step."""
    import numpy as np
    bits = ELEM_BITS[wl.kv_dtype]
    qb = 4 if wl.q_dtype == "f32" else 2
    ob = 4 if wl.out_dtype == "f32" else 2
    L = seq_lens.astype(np.int64)
    pages = (L + wl.P - 1) // wl.P
    kv = int(L.sum()) * wl.Hkv * wl.D * bits // 8 * 2
    dec = kv + wl.B * wl.Hq * wl.D * (qb + ob) + int(pages.sum()) * 4 + wl.B * 4
    if wl.kv_dtype in SCALED:
        dec += int(pages.sum()) * wl.Hkv * 4 * 2
    if quantises_on_write(wl):
        # read the bf16 rows, write fp8 rows, read and write both page scales
        app = wl.B * wl.Hkv * (2 * wl.D * 2 + 2 * wl.D * bits // 8 + 2 * 4 * 2) + wl.B * 8
    else:
        app = 2 * (wl.B * wl.Hkv * wl.D * bits // 8 * 2) + wl.B * 8
    return dec, app, kv


def copy_probe():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "ms": ms,
                      "copy_gbs_read_plus_write": 2 * n / ms / 1e6}))


class DeviceEvents:
    """HIP timing events recorded on the launch stream with a device-scope release.

    hipEventReleaseToDevice keeps the record from adding the system-scope cache
    write-back that a default event performs, which would otherwise open a gap of
    several microseconds between the kernels being timed.
    """
    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self, n):
        import ctypes
        import torch
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch already loaded
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.RELEASE_TO_DEVICE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)

    def record(self, i):
        rc = self.hip.hipEventRecord(self.ev[i], self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, i):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[2 * i], self.ev[2 * i + 1])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def cpu_share():
    """Host cores this process may use: the CPUs in its affinity mask, capped by
    the thread budget the environment sets (OMP_NUM_THREADS) when it is lower."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


def oracle_threads():
    return max(1, cpu_share())


def cpu_baseline(wl, steps, seconds):
    """The fp64 C oracle on this host: repeated full steps (append + decode)."""
    import numpy as np
    from oracle import c_oracle
    threads = oracle_threads()
    from oracle import paged
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    ks = None if wl.k_scales is None else wl.k_scales.copy()
    vs = None if wl.v_scales is None else wl.v_scales.copy()
    reps, kv_total, seqs, t0 = 0, 0, 0, time.perf_counter()
    while True:
        st = steps[reps % len(steps)]
        if quantises_on_write(wl):
            paged.append_dynamic(wl.kv_dtype, st["k_new"], st["v_new"], wl.new_dtype, wl.block_tables,
                                 st["seq_lens"], kp, vp, ks, vs, wl.P)
        else:
            c_oracle.append(st["k_new"], st["v_new"], wl.kv_dtype, wl.block_tables, st["seq_lens"], kp, vp,
                            wl.P)
        c_oracle.decode(wl.q, wl.q_dtype, kp, vp, wl.kv_dtype, wl.block_tables, st["seq_lens"], wl.Hq,
                        wl.P, wl.scale, ks, vs, nthreads=threads)
        d, a, _ = alg_bytes(wl, st["seq_lens"])
        kv_total += d + a
        seqs += wl.B
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # one decode of the first step's cache on a single thread: the oracle's own
    # scaling with threads, for context
    st = steps[0]
    t1 = time.perf_counter()
    c_oracle.decode(wl.q, wl.q_dtype, kp, vp, wl.kv_dtype, wl.block_tables, st["seq_lens"], wl.Hq, wl.P,
                    wl.scale, ks, vs, nthreads=1)
    el1 = time.perf_counter() - t1
    d1, _, _ = alg_bytes(wl, st["seq_lens"])
    return {"value": kv_total / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host_cpus_visible": len(os.sched_getaffinity(0)), "cpu_share": cpu_share(),
            "seqs_per_s_per_layer": seqs / el,
            "sample": f"full batch of {wl.B} sequences, {reps} step(s) of append + fp64 decode "
                      f"(C oracle, {threads} threads), {el:.1f} s",
            "one_thread_decode": {"value": d1 / el1 / 1e9, "unit": "GB/s", "seconds": round(el1, 2)}}


def cpu_baseline_prefill(wl, seconds):
    """The fp64 numpy oracle on this host: whole sequences (shortest cached context
    first, one per thread) until the time budget is spent; flops counted as for
    the GPU."""
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait

    import numpy as np
    from oracle import paged
    threads = oracle_threads()
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    t0 = time.perf_counter()
    paged.append_chunk(wl.k_new, wl.v_new, wl.kv_dtype, wl.cu_q, wl.block_tables, wl.seq_lens, kp, vp, wl.P)
    ctx = wl.seq_lens - wl.chunk_lens
    order = [int(b) for b in np.argsort(ctx, kind="stable")]

    def one(b):
        paged.prefill(wl.q, wl.q_dtype, wl.cu_q, kp, vp, wl.kv_dtype, wl.block_tables, wl.seq_lens, wl.Hq, wl.P,
                      wl.scale, batches=[b], k_scales=wl.k_scales, v_scales=wl.v_scales)
        L, C = int(wl.seq_lens[b]), int(wl.chunk_lens[b])
        return 4 * wl.Hq * wl.D * (C * (L - C + 1) + C * (C - 1) // 2)

    flops, done = 0, 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        pending = {ex.submit(one, b) for b in order[:threads]}
        nxt = threads
        while pending:
            fin, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in fin:
                flops += f.result()
                done += 1
            if time.perf_counter() - t0 < seconds:
                while nxt < len(order) and len(pending) < threads:
                    pending.add(ex.submit(one, order[nxt]))
                    nxt += 1
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_cpus_visible": len(os.sched_getaffinity(0)), "cpu_share": cpu_share(),
            "sample": f"chunk append + fp64 prefill of {done} of {wl.B} sequences (shortest cached "
                      f"context first; numpy, one sequence per thread, {threads} threads), {el:.1f} s"}


def bench_prefill(args):
    """One chunked-prefill step of one layer: kv_append_chunk of every sequence's
    chunk, then causal prefill attention of its query rows over the pages."""
    import numpy as np
    import torch
    import paged_kv_attention_decode_amd as pkv
    from workloads import configs

    wl = configs.PREFILL_CONFIGS[args.workload]()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    pool_bytes = wl.k_pool.nbytes + wl.v_pool.nbytes
    layers = args.layers or max(1, min(8, math.ceil(2.0e9 / pool_bytes)))
    q, cu, bt, sl = T(wl.q), T(wl.cu_q), T(wl.block_tables), T(wl.seq_lens)
    kn, vn = T(wl.k_new), T(wl.v_new)
    kps = [T(wl.k_pool) for _ in range(layers)]
    vps = [T(wl.v_pool) for _ in range(layers)]
    # an fp8 cache's page scales are set before the chunk lands (the append copies codes)
    ks = None if wl.k_scales is None else T(wl.k_scales)
    vs = None if wl.v_scales is None else T(wl.v_scales)
    out = torch.empty((wl.T, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def append(i):
        pkv.kv_append_chunk(kn, vn, wl.kv_dtype, cu, bt, sl, kps[i % layers], vps[i % layers], wl.Hkv, wl.D, wl.P)

    def attend(i):
        if wl.kv_dtype == "fp8":
            pkv.paged_prefill_fp8(q, wl.q_dtype, cu, kps[i % layers], vps[i % layers], ks, vs, bt, sl, wl.Hq,
                                  wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype)
        else:
            pkv.paged_prefill(q, wl.q_dtype, cu, kps[i % layers], vps[i % layers], wl.kv_dtype, bt, sl, wl.Hq,
                              wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype)

    for i in range(args.warmup):
        append(i)
        attend(i)
    evs = DeviceEvents(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs.record(0)
    for i in range(args.steps):
        append(args.warmup + i)
        attend(args.warmup + i)
    evs.record(1)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    step_ev = evs.elapsed_ms(0) / args.steps
    evs.close()
    # The prefill kernel (the dominant one) inside the same steps: K more steps,
    # an event pair around each prefill launch only, so every timed launch
    # follows its step's chunk append exactly as in the timed region.  Every
    # prefill launch of the run is of this kind, so a kernel trace of the whole
    # command averages the same launches.
    pev = DeviceEvents(args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        k = args.warmup + args.steps + i
        append(k)
        pev.record(2 * i)
        attend(k)
        pev.record(2 * i + 1)
    torch.cuda.synchronize()
    pre_all = [pev.elapsed_ms(i) for i in range(args.steps)]
    pev.close()
    pre_ms = float(np.mean(pre_all))
    flops = wl.flops()
    tfs = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (pre_ms * 1e-3) / 1e12
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"prefill_{args.workload}_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == kernel_hash(PREFILL_SRCS):
            traffic = tr.get("hbm_bytes_per_prefill_call")
    rec = {
        "metric": PREFILL_METRIC, "value": round(tfs, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 (kv) / bf16 (q, out, products)" if wl.kv_dtype == "fp8" else "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled pages)",
        "config": {"workload": args.workload, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.D, "page_size": wl.P, "chunk_tokens": int(wl.T),
                   "mean_cached_context": float(np.mean(wl.seq_lens - wl.chunk_lens)), "layers_rotated": layers,
                   "step": "kv_append_chunk of every chunk, then causal paged prefill attention"},
        "flops_per_step": int(flops), "kv_bytes_per_step": int(wl.kv_bytes()),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4), "traffic": traffic,
                     "kernel": "prefill_kernel (inside append + prefill steps)", "call_ms_mean": round(pre_ms, 5),
                     "alg_flops_per_call": int(flops)},
        "diagnostics": {"step_ms_events": round(step_ev, 5), "append_chunk_ms": round(step_ev - pre_ms, 5),
                        "prefill_ms_median_p10_p90": [round(float(np.percentile(pre_all, p)), 5)
                                                      for p in (50, 10, 90)]},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_prefill(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def read_probe_gbs(pkv, gib=4, n=10):
    """Streaming-read rate of this GPU: a 4 GiB buffer (16 times the MALL) read
    once per call with 16-byte nontemporal loads and nothing else; median of n
    timed calls (HIP events around each)."""
    import numpy as np
    import torch
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pkv.debug_read_probe(buf, sink)
    ev = DeviceEvents(n)
    torch.cuda.synchronize()
    for i in range(n):
        ev.record(2 * i)
        pkv.debug_read_probe(buf, sink)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    ms = float(np.median([ev.elapsed_ms(i) for i in range(n)]))
    ev.close()
    del buf
    return (gib << 30) / (ms * 1e-3) / 1e9


def diagnostics(pkv, wl, q, bt, kps, vps, kss, vss, dsteps, out, ws, step, i0, n=30):
    """Per-launch spread and the parts of a step, measured after the timed region.

    Each launch here is bracketed by its own event pair (whose packets add a few
    microseconds, which is why the timed region does not use them): decode_step
    median / p10 / p90, the standalone kv_append and paged decode calls, and the
    step on one cache copy reused (warm MALL) for contrast.  The append and the
    decode alone each miss what the append's stores cost the decode that reads
    the cache next; append_then_decode times the two unfused calls back to back."""
    import numpy as np
    import torch
    layers = len(kps)
    s0 = dsteps[0]

    def timed(fn):
        for i in range(3):
            fn(i)
        ev = DeviceEvents(n)
        torch.cuda.synchronize()
        for i in range(n):
            ev.record(2 * i)
            fn(i)
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        us = np.array([ev.elapsed_ms(i) * 1e3 for i in range(n)])
        ev.close()
        return us

    def app(i):
        # the timed loop's sequence of steps and cache copies, so that a
        # quantising append meets the page-scale rises (and re-encodes) it meets there
        k = i0 + i
        s, c = dsteps[k % len(dsteps)], k % layers
        if quantises_on_write(wl):
            append_quant_fn(pkv, wl.kv_dtype)(s["kn"], s["vn"], wl.new_dtype, bt, s["sl"], kps[c], vps[c],
                                              kss[c], vss[c], wl.Hkv, wl.D, wl.P)
        else:
            pkv.kv_append(s["kn"], s["vn"], wl.kv_dtype, bt, s["sl"], kps[c], vps[c], wl.Hkv, wl.D, wl.P)

    def dec_on(c, sl):
        if wl.kv_dtype in SCALED:
            decode_fn(pkv, wl.kv_dtype)(q, wl.q_dtype, kps[c], vps[c], kss[c], vss[c], bt, sl,
                                        wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype, ws,
                                        wl.partition_tokens)
        else:
            pkv.paged_attn_decode(q, wl.q_dtype, kps[c], vps[c], wl.kv_dtype, bt, sl,
                                  wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype, ws,
                                  wl.partition_tokens)

    def dec(i):
        dec_on(i % layers, s0["sl"])

    def app_dec(i):
        # the two unfused calls back to back on one step's lengths and cache copy
        k = i0 + i
        app(i)
        dec_on(k % layers, dsteps[k % len(dsteps)]["sl"])

    # Device page allocation on this batch's tables: every sequence whose newest
    # token opens a page takes one from the free stack (alloc), and one sequence
    # in 50 finishes and returns its pages (release).  Each call gets its own
    # fresh copy of the table and the stack count, made before timing.
    sl = s0["sl"]
    B, MP = bt.shape
    opens = (sl >= 1) & ((sl - 1) % wl.P == 0) & ((sl - 1) // wl.P < MP)
    rows = torch.arange(B, device=bt.device)[opens]
    cols = ((sl - 1) // wl.P).long()[opens]
    bt_open = bt.clone()
    bt_open[rows, cols] = -1
    cap = B + 64
    free_a = torch.arange(cap, dtype=torch.int32, device=bt.device)
    rel = torch.zeros(B, dtype=torch.int32, device=bt.device)
    rel[::50] = 1
    free_r = torch.empty(wl.num_pages, dtype=torch.int32, device=bt.device)
    ncopy = n + 3
    bts_a = [bt_open.clone() for _ in range(ncopy)]
    bts_r = [bt.clone() for _ in range(ncopy)]
    cnt_a = [torch.full((1,), cap, dtype=torch.int32, device=bt.device) for _ in range(ncopy)]
    cnt_r = [torch.zeros(1, dtype=torch.int32, device=bt.device) for _ in range(ncopy)]
    calls = {"a": 0, "r": 0}

    def alloc(i):
        k = calls["a"]
        calls["a"] += 1
        pkv.alloc_pages(sl, bts_a[k], wl.P, free_a, cnt_a[k])

    def release(i):
        k = calls["r"]
        calls["r"] += 1
        pkv.release_pages(rel, sl, bts_r[k], wl.P, wl.num_pages, free_r, cnt_r[k])

    st = timed(lambda i: step(i0 + i))
    ap = timed(app)
    de = timed(dec)
    ad = timed(app_dec)
    hot = timed(lambda i: step(i0 + i * layers))      # always the same cache copy
    al = timed(alloc)
    re = timed(release)
    q3 = lambda a: [round(float(np.percentile(a, p)), 2) for p in (50, 10, 90)]  # noqa: E731
    return {"note": "per-launch HIP events around each call (adds event packets); us as [median, p10, p90]",
            "decode_step_us": q3(st), "kv_append_us": q3(ap), "paged_decode_us": q3(de),
            "append_then_decode_us": q3(ad),
            "decode_step_same_cache_copy_us": q3(hot),
            "alloc_pages_us": q3(al), "release_pages_us": q3(re),
            "alloc_pages_requests": int(opens.sum().item()), "release_pages_sequences": int(rel.sum().item()),
            "seqs_per_s_append_then_decode": round(wl.B / (np.median(ad) * 1e-6), 1)}


def main():
    args = parse()
    if args.gpus != 1:
        sys.exit("bench.py measures one GPU: the decode path runs on a single MI355X and has no "
                 "multi-GPU mode (use --gpus 1)")
    if args.copy_probe:
        copy_probe()
        return
    from workloads import configs
    if args.workload in configs.PREFILL_CONFIGS:
        bench_prefill(args)
        return
    rec = bench_decode(args, args.workload)
    # The default run also measures the in-flight mixed batch (the second
    # configuration the decode is held to >= 70 % of the HBM peak on) and nests
    # its record, with its own roofline and CPU baseline, under its name.
    for name in ([] if args.workload_given else args.also):
        import torch
        torch.cuda.empty_cache()
        rec[name] = bench_decode(args, name, nested=True)
    print(json.dumps(rec), flush=True)


def bench_decode(args, name, nested=False):
    import numpy as np
    import torch
    import paged_kv_attention_decode_amd as pkv
    from workloads import configs

    gen = configs.CONFIGS[name]
    wl = gen()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    # Per-step inputs: the in-flight workload carries its own growing steps;
    # the others re-append the token at position L-1 every step (same cost).
    rng = np.random.default_rng(1234)
    if wl.steps:
        steps = [{"seq_lens": s.seq_lens, "k_new": s.k_new, "v_new": s.v_new} for s in wl.steps]
    else:
        eb_dt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "i8": np.uint8, "i4": np.uint8}[wl.kv_dtype]
        if wl.kv_dtype == "f32":
            kn = rng.standard_normal((wl.B, wl.Hkv, wl.D)).astype(np.float32)
            vn = rng.standard_normal((wl.B, wl.Hkv, wl.D)).astype(np.float32)
        else:
            from workloads import codec
            kf = rng.standard_normal((wl.B, wl.Hkv, wl.D)).astype(np.float32)
            vf = rng.standard_normal((wl.B, wl.Hkv, wl.D)).astype(np.float32)
            if wl.kv_dtype == "bf16":
                kn, vn = codec.f32_to_bf16_bits(kf), codec.f32_to_bf16_bits(vf)
            elif wl.kv_dtype == "fp8":  # bytes at a typical quantised magnitude
                kn, vn = codec.e4m3_encode(kf * 100), codec.e4m3_encode(vf * 100)
            elif wl.kv_dtype == "i8":
                kn, vn = codec.int8_encode(kf * 30), codec.int8_encode(vf * 30)
            else:                       # int4 rows, two codes per byte
                from workloads import layout
                kn = layout.pack_nibbles(codec.int4_encode(kf * 2))
                vn = layout.pack_nibbles(codec.int4_encode(vf * 2))
        steps = [{"seq_lens": wl.seq_lens.copy(), "k_new": kn.astype(eb_dt), "v_new": vn.astype(eb_dt)}]

    pool_bytes = wl.k_pool.nbytes + wl.v_pool.nbytes
    layers = args.layers or max(1, min(8, math.ceil(2.0e9 / pool_bytes)))
    q = T(wl.q)
    bt = T(wl.block_tables)
    kps = [T(wl.k_pool) for _ in range(layers)]
    vps = [T(wl.v_pool) for _ in range(layers)]
    # each cache copy has its own scales (an fp8 append may change them)
    kss = [None if wl.k_scales is None else T(wl.k_scales) for _ in range(layers)]
    vss = [None if wl.v_scales is None else T(wl.v_scales) for _ in range(layers)]
    dsteps = [{"sl": T(s["seq_lens"]), "kn": T(s["k_new"]), "vn": T(s["v_new"])} for s in steps]
    odt = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    out = torch.empty((wl.B, wl.Hq, wl.D), dtype=odt, device=dev)
    ws = torch.zeros(pkv.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    quant = quantises_on_write(wl)

    def step(i):
        """One decode iteration of one layer: append + attention in one call
        (decode_step; a quantised cache fed bf16 rows: decode_step_quant, which
        quantises them on write inside the same two kernels)."""
        s = dsteps[i % len(dsteps)]
        kp, vp, ks, vs = kps[i % layers], vps[i % layers], kss[i % layers], vss[i % layers]
        if quant:
            pkv.decode_step_quant(q, wl.q_dtype, s["kn"], s["vn"], wl.new_dtype, kp, vp, wl.kv_dtype, ks, vs, bt,
                                  s["sl"], wl.Hq, wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype, ws,
                                  partition_tokens=wl.partition_tokens)
        else:
            pkv.decode_step(q, wl.q_dtype, s["kn"], s["vn"], kp, vp, wl.kv_dtype, bt, s["sl"], wl.Hq,
                            wl.Hkv, wl.D, wl.P, wl.scale, out, wl.out_dtype, ws, k_scales=ks, v_scales=vs,
                            partition_tokens=wl.partition_tokens)

    for i in range(args.warmup):
        step(i)
    # Timed region: the K steps back to back, as a serving loop issues them.  One
    # event pair on the launch stream brackets the region (events between the
    # steps would add their own packets to the timeline); the mean launch
    # duration is the span over K.
    evs = DeviceEvents(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs.record(0)
    for i in range(args.steps):
        step(args.warmup + i)
    evs.record(1)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    dec_mean = evs.elapsed_ms(0) / args.steps
    evs.close()

    diag = diagnostics(pkv, wl, q, bt, kps, vps, kss, vss, dsteps, out, ws, step, args.warmup + args.steps)

    step_bytes, kv_bytes = 0, 0
    for i in range(args.steps):
        d, a, kvb = alg_bytes(wl, steps[(args.warmup + i) % len(steps)]["seq_lens"])
        step_bytes += d + a
        kv_bytes += kvb
    step_bytes /= args.steps
    kv_bytes /= args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = step_bytes / (dec_mean * 1e-3) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"decode_{name}_traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == kernel_hash():
            traffic = tr.get("hbm_bytes_per_decode_call")

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8e4m3 (kv) / bf16 (q, out)", "i8": "int8 (kv) / bf16 (q, out)",
                  "i4": "int4 (kv) / bf16 (q, out)", "f32": "f32"}[wl.kv_dtype],
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled pages)",
        "config": {"workload": name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.D, "page_size": wl.P,
                   "mean_seq_len": float(np.mean(steps[0]["seq_lens"])),
                   "partition_tokens": wl.partition_tokens, "layers_rotated": layers,
                   "step": ("decode_step_quant: quantising append (dynamic page scales) fused into the "
                            "paged decode (split kernel + LSE merge kernel)"
                            if quant else
                            "decode_step: kv_append fused into paged decode (split kernel + LSE merge kernel)")},
        "seqs_per_s_per_layer": round(wl.B / (ms_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": int(kv_bytes),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": ("decode_step_quant launch (decode_split_kernel + decode_merge_quant_kernel)"
                                if quant else
                                "decode_step launch (decode_split_kernel + decode_merge_kernel)"),
                     "call_ms_mean": round(dec_mean, 5), "alg_bytes_per_call": int(step_bytes)},
    }
    probe = read_probe_gbs(pkv)
    diag["read_probe_GBs"] = round(probe, 1)
    diag["frac_of_read_probe"] = round(achieved / probe, 4)
    rec["diagnostics"] = diag
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, steps, args.cpu_seconds)
    if nested:
        for k in ("n_gpus", "higher_is_better", "scaling", "vs_baseline", "data"):
            rec.pop(k, None)
    return rec


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the paged decode-attention hot path on one MI355X.

A step is one continuous-batching decode step of one attention layer over a batch that is
already resident in HBM: the cache append of every sequence's new token and paged decode
attention over all cached tokens.  By default the step is paged_attention_decode_append (the
append fused into the decode kernel), single pass per (sequence, KV head) with the work handed
out longest sequence first; --partition-size P > 0 splits the context into P-token partitions
merged by the log-sum-exp reduce; --separate times paged_cache_append followed by
paged_attention_decode instead, and --overlap paged_attention_decode_newest with the append on a
second stream.  Default workload: Llama-3-8B-shaped layer, 32 q / 8 kv heads of 128, bf16, batch 64,
context lengths ~ U[128, 2048], 16-token blocks scattered through a shuffled pool.  Also reported
in the same line: the chunked-prefill kernel (512 rows after 4,096 cached tokens) and the
long-context decode (batch 8 x 32,768 tokens, 512-token partitions).

Metric: effective KV+Q bytes per step / step time (GB/s), with KV = sum_b L_b * Hkv * D * 2 * 2 B
(each cached token's K and V once per KV head) and Q = B * Hq * D * 2 B; also seqs*steps/s.
Inputs rotate over R replicas of the caches (>= 1 GiB in total) so that the 256 MB last-level
cache cannot serve repeated reads.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload llama|long]
                    [--separate | --overlap]
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

METRIC = "paged decode attn: effective KV HBM GB/s (% of peak); seqs*steps/s"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=["llama", "long"], default="llama")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="0 = single pass; default 0 for the Llama-shaped batch, 512 for the long-context one")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for >= 1 GiB of caches")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-order", action="store_true",
                    help="do not pass the host copy of the context lengths (longest-first work order)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the chunked-prefill and long-context measurements reported beside the main line")
    ap.add_argument("--extras", default="tiny,prefill,prefill_fp8,long,prefix,fp8,mixed,trace",
                    help="comma-separated side lines to run beside the main line (default: all of them)")
    mode = ap.add_mutually_exclusive_group()
    mode.add_argument("--overlap", action="store_true",
                    help="time paged_attention_decode_newest with paged_cache_append on a second stream, each "
                         "step's decode waiting for the previous step's append")
    mode.add_argument("--separate", action="store_true",
                    help="time paged_cache_append + paged_attention_decode as two calls instead of the fused "
                         "paged_attention_decode_append")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="print the oracle CPU baseline of the workload as one JSON line and exit (no GPU use); "
                         "the bench runs it in a child process pinned to one BLAS/OpenMP thread")
    ap.add_argument("--only", choices=sorted(TRAFFIC_LINES),
                    help="counter run: measure this one line alone (llama = the main line without side lines), "
                         "end with a 1 GiB device copy for calibration, print its JSON")
    ap.add_argument("--traffic-from", nargs=3, metavar=("LINE", "FETCH_CSV", "WRITE_CSV"),
                    help="write the line's HBM traffic record from the counter_collection.csv files of two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of --only LINE, then exit")
    return ap.parse_args()


# HBM traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE) per reported line: the dispatches counted
# (kernel-name pattern), the sources that kernel is compiled from (a record counts only while their
# sha256 matches), and whether the figure is per launch (mean over the dispatches) or per replay of
# the trace (sum over them).
_DEC_SRC = ("decode.hip", "decode_part.h", "decode_host.h", "device.h")
_PRE_SRC = ("prefill_tile.h", "device.h", "fp8_device.h")
TRAFFIC_LINES = {
    "llama": (r"decode_mfma_kernel<.*, true>", _DEC_SRC, "launch"),
    "long": (r"decode_mfma_kernel<.*, true>", _DEC_SRC, "launch"),
    "tiny": (r"decode_valu_kernel<", _DEC_SRC + ("decode_valu.h",), "launch"),
    "prefill": (r"prefill_mfma_kernel<", ("prefill.hip",) + _PRE_SRC, "launch"),
    "prefill_fp8": (r"prefill_fp8_kernel<", ("prefill_fp8.hip",) + _PRE_SRC, "launch"),
    "fp8": (r"decode_fp8_kernel<.*, false>", ("fp8.hip", "decode_fp8_part.h", "fp8_device.h", "device.h"), "launch"),
    "mixed": (r"decode_group_kernel<", ("decode_group.hip", "decode_group.h") + _DEC_SRC, "launch"),
    "trace": (r"decode_(mfma|reduce)_kernel<", _DEC_SRC, "replay"),
}
# The mixed step's counter run times this one decode variant (the fastest one on record).
MIXED_COUNTED_VARIANT = "decode_grouped_2_split512"


def source_digest(line: str) -> str:
    """sha256 over the sources the counted kernel of `line` is compiled from."""
    h = hashlib.sha256()
    for name in TRAFFIC_LINES[line][1]:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_404_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def measured_traffic(line: str):
    """HBM bytes per launch (per trace replay) of the line's kernel from the committed counter
    record, when it was taken on the current kernel sources; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get(line)
    if not entry or entry.get("sources_sha256") != source_digest(line):
        return None
    return entry.get("hbm_bytes_per_launch", entry.get("hbm_bytes_per_replay"))


def write_traffic(line: str, fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes of the line's kernel from two counter runs of `bench.py --only LINE`.

    FETCH_SIZE and WRITE_SIZE are KiB per dispatch.  Each is scaled by what the same counter
    reads for the 1 GiB device-to-device copy every such run ends with (known bytes: 1 GiB read
    and 1 GiB written), so the figure is in true bytes whatever the counter's granularity."""
    import csv
    import re

    pattern, _, per = TRAFFIC_LINES[line]

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        sel = [r for r in rows if re.search(pattern, r["Kernel_Name"])]
        names = {r["Kernel_Name"] for r in sel}
        if not sel or (per == "launch" and len(names) != 1):
            raise SystemExit(f"{path}: need dispatches of exactly one kernel matching {pattern!r}, found {names}")
        vals = [float(r["Counter_Value"]) for r in sel]
        return copy, (sum(vals) / len(vals) if per == "launch" else sum(vals)), len(vals), sorted(names)

    f_copy, f_k, n_f, names = per_kernel(fetch_csv, "FETCH_SIZE")
    w_copy, w_k, n_w, _ = per_kernel(write_csv, "WRITE_SIZE")
    known = float(1 << 30)
    f_scale, w_scale = known / (f_copy * 1024), known / (w_copy * 1024)
    hbm = f_k * 1024 * f_scale + w_k * 1024 * w_scale
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        rec = {}
    unit = "per_dispatch" if per == "launch" else "per_replay"
    rec[line] = {
        "kernels": names,
        "sources_sha256": source_digest(line),
        f"hbm_bytes_per_{per}": round(hbm),
        f"fetch_kib_{unit}": round(f_k, 1),
        f"write_kib_{unit}": round(w_k, 1),
        "dispatches": [n_f, n_w],
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "calibration": "1 GiB device-to-device copy (__amd_rocclr_copyBuffer) in the same run: "
                       f"FETCH_SIZE {f_copy:.1f} KiB, WRITE_SIZE {w_copy:.1f} KiB",
        "counter_runs": f"rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE -- python3 bench.py --only {line} --steps 5 "
                        "--warmup 2",
    }
    if line == "mixed":
        rec[line]["variant"] = MIXED_COUNTED_VARIANT
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec[line]


def _traffic_fields(line: str, algorithmic_bytes: int) -> dict:
    """`traffic` (HBM bytes per launch from the line's counter record, None when the kernel changed
    since) and its ratio to the launch's algorithmic bytes."""
    t = measured_traffic(line)
    return {"traffic": t, "algorithmic_bytes": algorithmic_bytes,
            "traffic_over_algorithmic": round(t / algorithmic_bytes, 4) if t else None}


def _prefill_bytes(ctx: int, C: int, Hq: int, Hkv: int, D: int, fp8: bool) -> int:
    """Bytes a prefill chunk must move at least: the K/V of its ctx + C visible tokens once (fp8:
    codes + fp32 K and V scales per slot), the queries in, the fp32 outputs out."""
    T = ctx + C
    kv = T * Hkv * (2 * D + 8) if fp8 else T * Hkv * D * 2 * 2
    return kv + C * Hq * D * 2 + C * Hq * D * 4


def calibration_copy(dev) -> None:
    """One 1 GiB device-to-device copy: the known-size kernel the counter records are scaled by."""
    import torch

    src = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def _events_avg_us(torch, stream, fn, n):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def measure_prefill(args, dev, fp8=False):
    """paged_attention_prefill_chunk on the mixed step's chunk: 512 rows at positions 4096..4607
    of one sequence (32 q / 8 kv heads of 128, bf16), causal against the paged cache; with fp8,
    paged_attention_prefill_chunk_fp8 over the same tokens quantised into an fp8 cache (bf16
    queries).  Work: 4 * head_dim flops per visible (row, key) pair and query head."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    w = wl.mixed_step(5)
    ctx, C, Hq, Hkv, D = w.ctx_start, w.chunk, w.Hq, w.Hkv, w.D
    pool = BlockPool(w.num_blocks, 16, w.free_order)
    s = pool.new_seq()
    pool.append(s, ctx + C)
    table, _ = pool.block_tables([s], wl.blocks_for(ctx + C))
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    tb = torch.from_numpy(table[0]).to(dev)
    # Replicas of the whole input (caches, queries, output) rotated call by call, at least 1 GiB
    # in all, so that no call finds the previous one's K/V in the last-level cache.
    per_rep = 2 * w.num_blocks * Hkv * 16 * (D + 4 if fp8 else 2 * D) + C * Hq * D * 6
    R = max(1, math.ceil((1 << 30) / per_rep))
    T = ctx + C
    slots = torch.from_numpy((table[0][np.arange(T) // 16].astype(np.int64) * 16 + np.arange(T) % 16)
                             .astype(np.int32)).to(dev)
    calls = []
    for r in range(R):
        q = torch.randn((C, Hq, D), generator=g, device=dev).to(torch.bfloat16)
        out = torch.empty((C, Hq, D), dtype=torch.float32, device=dev)
        if fp8:
            k, v, ks, vs = ops.fp8_cache(w.num_blocks, Hkv, D, device=dev)
            kr = torch.randn((T, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            vr = torch.randn((T, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
            ops.paged_cache_append_fp8(k, v, ks, vs, kr, vr, slots)
            del kr, vr
            calls.append(lambda out=out, q=q, k=k, v=v, ks=ks, vs=vs:
                         ops.paged_attention_prefill_chunk_fp8(out, q, k, v, ks, vs, tb, ctx, w.scale))
        else:
            k = torch.randn((w.num_blocks, Hkv, 16 * D), generator=g, device=dev).to(torch.bfloat16)
            v = torch.randn((w.num_blocks, Hkv, 16 * D), generator=g, device=dev).to(torch.bfloat16)
            calls.append(lambda out=out, q=q, k=k, v=v: ops.paged_attention_prefill_chunk(out, q, k, v, tb, ctx,
                                                                                            w.scale))
    fn = lambda i: calls[i % R]()  # noqa: E731
    for i in range(5):
        fn(i)
    us = _events_avg_us(torch, torch.cuda.current_stream(), fn, max(20, args.steps // 4))
    pairs = sum(ctx + i + 1 for i in range(C))
    flops = pairs * Hq * 4 * D
    tflops = flops / (us * 1e-6) / 1e12
    res = {
        "workload": f"prefill_chunk_{C}_after_{ctx}_gqa{Hq}x{Hkv}_d{D}_" + ("fp8_cache_bf16_query" if fp8 else "bf16"),
        "us_per_call": round(us, 3),
        "flops_per_call": flops,
        "replicas": R,
        "roofline": {"bound": "mfma", "kernel": "prefill_fp8_kernel" if fp8 else "prefill_mfma_kernel",
                     "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     **_traffic_fields("prefill_fp8" if fp8 else "prefill", _prefill_bytes(ctx, C, Hq, Hkv, D, fp8))},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(ctx, Hq, Hkv, D, w.scale, args.cpu_seconds / 2, fp8=fp8)
    return res


def cpu_baseline_prefill(ctx, Hq, Hkv, D, scale, seconds, fp8=False):
    """The oracle's prefill (numpy fp64) on the first R rows of the same chunk shape, R grown
    until the sample takes about `seconds` (fp8: over the oracle's quantised cache)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import CacheModel, Fp8CacheModel, PoolModel
    from oracle import attention as oatt

    rng = np.random.default_rng(1005)
    R = 4
    while True:
        N = wl.blocks_for(ctx + R) + 1
        pool = PoolModel(N, 16, rng.permutation(N))
        sq = pool.new_seq()
        slots, _ = pool.append(sq, ctx + R)
        kb, vb = wl.normal_bits(rng, (ctx + R, Hkv, D), "bf16"), wl.normal_bits(rng, (ctx + R, Hkv, D), "bf16")
        if fp8:
            cache = Fp8CacheModel(N, Hkv, D)
            cache.append(oatt.bits_to_f64(kb, "bf16").astype(np.float32),
                         oatt.bits_to_f64(vb, "bf16").astype(np.float32), slots)
        else:
            cache = CacheModel(N, Hkv, D, "bf16", fill_nan=True)
            cache.append(kb, vb, slots)
        q = wl.normal_bits(rng, (R, Hq, D), "bf16")
        table, _ = pool.block_tables([sq], len(pool.tables[sq]))
        t0 = time.perf_counter()
        oatt.prefill_chunk(q, cache, table[0], ctx, scale, q_dtype="bf16")
        el = time.perf_counter() - t0
        if el >= seconds or R >= 512:
            break
        R = min(512, max(R * 2, int(R * seconds / max(el, 1e-3))))
    flops = sum(ctx + i + 1 for i in range(R)) * Hq * 4 * D
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {R} of 512 chunk rows after {ctx} cached tokens" + (" (fp8 cache)" if fp8 else "") +
                      f", numpy fp64, {el:.1f} s"}


def trace_partition_size(B: int, Hkv: int, max_len: int) -> int:
    """Partition size of one trace step: 512-token partitions + reduce (fixed positions, so batch
    invariant).  Measured on this trace against single pass (40 % of peak), 1024 and 2048 (55 %),
    and single pass only while the batch fills the chip (55 %)."""
    return 512


def measure_trace(dev, choose_ps=trace_partition_size, counters=False):
    """The continuous-batching trace: 512 seeded requests (Poisson arrivals, lognormal prompts
    around 512 tokens, geometric outputs around 200), at most 128 running, a 12,288-block pool,
    32 q / 8 kv heads of 128, bf16.

    Host phase: the library's pool retires finished requests, admits waiting ones first come first
    served while the pool holds their tokens plus one, and appends one token per running request
    (preempting the newest on out-of-blocks); the builders give the step's tables and lengths.
    Its wall time is the host time.  Device phase: every step's arrays are uploaded once, then the
    steps replay back to back: the admitted prompts' K/V (paged_cache_append), then the fused
    append + decode over the live batch.  Behind a bounded spin the host enqueues the whole replay
    ahead of the GPU, so one event pair around it times device work only; the decode calls alone
    and the prompt appends alone are replayed the same way for their own times.

    counters: a counter run; the decode calls of one replay run once (nothing else of the trace
    on the GPU), so the counter record sums the HBM traffic of exactly one replay's decode."""
    import collections

    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    seed, N, n_req, max_active = 3, 12288, 512, 128
    Hq, Hkv, D = 32, 8, 128
    reqs = wl.trace_requests(seed, n=n_req)
    pool = BlockPool(N, 16, wl.shuffled_free_order(seed, N))
    waiting = collections.deque(range(n_req))
    running, seq_of, generated = [], {}, [0] * n_req
    steps, util = [], []
    preempted, step = 0, 0
    t0 = time.perf_counter()
    while waiting or running:
        for r in [r for r in running if generated[r] >= reqs[r].output_len]:
            pool.free(seq_of.pop(r))
            running.remove(r)
        admitted = []
        while waiting and len(running) < max_active and reqs[waiting[0]].arrival_step <= step:
            r = waiting[0]
            ntok = reqs[r].prompt_len + generated[r]
            if pool.num_free() < wl.blocks_for(ntok + 1):
                break
            waiting.popleft()
            s = pool.new_seq()
            slots, _ = pool.append(s, ntok)
            admitted.append(slots)
            seq_of[r] = s
            running.append(r)
        if not running:
            step += 1
            continue
        pending = list(running)
        while pending:
            status, done, _, _ = pool.append_many([seq_of[r] for r in pending], [1] * len(pending))
            if status == 0:
                break
            victim = running.pop()  # the newest request gives its blocks back and waits again
            pool.free(seq_of.pop(victim))
            waiting.appendleft(victim)
            preempted += 1
            pending = [r for r in pending[done:] if r != victim]
        for r in running:
            generated[r] += 1
        seqs = [seq_of[r] for r in running]
        nblk = [pool.seq_num_blocks(s) for s in seqs]
        tables, lens = pool.block_tables(seqs, max(nblk))
        util.append(int(lens.sum()) / (16.0 * sum(nblk)))
        steps.append((tables, lens, np.concatenate(admitted).astype(np.int32) if admitted else None))
        step += 1
    host_s = time.perf_counter() - t0

    adm = [a for _, _, a in steps if a is not None]
    max_adm = max((len(a) for a in adm), default=1)
    flat_tab = torch.from_numpy(np.concatenate([t.ravel() for t, _, _ in steps])).to(dev)
    flat_len = torch.from_numpy(np.concatenate([ln for _, ln, _ in steps])).to(dev)
    flat_adm = torch.from_numpy(np.concatenate(adm)).to(dev) if adm else None
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    bf = torch.bfloat16
    kc = torch.randn((N, Hkv, 16 * D), generator=g, device=dev).to(bf)
    vc = torch.randn((N, Hkv, 16 * D), generator=g, device=dev).to(bf)
    src_k = torch.randn((max_adm, Hkv, D), generator=g, device=dev).to(bf)
    src_v = torch.randn((max_adm, Hkv, D), generator=g, device=dev).to(bf)
    q = torch.randn((max_active, Hq, D), generator=g, device=dev).to(bf)
    nk = torch.randn((max_active, Hkv, D), generator=g, device=dev).to(bf)
    nv = torch.randn((max_active, Hkv, D), generator=g, device=dev).to(bf)
    out = torch.empty((max_active, Hq, D), dtype=torch.float32, device=dev)
    max_ctx = max(int(ln.max()) for _, ln, _ in steps)
    step_ps = [choose_ps(len(ln), Hkv, int(ln.max())) for _, ln, _ in steps]
    ws_bytes = max(ops.decode_workspace_bytes(len(ln), Hq, D, int(ln.max()), ps) for (_, ln, _), ps in zip(steps, step_ps))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    calls = []
    to = lo = ao = 0
    kv_bytes = 0
    for (tables, lens, a), ps in zip(steps, step_ps):
        B, mb = tables.shape
        app = None
        if a is not None:
            app = ops.PreparedAppend(kc, vc, src_k[:len(a)], src_v[:len(a)], flat_adm[ao:ao + len(a)])
            ao += len(a)
        dec = ops.PreparedDecode(out[:B], q[:B], kc, vc, flat_tab[to:to + B * mb].view(B, mb), flat_len[lo:lo + B],
                                 int(lens.max()), scale, ps, ws, new_key=nk[:B], new_value=nv[:B],
                                 host_context_lens=lens)
        to += B * mb
        lo += B
        kv_bytes += int(lens.sum()) * Hkv * 2 * D * 2 + B * Hq * D * 2
        calls.append((app, dec))
    stream = torch.cuda.current_stream()
    if counters:
        for _, dec in calls:
            dec()
        torch.cuda.synchronize()
        return {"counted": "the decode calls of one replay", "steps": len(steps), "decode_kv_plus_q_bytes": kv_bytes}
    for app, dec in calls[:20]:  # warm-up (loads the kernels)
        if app is not None:
            app()
        dec()
    torch.cuda.synchronize()
    # A bounded spin kernel first, so that the host enqueues the replay ahead of the GPU and the
    # events time the device work alone (no launch gaps inside a step).
    probe = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    probe[0].record(stream)
    torch.cuda._sleep(1 << 20)
    probe[1].record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(probe[0].elapsed_time(probe[1]), 1e-3)
    seg, spin_ms = 200, 200.0
    spin = int(cycles_per_ms * spin_ms)

    def replay(run_app: bool, run_dec: bool):
        """The steps back to back in segments of `seg` steps, each behind its own spin with one
        event pair around it (events between launches would serialise them and add their own cost
        to every step).  A segment's launches fit the hardware queue, so the host enqueues all of
        them while the GPU spins, and the events time device work alone; the replay's time is the
        sum over its segments.  Returns (GPU ms, the longest segment enqueue in ms)."""
        gpu_ms, enq_ms = 0.0, 0.0
        for s0 in range(0, len(calls), seg):
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            torch.cuda._sleep(spin)
            w0 = time.perf_counter()
            ev[0].record(stream)
            for app, dec in calls[s0:s0 + seg]:
                if run_app and app is not None:
                    app()
                if run_dec:
                    dec()
            ev[1].record(stream)
            enq_ms = max(enq_ms, (time.perf_counter() - w0) * 1e3)
            torch.cuda.synchronize()
            gpu_ms += ev[0].elapsed_time(ev[1])
        return gpu_ms, enq_ms

    total_ms, enqueue_ms = replay(True, True)
    dec_ms, enq_dec = replay(False, True)
    adm_ms, enq_adm = replay(True, False)
    enqueue_ms = max(enqueue_ms, enq_dec, enq_adm)
    dec_us, adm_us = dec_ms * 1e3, adm_ms * 1e3
    seq_steps = sum(len(ln) for _, ln, _ in steps)
    gbs = kv_bytes / (dec_us * 1e-6) / 1e9
    return {
        "workload": f"trace_{n_req}_requests_max{max_active}_pool{N}_gqa{Hq}x{Hkv}_d{D}_bf16",
        "steps": len(steps),
        "seq_steps": seq_steps,
        "max_running": max(len(ln) for _, ln, _ in steps),
        "max_context": max_ctx,
        "preemptions": preempted,
        "prompt_tokens_appended": int(sum(len(a) for a in adm)),
        "decode_call": "paged_attention_decode_append, 512-token partitions + reduce",
        "gpu_ms": {"decode_steps": round(dec_us / 1e3, 3), "prompt_appends": round(adm_us / 1e3, 3)},
        "decode_kv_plus_q_bytes": kv_bytes,
        "decode_gbs": round(gbs, 1),
        "decode_pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "decode_mfma_kernel + decode_reduce_kernel, every decode call of "
                     "one replay (traffic and algorithmic bytes per replay)", "achieved": round(gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     **_traffic_fields("trace", kv_bytes)},
        "seqs_steps_per_s_gpu": round(seq_steps / (total_ms * 1e-3), 1),
        "timing": f"three replays, each in segments of {seg} back-to-back steps behind a {spin_ms:.0f} ms spin "
                  "with one event pair per segment, summed: the whole interleaved replay "
                  "(seqs_steps_per_s_gpu, replay_gpu_ms), its decode calls alone (decode_steps, decode_gbs) "
                  "and its prompt appends alone (prompt_appends)",
        "host_us_per_step": round(host_s / len(steps) * 1e6, 1),
        "host_note": "pool, scheduler and builders through the Python binding, measured apart from the GPU replay",
        "pool_utilisation": {"mean": round(float(np.mean(util)), 5), "min": round(float(np.min(util)), 5)},
        "replay_gpu_ms": round(total_ms, 3),
        "segment_enqueue_ms_max": round(enqueue_ms, 2),
        # Each segment's spin covers its enqueue, so no step waited for the host (events time the GPU only).
        "enqueue_within_spin": bool(enqueue_ms < spin_ms),
        # lengths of the step with the median batch, for the oracle's sampled baseline (popped by main)
        "_median_step_lens": sorted((ln for _, ln, _ in steps), key=len)[len(steps) // 2].tolist(),
    }


def measure_prefix_cache():
    """Host prefix cache on a long-context-sized pool (18,023 blocks): register a 2,048-token
    prompt (128 blocks), then time lookups of that prompt plus 64 new tokens (128 trie probes, 128
    new references) each followed by freeing the new sequence, and re-registration (128 probes)."""
    import numpy as np

    from paged_kv_cache_404_amd import BlockPool
    rng = np.random.default_rng(9)
    N = 18023
    pool = BlockPool(N, 16, rng.permutation(N))
    prompt = rng.integers(0, 128000, 2048).astype(np.int32)
    s = pool.new_seq()
    pool.append(s, 2048)
    assert pool.prefix_insert(s, prompt) == 128
    req = np.concatenate([prompt, rng.integers(0, 128000, 64).astype(np.int32)])
    n_iter = 2000
    t0 = time.perf_counter()
    for _ in range(n_iter):
        q, n = pool.prefix_lookup(req)
        pool.free(q)
    lookup_us = (time.perf_counter() - t0) / n_iter * 1e6
    assert n == 2048
    t0 = time.perf_counter()
    for _ in range(n_iter):
        pool.prefix_insert(s, prompt)
    insert_us = (time.perf_counter() - t0) / n_iter * 1e6
    return {"workload": "prefix_cache_lookup_2048_tokens_pool_18023", "lookup_and_free_us": round(lookup_us, 2),
            "reinsert_us": round(insert_us, 2), "matched_tokens": int(n), "blocks_per_lookup": 128,
            "note": "host time per call through the Python binding (ctypes call overhead included)",
            "roofline": None,
            "roofline_note": "host code only (a trie walk over 128 block hashes): no device kernel, no HBM roofline",
            "cpu_baseline": cpu_baseline_prefix(prompt, req)}


def cpu_baseline_prefix(prompt, req):
    """The oracle pool's prefix cache on the same request: register the 2,048-token prompt, then
    time lookups of the prompt plus 64 new tokens, each followed by freeing the new sequence."""
    import numpy as np

    from oracle import PoolModel

    N = 18023
    pool = PoolModel(N, 16, np.random.default_rng(9).permutation(N))
    s = pool.new_seq()
    pool.append(s, 2048)
    pool.prefix_insert(s, [int(t) for t in prompt])
    toks = [int(t) for t in req]
    reps, t0 = 0, time.perf_counter()
    while True:
        q, n = pool.prefix_lookup(toks)
        pool.free_seq(q)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 1.0 and reps >= 10:
            break
    return {"value": round(el / reps * 1e6, 2), "unit": "us per lookup and free", "cores": 1, "kind": "oracle",
            "matched_tokens": int(n), "sample": f"{reps} lookups of the same request, pure Python, {el:.1f} s"}


def measure_fp8(args, dev, bf16_kernel_us):
    """The batch-64 Llama-shaped decode over an FP8 (E4M3) cache: the lengths and block scatter of
    the main line, the cache filled by the quantising append.  A step = paged_attention_decode_append_fp8
    (every sequence's new token quantised into its slot inside the single-pass decode, longest
    first); the fp8 append + decode as two launches is reported beside it.  Algorithmic bytes per step: the
    1-byte K and V codes of every cached token per KV head, their fp32 scales, and Q.  Also the
    format's own error: the same K/V in a bf16 cache against the fp8 cache, same queries."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    w = wl.llama_decode(2)
    pool = BlockPool(w.num_blocks, 16, w.free_order)
    seqs = [pool.new_seq() for _ in range(w.B)]
    st, _, pre_slots, _ = pool.append_many(seqs, [int(L) - 1 for L in w.lens])
    st2, _, step_slots, _ = pool.append_many(seqs, [1] * w.B)
    assert st == 0 and st2 == 0
    tables, lens = pool.block_tables(seqs, w.max_blocks_per_seq)
    tables_t, lens_t = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    pre_t, step_t = torch.from_numpy(pre_slots).to(dev), torch.from_numpy(step_slots).to(dev)
    maxL = int(lens.max())
    per_rep = 2 * w.num_blocks * w.Hkv * 16 * (w.D + 4)
    R = max(1, math.ceil((1 << 30) / per_rep))
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 100)
    T = int(pre_slots.size)
    reps, err = [], None
    for r in range(R):
        k, v, ks, vs = ops.fp8_cache(w.num_blocks, w.Hkv, w.D, device=dev)
        kb = torch.randn((T, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
        vb = torch.randn((T, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
        ops.paged_cache_append_fp8(k, v, ks, vs, kb, vb, pre_t)
        q = torch.randn((w.B, w.Hq, w.D), generator=g, device=dev).to(torch.bfloat16)
        sk = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
        sv = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
        out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
        ws = ops.decode_workspace(w.B, w.Hq, w.D, maxL, 0, device=dev)
        if r == 0:  # the same K/V through a bf16 cache: the format's own error on this batch
            k16 = torch.empty((w.num_blocks, w.Hkv, 16 * w.D), dtype=torch.bfloat16, device=dev)
            v16 = torch.empty((w.num_blocks, w.Hkv, 16 * w.D), dtype=torch.bfloat16, device=dev)
            ops.paged_cache_append(k16, v16, kb, vb, pre_t)
            ops.paged_cache_append(k16, v16, sk, sv, step_t)
            ops.paged_cache_append_fp8(k, v, ks, vs, sk, sv, step_t)
            o16 = torch.empty_like(out)
            ops.paged_attention_decode(o16, q, k16, v16, tables_t, lens_t, maxL, w.scale, 0, ws)
            ops.paged_attention_decode_fp8(out, q, k, v, ks, vs, tables_t, lens_t, maxL, w.scale, 0, ws)
            torch.cuda.synchronize()
            d = (out - o16).abs()
            err = {"max_abs": round(float(d.max()), 5), "mean_abs": round(float(d.mean()), 6),
                   "output_rms": round(float(o16.pow(2).mean().sqrt()), 5)}
            del k16, v16, o16
        del kb, vb
        reps.append((ops.PreparedAppendFp8(k, v, ks, vs, sk, sv, step_t),
                     ops.PreparedDecodeFp8(out, q, k, v, ks, vs, tables_t, lens_t, maxL, w.scale, 0, ws,
                                           host_context_lens=lens),
                     ops.PreparedDecodeFp8(out, q, k, v, ks, vs, tables_t, lens_t, maxL, w.scale, 0, ws,
                                           host_context_lens=lens, new_key=sk, new_value=sv)))
    stream = torch.cuda.current_stream()

    def events(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def separate(i):
        app, dec, _ = reps[i % R]
        app()
        dec.partitions()

    for i in range(args.warmup):
        separate(i)
        reps[i % R][2]()
    step_us = events(lambda i: reps[i % R][2](), args.steps)
    sep_us = events(separate, args.steps)
    kern_us = events(lambda i: reps[i % R][1].partitions(), args.steps)
    app_us = events(lambda i: reps[i % R][0](), args.steps)
    total_tokens = int(lens.sum())
    nbytes = total_tokens * w.Hkv * w.D * 2 + total_tokens * w.Hkv * 2 * 4 + w.B * w.Hq * w.D * 2
    achieved = nbytes / (kern_us * 1e-6) / 1e9
    return {
        "workload": w.name + "_fp8_e4m3_cache",
        "kv_codes_scales_q_bytes_per_step": nbytes,
        "us_per_step": round(step_us, 3),
        "gbs_per_step": round(nbytes / (step_us * 1e-6) / 1e9, 1),
        "seqs_steps_per_s": round(w.B / (step_us * 1e-6), 1),
        "step": "paged_attention_decode_append_fp8 (quantising append fused into the decode kernel), single pass",
        "separate_launches_us_per_step": round(sep_us, 3),
        "kernel_us": {"append_fp8": round(app_us, 3), "decode_fp8": round(kern_us, 3),
                      "decode_fp8_fused_append": round(step_us, 3)},
        "decode_speedup_over_bf16_cache": round(bf16_kernel_us / kern_us, 3) if bf16_kernel_us else None,
        "roofline": {"bound": "hbm", "kernel": "decode_fp8_kernel (decode alone, no append)", "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     **_traffic_fields("fp8", nbytes)},
        "format_error_vs_bf16_cache": err,
        "replicas": R,
        **({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_fp8(w, args.cpu_seconds / 2)}),
    }


def cpu_baseline_fp8(w, seconds: float, max_seqs: int = 8):
    """The oracle over its FP8 cache model (codes times per-slot scales, fp64 attention) on the first
    S = min(B, max_seqs) sequences of the batch, bf16 queries; bytes counted as on the GPU line."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import Fp8CacheModel, PoolModel
    from oracle import attention as oatt

    S = min(w.B, max_seqs)
    lens = w.lens[:S]
    rng = np.random.default_rng(1002)
    N = sum(wl.blocks_for(int(L)) for L in lens) + 1
    pool = PoolModel(N, 16, rng.permutation(N))
    cache = Fp8CacheModel(N, w.Hkv, w.D)
    seqs = []
    for L in lens:
        s = pool.new_seq()
        slots, _ = pool.append(s, int(L))
        cache.append(rng.standard_normal((int(L), w.Hkv, w.D)).astype(np.float32),
                     rng.standard_normal((int(L), w.Hkv, w.D)).astype(np.float32), slots)
        seqs.append(s)
    q = wl.normal_bits(rng, (S, w.Hq, w.D), "bf16")
    tables, tl = pool.block_tables(seqs, max(len(pool.tables[s]) for s in seqs))
    tok = int(np.sum(lens.astype(np.int64)))
    sample_bytes = tok * w.Hkv * w.D * 2 + tok * w.Hkv * 2 * 4 + S * w.Hq * w.D * 2
    reps, t0 = 0, time.perf_counter()
    while True:
        oatt.paged_decode(q, cache, tables, tl, w.scale, q_dtype="bf16")
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds and reps >= 3:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    per = el / reps
    return {"value": round(sample_bytes / per / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "seqs_steps_per_s": round(S / per, 3),
            "sample": f"{S} of {w.B} sequences ({tok} cached tokens, {sample_bytes} B of codes, scales and Q), "
                      f"numpy fp64 over dequantised codes, {reps} calls in {el:.1f} s"}


def _spin_cycles_per_ms(torch, stream):
    """Cycles of torch.cuda._sleep per millisecond on this device (for spins that hide enqueue time)."""
    probe = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    probe[0].record(stream)
    torch.cuda._sleep(1 << 20)
    probe[1].record(stream)
    torch.cuda.synchronize()
    return (1 << 20) / max(probe[0].elapsed_time(probe[1]), 1e-3)


def _spun_avg_us(torch, stream, fn, n, spin_cycles):
    """Average device time of fn(i), i < n, run back to back behind a bounded spin kernel: the host
    enqueues all n calls while the spin runs, so the one event pair after the spin times GPU work
    only (calls whose enqueue takes longer than their kernels would otherwise time the host)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(spin_cycles)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def _mixed_case(args, dev, prefix_len, n, spin, counted=False):
    """One prefix-sharing step: 16 samples forked from a prefix_len-token prefix decode one token
    each, a 512-row chunk is prefilled after 4,096 cached tokens.  Times (HIP events behind a spin)
    the decode alone (plain single pass, grouped 2 and 4 samples per workgroup), the prefill alone,
    both as separate launches and as one mixed launch (plain and grouped), and the step = the
    copy-on-write block copies (if any) + the append of its 16 + 512 tokens + attention.  counted:
    only n calls of the decode variant the counter record covers (a counter run)."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    mw = wl.mixed_step(5, prefix_len=prefix_len)
    pool = BlockPool(mw.num_blocks, 16, mw.free_order)
    s0 = pool.new_seq()
    pool.append(s0, mw.prefix_len)
    samples = [s0] + [pool.fork(s0) for _ in range(mw.samples - 1)]
    pf = pool.new_seq()
    pool.append(pf, mw.ctx_start)
    st, _, step_slots, cow = pool.append_many(samples + [pf], [1] * mw.samples + [mw.chunk])
    assert st == 0
    dtab, dlens = pool.block_tables(samples, wl.blocks_for(mw.prefix_len + 1))
    ptab, _ = pool.block_tables([pf], wl.blocks_for(mw.ctx_start + mw.chunk))
    cache_bytes = 2 * mw.num_blocks * mw.Hkv * 16 * mw.D * 2
    R = max(1, math.ceil((1 << 30) / cache_bytes))
    g = torch.Generator(device=dev)
    g.manual_seed(55)
    tdt = torch.bfloat16
    dt_t, dl_t = torch.from_numpy(dtab).to(dev), torch.from_numpy(dlens).to(dev)
    pt_t = torch.from_numpy(ptab).to(dev)
    slots_t = torch.from_numpy(step_slots).to(dev)
    cow_t = torch.from_numpy(np.ascontiguousarray(cow, dtype=np.int32).reshape(-1, 2)).to(dev)
    T = mw.samples + mw.chunk
    mcl = int(dlens.max())
    reps = []
    for r in range(R):
        k = torch.randn((mw.num_blocks, mw.Hkv, 16 * mw.D), generator=g, device=dev).to(tdt)
        v = torch.randn((mw.num_blocks, mw.Hkv, 16 * mw.D), generator=g, device=dev).to(tdt)
        sk = torch.randn((T, mw.Hkv, mw.D), generator=g, device=dev).to(tdt)
        sv = torch.randn((T, mw.Hkv, mw.D), generator=g, device=dev).to(tdt)
        qd = torch.randn((mw.samples, mw.Hq, mw.D), generator=g, device=dev).to(tdt)
        qp = torch.randn((mw.chunk, mw.Hq, mw.D), generator=g, device=dev).to(tdt)
        od = torch.empty((mw.samples, mw.Hq, mw.D), dtype=torch.float32, device=dev)
        op = torch.empty((mw.chunk, mw.Hq, mw.D), dtype=torch.float32, device=dev)
        ws = ops.decode_workspace(mw.samples, mw.Hq, mw.D, mcl, 512)
        mix_args = (od, qd, dt_t, dl_t, mcl, op, qp, pt_t, [mw.ctx_start], [mw.chunk], k, v, mw.scale)
        reps.append({
            "copy": (lambda k=k, v=v: ops.paged_cache_copy_blocks(k, v, cow_t)) if len(cow) else (lambda: None),
            "append": ops.PreparedAppend(k, v, sk, sv, slots_t),
            "dec": ops.PreparedDecode(od, qd, k, v, dt_t, dl_t, mcl, mw.scale, 0, None, host_context_lens=dlens),
            "dec_p512": ops.PreparedDecode(od, qd, k, v, dt_t, dl_t, mcl, mw.scale, 512, ws, host_context_lens=dlens),
            "dec_g2": ops.PreparedDecode(od, qd, k, v, dt_t, dl_t, mcl, mw.scale, 0, None, group_size=2),
            "dec_g4": ops.PreparedDecode(od, qd, k, v, dt_t, dl_t, mcl, mw.scale, 0, None, group_size=4),
            "dec_g2_p512": ops.PreparedDecode(od, qd, k, v, dt_t, dl_t, mcl, mw.scale, 512, ws, group_size=2),
            "pre": ops.PreparedPrefill(op, qp, k, v, pt_t[0], mw.ctx_start, mw.scale),
            "mix": ops.PreparedMixed(*mix_args, host_dec_lens=dlens),
            "mix_g2_p512": ops.PreparedMixed(*mix_args, dec_group_size=2, dec_partition_size=512, workspace=ws),
        })
    stream = torch.cuda.current_stream()

    def run(*names):
        def fn(i):
            r = reps[i % R]
            for nm in names:
                r[nm]()
        return fn

    variants = {
        "decode": ("dec",), "decode_split512": ("dec_p512",), "decode_grouped_2": ("dec_g2",),
        "decode_grouped_4": ("dec_g4",), "decode_grouped_2_split512": ("dec_g2_p512",),
        "prefill": ("pre",), "separate": ("dec", "pre"), "separate_grouped": ("dec_g2_p512", "pre"),
        "mixed": ("mix",), "mixed_grouped": ("mix_g2_p512",),
        "step_separate": ("copy", "append", "dec", "pre"), "step_mixed": ("copy", "append", "mix"),
        "step_mixed_grouped": ("copy", "append", "mix_g2_p512"), "copies_and_append": ("copy", "append")}
    if counted:
        for i in range(n):
            run(*variants[MIXED_COUNTED_VARIANT])(i)
        torch.cuda.synchronize()
        return {"counted_variant": MIXED_COUNTED_VARIANT, "calls": n}
    for nm in reps[0]:
        for i in range(3):
            run(nm)(i)
    t = {key: _spun_avg_us(torch, stream, run(*names), n, spin) for key, names in variants.items()}
    # Algorithmic decode bytes: every distinct cached token once (the shared prefix's blocks are
    # the same physical blocks in all 16 tables) plus each sample's own tokens, K and V of the 8 KV
    # heads, and the queries.  Logical bytes count each sample's whole context.
    shared_blocks = 0
    for j in range(dtab.shape[1]):
        if (dtab[:, j] == dtab[0, j]).all() and dtab[0, j] >= 0:
            shared_blocks += 1
        else:
            break
    shared_tok = shared_blocks * 16
    tok_bytes = mw.Hkv * mw.D * 2 * 2
    q_bytes = mw.samples * mw.Hq * mw.D * 2
    unique = (shared_tok + int(np.sum(dlens - shared_tok))) * tok_bytes + q_bytes
    logical = int(np.sum(dlens)) * tok_bytes + q_bytes
    pairs = sum(mw.ctx_start + i + 1 for i in range(mw.chunk))
    flops = pairs * mw.Hq * 4 * mw.D
    best_key = min(("decode_grouped_2", "decode_grouped_4", "decode_grouped_2_split512"), key=lambda x: t[x])
    best_dec = t[best_key]
    ach = unique / (best_dec * 1e-6) / 1e9
    pre_tf = flops / (t["prefill"] * 1e-6) / 1e12
    return {
        "workload": f"mixed_step_16_samples_prefix{prefix_len}_plus_chunk512_ctx4096_gqa32x8_d128_bf16",
        "block_copies": int(len(cow)),
        "shared_prefix_tokens": shared_tok,
        "decode_unique_bytes": unique,
        "decode_logical_bytes": logical,
        "prefill_flops": flops,
        "us": {k: round(x, 2) for k, x in t.items()},
        "decode_grouped_speedup": round(t["decode"] / best_dec, 2),
        "mixed_grouped_speedup_over_separate": round(t["separate"] / t["mixed_grouped"], 3),
        "step_speedup": round(t["step_separate"] / min(t["step_mixed"], t["step_mixed_grouped"]), 3),
        "decode_roofline": {"bound": "hbm", "kernel": f"decode_group_kernel ({best_key})", "achieved": round(ach, 1),
                            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                            **(_traffic_fields("mixed", unique) if best_key == MIXED_COUNTED_VARIANT and
                               prefix_len == 2048 else {"traffic": None}),
                            "note": "unique algorithmic bytes (each distinct cached token once + queries); "
                                    "traffic: the grouped kernel's launch, its reduce not counted"},
        "decode_plain_unique_frac": round(unique / (t["decode"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "decode_logical_gbs": {"plain": round(logical / (t["decode"] * 1e-6) / 1e9, 1),
                               "grouped": round(logical / (best_dec * 1e-6) / 1e9, 1)},
        "prefill_roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel", "achieved": round(pre_tf, 2),
                             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(pre_tf / PEAK_BF16_TFLOPS, 4),
                             **_traffic_fields("prefill", _prefill_bytes(mw.ctx_start, mw.chunk, mw.Hq, mw.Hkv,
                                                                         mw.D, False))},
        "replicas": R,
    }


def cpu_baseline_mixed(seconds: float):
    """The oracle on the prefix-sharing step: the 16 samples' decode over their 2,049 tokens, whole,
    and the prefill of the first R chunk rows (R grown until the prefill sample takes about
    `seconds`), its time scaled to the chunk's 512 rows by their (row, key) pairs."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import CacheModel, PoolModel
    from oracle import attention as oatt

    mw = wl.mixed_step(5, prefix_len=2048)
    rng = np.random.default_rng(1055)
    pool = PoolModel(mw.num_blocks, 16, mw.free_order)
    cache = CacheModel(mw.num_blocks, mw.Hkv, mw.D, "bf16", fill_nan=True)
    s0 = pool.new_seq()
    slots, _ = pool.append(s0, mw.prefix_len)
    cache.append(wl.normal_bits(rng, (mw.prefix_len, mw.Hkv, mw.D), "bf16"),
                 wl.normal_bits(rng, (mw.prefix_len, mw.Hkv, mw.D), "bf16"), slots)
    samples = [s0] + [pool.fork(s0) for _ in range(mw.samples - 1)]
    for s in samples:
        sl, cw = pool.append(s, 1)
        cache.copy_blocks(cw)
        cache.append(wl.normal_bits(rng, (1, mw.Hkv, mw.D), "bf16"), wl.normal_bits(rng, (1, mw.Hkv, mw.D), "bf16"), sl)
    q = wl.normal_bits(rng, (mw.samples, mw.Hq, mw.D), "bf16")
    tables, lens = pool.block_tables(samples, len(pool.tables[s0]))
    t0 = time.perf_counter()
    oatt.paged_decode(q, cache, tables, lens, mw.scale)
    dec_s = time.perf_counter() - t0
    pre = cpu_baseline_prefill(mw.ctx_start, mw.Hq, mw.Hkv, mw.D, mw.scale, seconds)
    flops = sum(mw.ctx_start + i + 1 for i in range(mw.chunk)) * mw.Hq * 4 * mw.D
    pre_s = flops / (pre["value"] * 1e12)
    step_s = dec_s + pre_s
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(1.0 / step_s, 4), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "us_per_step": round(step_s * 1e6, 1),
            "sample": (f"decode of all 16 samples ({dec_s:.2f} s) + prefill {pre['sample']}, scaled to 512 rows "
                       f"({pre_s:.2f} s); numpy fp64")}


def _mixed_fp8_case(args, dev, n, spin):
    """The prefix-sharing step's attention over an FP8 cache (the same scene: 16 samples on a
    2,048-token prefix, a 512-row chunk after 4,096 tokens, every slot of the pool filled by the
    quantising append, bf16 queries): the FP8 decode and FP8 prefill as separate launches against
    one paged_attention_mixed_fp8 launch, single pass and with 512-token partitions."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    mw = wl.mixed_step(5, prefix_len=2048)
    pool = BlockPool(mw.num_blocks, 16, mw.free_order)
    s0 = pool.new_seq()
    pool.append(s0, mw.prefix_len)
    samples = [s0] + [pool.fork(s0) for _ in range(mw.samples - 1)]
    pf = pool.new_seq()
    pool.append(pf, mw.ctx_start)
    st, _, _, _ = pool.append_many(samples + [pf], [1] * mw.samples + [mw.chunk])
    assert st == 0
    dtab, dlens = pool.block_tables(samples, wl.blocks_for(mw.prefix_len + 1))
    ptab, _ = pool.block_tables([pf], wl.blocks_for(mw.ctx_start + mw.chunk))
    dt_t, dl_t, pt_t = (torch.from_numpy(x).to(dev) for x in (dtab, dlens, ptab))
    mcl = int(dlens.max())
    T = mw.num_blocks * 16
    all_slots = torch.arange(T, dtype=torch.int32, device=dev)
    per_rep = 2 * mw.num_blocks * mw.Hkv * 16 * (mw.D + 4)
    R = max(1, math.ceil((1 << 30) / per_rep))
    g = torch.Generator(device=dev)
    g.manual_seed(56)
    reps = []
    for r in range(R):
        k, v, ks, vs = ops.fp8_cache(mw.num_blocks, mw.Hkv, mw.D, device=dev)
        kb = torch.randn((T, mw.Hkv, mw.D), generator=g, device=dev).to(torch.bfloat16)
        vb = torch.randn((T, mw.Hkv, mw.D), generator=g, device=dev).to(torch.bfloat16)
        ops.paged_cache_append_fp8(k, v, ks, vs, kb, vb, all_slots)
        del kb, vb
        qd = torch.randn((mw.samples, mw.Hq, mw.D), generator=g, device=dev).to(torch.bfloat16)
        qp = torch.randn((mw.chunk, mw.Hq, mw.D), generator=g, device=dev).to(torch.bfloat16)
        od = torch.empty((mw.samples, mw.Hq, mw.D), dtype=torch.float32, device=dev)
        op = torch.empty((mw.chunk, mw.Hq, mw.D), dtype=torch.float32, device=dev)
        ws = ops.decode_workspace(mw.samples, mw.Hq, mw.D, mcl, 512)
        mix = (od, qd, dt_t, dl_t, mcl, op, qp, pt_t, [mw.ctx_start], [mw.chunk], k, v, ks, vs, mw.scale)
        reps.append({
            "dec": ops.PreparedDecodeFp8(od, qd, k, v, ks, vs, dt_t, dl_t, mcl, mw.scale, 0, None,
                                         host_context_lens=dlens),
            "dec_p512": ops.PreparedDecodeFp8(od, qd, k, v, ks, vs, dt_t, dl_t, mcl, mw.scale, 512, ws,
                                              host_context_lens=dlens),
            "dec_g2_p512": lambda od=od, qd=qd, k=k, v=v, ks=ks, vs=vs, ws=ws: ops.paged_attention_decode_grouped_fp8(
                od, qd, k, v, ks, vs, dt_t, dl_t, mcl, mw.scale, 2, 512, ws),
            "pre": ops.PreparedPrefillFp8(op, qp, k, v, ks, vs, pt_t[0], mw.ctx_start, mw.scale),
            "mix": lambda mix=mix: ops.paged_attention_mixed_fp8(*mix, host_dec_lens=dlens),
            "mix_p512": lambda mix=mix, ws=ws: ops.paged_attention_mixed_fp8(*mix, host_dec_lens=dlens,
                                                                              dec_partition_size=512, workspace=ws),
        })
    stream = torch.cuda.current_stream()

    def run(*names):
        def fn(i):
            r = reps[i % R]
            for nm in names:
                r[nm]()
        return fn

    for nm in reps[0]:
        for i in range(3):
            run(nm)(i)
    variants = {"decode": ("dec",), "decode_split512": ("dec_p512",), "decode_grouped_2_split512": ("dec_g2_p512",),
                "prefill": ("pre",), "separate": ("dec", "pre"), "separate_split512": ("dec_p512", "pre"),
                "separate_grouped": ("dec_g2_p512", "pre"), "mixed": ("mix",), "mixed_split512": ("mix_p512",)}
    t = {key: _spun_avg_us(torch, stream, run(*names), n, spin) for key, names in variants.items()}
    best_sep = min(t["separate"], t["separate_split512"])
    best_mix = min(t["mixed"], t["mixed_split512"])
    return {"workload": "mixed_step_16_samples_prefix2048_plus_chunk512_ctx4096_gqa32x8_d128_fp8_cache_bf16_query",
            "us": {k: round(x, 2) for k, x in t.items()}, "mixed_speedup_over_separate": round(best_sep / best_mix, 3),
            "decode_grouped_speedup": round(min(t["decode"], t["decode_split512"]) / t["decode_grouped_2_split512"], 2),
            "grouped": "paged_attention_decode_grouped_fp8, 2 samples per workgroup, 512-token partitions",
            "replicas": R}


def measure_mixed(args, dev, counted=False):
    """The mixed prefix-sharing step (a 2,048-token shared prefix), and its copy-on-write variant
    (2,040 tokens: the partial last prefix block is copied for 15 of the 16 samples).  counted:
    the counter run of the decode variant the traffic record covers."""
    import torch

    stream = torch.cuda.current_stream()
    if counted:
        return _mixed_case(args, dev, 2048, max(5, args.steps), 0, counted=True)
    spin = int(_spin_cycles_per_ms(torch, stream) * 50)
    n = max(20, args.steps // 4)
    res = _mixed_case(args, dev, 2048, n, spin)
    res["copy_on_write_variant"] = _mixed_case(args, dev, 2040, n, spin)
    res["fp8_cache"] = _mixed_fp8_case(args, dev, n, spin)
    res["timing"] = (f"{n} back-to-back calls behind a 50 ms spin, one HIP event pair (device time only); "
                     "grouped = paged_attention_decode_grouped / paged_attention_mixed with dec_group_size "
                     "(2 samples per workgroup), split512 = 512-token partitions + reduce; every decode variant's "
                     "outputs are bit for bit the plain decode's with the same partition size")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_mixed(args.cpu_seconds / 2)
    return res


def measure_tiny(args, dev, counted=False):
    """The tiny fp32 step: batch 4, 8 q = 8 kv heads of 64, a 32-block pool handed out from a seeded
    permutation, lengths {5, 17, 32, 40}.  A step = paged_attention_decode_append: the step's 4
    tokens written into their slots inside the decode launch (the vector-ALU kernel's fused append);
    the append + decode as two launches is reported beside it.  Device time of n back-to-back steps
    behind a spin; the step moves 0.4 MB, so launch latency, not HBM, sets its time.  counted: the
    counter run, which launches the fused step only."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    w = wl.tiny_decode(1)
    pool = BlockPool(w.num_blocks, 16, w.free_order)
    seqs = [pool.new_seq() for _ in range(w.B)]
    st, _, _, _ = pool.append_many(seqs, [int(L) - 1 for L in w.lens])
    st2, _, step_slots, _ = pool.append_many(seqs, [1] * w.B)
    assert st == 0 and st2 == 0
    tables, lens = pool.block_tables(seqs, w.max_blocks_per_seq)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    f32 = torch.float32
    k = torch.randn((w.num_blocks, w.Hkv, 16 * w.D), generator=g, device=dev, dtype=f32)
    v = torch.randn((w.num_blocks, w.Hkv, 16 * w.D), generator=g, device=dev, dtype=f32)
    q = torch.randn((w.B, w.Hq, w.D), generator=g, device=dev, dtype=f32)
    sk = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev, dtype=f32)
    sv = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev, dtype=f32)
    out = torch.empty((w.B, w.Hq, w.D), dtype=f32, device=dev)
    tables_t, lens_t = torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev)
    app = ops.PreparedAppend(k, v, sk, sv, torch.from_numpy(step_slots).to(dev))
    dec = ops.PreparedDecode(out, q, k, v, tables_t, lens_t, int(lens.max()), w.scale, 0, None,
                             host_context_lens=lens)
    fused = ops.PreparedDecode(out, q, k, v, tables_t, lens_t, int(lens.max()), w.scale, 0, None,
                               host_context_lens=lens, new_key=sk, new_value=sv)
    for _ in range(5):
        fused()
        if not counted:
            app()
            dec()
    stream = torch.cuda.current_stream()
    n = max(50, args.steps)
    spin = int(_spin_cycles_per_ms(torch, stream) * 20)
    step_us = _spun_avg_us(torch, stream, lambda i: fused(), n, spin)
    sep_us = dec_us = None
    if not counted:
        sep_us = _spun_avg_us(torch, stream, lambda i: (app(), dec()), n, spin)
        dec_us = _spun_avg_us(torch, stream, lambda i: dec(), n, spin)
    nbytes = w.kv_bytes() + w.q_bytes()
    gbs = nbytes / (step_us * 1e-6) / 1e9
    res = {
        "workload": w.name,
        "kv_plus_q_bytes_per_step": nbytes,
        "us_per_step": round(step_us, 3),
        "seqs_steps_per_s": round(w.B / (step_us * 1e-6), 1),
        "separate_launches_us_per_step": None if sep_us is None else round(sep_us, 3),
        "kernel_us": {"decode_fused_append": round(step_us, 3),
                      "decode_alone": None if dec_us is None else round(dec_us, 3)},
        "step": "paged_attention_decode_append (fp32: the new tokens written inside the vector-ALU decode), single pass",
        "roofline": {"bound": "hbm", "kernel": "decode_valu_kernel (append fused)", "achieved": round(gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 6),
                     **_traffic_fields("tiny", nbytes), "note": "latency-bound: 32 workgroups move 0.4 MB"},
        "timing": f"{n} back-to-back steps behind a 20 ms spin, one HIP event pair (device time only)",
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_tiny(w, args.cpu_seconds / 4)
    return res


def cpu_baseline_tiny(w, seconds):
    """The oracle on the whole tiny step: the 4 new tokens written into its cache model, then the
    fp64 decode of the 4 sequences, repeated for about `seconds`."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import CacheModel, PoolModel
    from oracle import attention as oatt

    rng = np.random.default_rng(1001)
    pool = PoolModel(w.num_blocks, 16, w.free_order)
    seqs = [pool.new_seq() for _ in range(w.B)]
    cache = CacheModel(w.num_blocks, w.Hkv, w.D, w.dtype, fill_nan=True)
    for s, L in zip(seqs, w.lens):
        slots, _ = pool.append(s, int(L) - 1)
        cache.append(wl.normal_bits(rng, (int(L) - 1, w.Hkv, w.D), "f32"),
                     wl.normal_bits(rng, (int(L) - 1, w.Hkv, w.D), "f32"), slots)
    step_slots = []
    for s in seqs:
        sl, _ = pool.append(s, 1)
        step_slots += sl
    tables, lens = pool.block_tables(seqs, w.max_blocks_per_seq)
    q = wl.normal_bits(rng, (w.B, w.Hq, w.D), "f32")
    nk, nv = wl.normal_bits(rng, (w.B, w.Hkv, w.D), "f32"), wl.normal_bits(rng, (w.B, w.Hkv, w.D), "f32")
    reps, t0 = 0, time.perf_counter()
    while True:
        cache.append(nk, nv, step_slots)
        oatt.paged_decode(q, cache, tables, lens, w.scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds and reps >= 3:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    per = el / reps
    return {"value": round((w.kv_bytes() + w.q_bytes()) / per / 1e9, 5), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "us_per_step": round(per * 1e6, 1), "seqs_steps_per_s": round(w.B / per, 1),
            "sample": f"the whole step (append + decode of all 4 sequences), {reps} steps in {el:.1f} s"}


def measure_long(args, dev):
    """The long-context decode: batch 8 at 32,768 tokens (2,048 scattered blocks each), split-K
    over 512-token partitions, fused append; KV + Q bytes per step as in the main line."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    w = wl.long_context_decode(4)
    pool = BlockPool(w.num_blocks, 16, w.free_order)
    seqs = [pool.new_seq() for _ in range(w.B)]
    st, _, _, _ = pool.append_many(seqs, [int(L) for L in w.lens])
    assert st == 0
    tables, lens = pool.block_tables(seqs, w.max_blocks_per_seq)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    k = torch.randn((w.num_blocks, w.Hkv, 16 * w.D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((w.num_blocks, w.Hkv, 16 * w.D), generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn((w.B, w.Hq, w.D), generator=g, device=dev).to(torch.bfloat16)
    sk = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
    sv = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    maxL = int(lens.max())
    ws = ops.decode_workspace(w.B, w.Hq, w.D, maxL, w.partition_size, device=dev)
    dec = ops.PreparedDecode(out, q, k, v, torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), maxL,
                             w.scale, w.partition_size, ws, new_key=sk, new_value=sv,
                             host_context_lens=None if args.no_order else lens)
    for _ in range(3):
        dec()
    n = max(10, args.steps // 10)
    stream = torch.cuda.current_stream()
    step_us = _events_avg_us(torch, stream, lambda i: dec(), n)
    part_us = _events_avg_us(torch, stream, lambda i: dec.partitions(), n)
    nbytes = w.kv_bytes() + w.q_bytes()
    gbs = nbytes / (part_us * 1e-6) / 1e9
    return {
        "workload": w.name,
        "kv_plus_q_bytes_per_step": nbytes,
        "us_per_step": round(step_us, 3),
        "gbs_per_step": round(nbytes / (step_us * 1e-6) / 1e9, 1),
        "seqs_steps_per_s": round(w.B / (step_us * 1e-6), 1),
        "kernel_us": {"decode_partitions": round(part_us, 3), "decode_reduce": round(step_us - part_us, 3)},
        "roofline": {"bound": "hbm", "kernel": "decode_mfma_kernel (partition pass, fused append)",
                     "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), **_traffic_fields("long", nbytes)},
    }


def cpu_baseline(w, seconds: float, max_seqs: int = 8):
    """The oracle (numpy fp64 gather + softmax attention) on a bounded sample of the same workload:
    the first S = min(B, max_seqs) sequences, inputs drawn on the host with the same generators."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import CacheModel, PoolModel
    from oracle import attention as oatt

    S = min(w.B, max_seqs)
    lens = w.lens[:S]
    need = sum(wl.blocks_for(int(L)) for L in lens)
    rng = np.random.default_rng(1000 + w.seed)
    N = need + 1
    pool = PoolModel(N, 16, rng.permutation(N))
    cache = CacheModel(N, w.Hkv, w.D, w.dtype, fill_nan=True)
    seqs = []
    for L in lens:
        s = pool.new_seq()
        slots, _ = pool.append(s, int(L))
        cache.append(wl.normal_bits(rng, (int(L), w.Hkv, w.D), w.dtype),
                     wl.normal_bits(rng, (int(L), w.Hkv, w.D), w.dtype), slots)
        seqs.append(s)
    q = wl.normal_bits(rng, (S, w.Hq, w.D), w.dtype)
    tables, tl = pool.block_tables(seqs, max(len(pool.tables[s]) for s in seqs))
    eb = wl.elem_bytes(w.dtype)
    sample_bytes = int(np.sum(lens.astype(np.int64))) * w.Hkv * w.D * 2 * eb + S * w.Hq * w.D * eb
    reps, t0 = 0, time.perf_counter()
    while True:
        oatt.paged_decode(q, cache, tables, tl, w.scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds and reps >= 3:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    per_call = el / reps
    return {
        "value": round(sample_bytes / per_call / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{S} of {w.B} sequences ({int(np.sum(lens))} cached tokens, {sample_bytes} B KV+Q), numpy fp64 "
                   f"gather + softmax attention, {reps} calls in {el:.1f} s; host has "
                   f"{len(os.sched_getaffinity(0))} usable cores"),
        "seqs_steps_per_s": round(S / per_call, 3),
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_one_core(args):
    """The same oracle sample in a child process with one BLAS/OpenMP thread (half the time budget)."""
    import subprocess

    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
               BLIS_NUM_THREADS="1", HIP_VISIBLE_DEVICES="")
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-only", "--workload", args.workload,
           "--cpu-seconds", str(args.cpu_seconds / 2)]
    try:
        p = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=120 + 4 * args.cpu_seconds)
        one = json.loads(p.stdout.strip().splitlines()[-1])
    except (subprocess.SubprocessError, ValueError, IndexError) as e:
        return {"error": f"single-core run failed: {e}"}
    return {k: one[k] for k in ("value", "unit", "cores", "sample", "seqs_steps_per_s") if k in one}


def measure_read_probe(dev, step_bytes: int) -> dict:
    """Achievable HBM read bandwidth: paged_probe_stream_read (16-byte nontemporal loads, the decode
    kernel's load form) over a 4 GiB buffer and over windows of one decode step's byte count,
    rotated through the 4 GiB so that no window is re-read from the 256 MB last-level cache.  The
    best of five grid sizes; HIP events on the launch stream around 20 back-to-back launches."""
    import torch

    from paged_kv_cache_404_amd import ops

    total = 4 << 30
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    out = {}
    for name, size in (("4GiB", total), ("step_bytes", step_bytes // 16 * 16)):
        windows = max(1, total // size)
        best = 0.0
        for wgs in (2048, 4096, 8192, 16384, 32768):
            n = 20
            ops.probe_stream_read(buf, size, sink, wgs)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(n):
                off = (i % windows) * size
                ops.probe_stream_read(buf[off:off + size], size, sink, wgs)
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, size * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        out[name] = round(best, 1)
    del buf
    return out


def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(write_traffic(*args.traffic_from)))
        return
    if args.cpu_baseline_only:
        import workloads as wl
        w = (wl.llama_decode(2, partition_size=0) if args.workload == "llama"
             else wl.long_context_decode(4, partition_size=512))
        print(json.dumps(cpu_baseline(w, args.cpu_seconds)), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); this library "
              "has no multi-GPU path in this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_404_amd import BlockPool, ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        args.no_cpu_baseline = True
        if args.only == "llama":
            args.no_extra = True
            args.workload = "llama"
        else:
            res = {"long": lambda: measure_long(args, dev), "tiny": lambda: measure_tiny(args, dev, counted=True),
                   "prefill": lambda: measure_prefill(args, dev), "prefill_fp8": lambda: measure_prefill(args, dev, True),
                   "fp8": lambda: measure_fp8(args, dev, None), "mixed": lambda: measure_mixed(args, dev, counted=True),
                   "trace": lambda: measure_trace(dev, counters=True)}[args.only]()
            calibration_copy(dev)
            print(json.dumps(res), flush=True)
            return
    if args.workload == "llama":
        w = wl.llama_decode(2, partition_size=0 if args.partition_size is None else args.partition_size)
    else:
        w = wl.long_context_decode(4, partition_size=512 if args.partition_size is None else args.partition_size)

    # Host pool + builders: the cached prefix, then this step's append (timed on the host).
    pool = BlockPool(w.num_blocks, 16, w.free_order)
    seqs = [pool.new_seq() for _ in range(w.B)]
    st, _, _, _ = pool.append_many(seqs, [int(L) - 1 for L in w.lens])
    assert st == 0
    st, _, step_slots, cow = pool.append_many(seqs, [1] * w.B)
    tables, lens = pool.block_tables(seqs, w.max_blocks_per_seq)
    assert st == 0 and len(cow) == 0 and np.array_equal(lens, w.lens)
    # Host time of one step's pool append + builders: median of 50 steps on a scratch pool in the
    # same state (room for the extra tokens), through the Python binding.
    spare = BlockPool(w.num_blocks + 4 * w.B, 16, None)
    sseqs = [spare.new_seq() for _ in range(w.B)]
    spare.append_many(sseqs, [int(L) - 1 for L in w.lens])
    host_t = []
    for _ in range(50):
        t0 = time.perf_counter()
        spare.append_many(sseqs, [1] * w.B)
        spare.block_tables(sseqs, w.max_blocks_per_seq + 4)
        host_t.append(time.perf_counter() - t0)
    host_us = float(np.median(host_t)) * 1e6
    del spare

    eb = wl.elem_bytes(w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    cache_bytes = 2 * w.num_blocks * w.Hkv * 16 * w.D * eb
    R = args.replicas or max(1, math.ceil((1 << 30) / cache_bytes))
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    tables_t = torch.from_numpy(tables).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    slots_t = torch.from_numpy(step_slots).to(dev)
    maxL = int(lens.max())
    side = torch.cuda.Stream(device=dev) if args.overlap else None
    reps = []
    for r in range(R):
        k = torch.randn((w.num_blocks, w.Hkv, 16 * w.D), generator=g, device=dev, dtype=torch.float32).to(tdt)
        v = torch.randn((w.num_blocks, w.Hkv, 16 * w.D), generator=g, device=dev, dtype=torch.float32).to(tdt)
        q = torch.randn((w.B, w.Hq, w.D), generator=g, device=dev, dtype=torch.float32).to(tdt)
        sk = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev, dtype=torch.float32).to(tdt)
        sv = torch.randn((w.B, w.Hkv, w.D), generator=g, device=dev, dtype=torch.float32).to(tdt)
        out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
        ws = ops.decode_workspace(w.B, w.Hq, w.D, maxL, w.partition_size, device=dev)
        reps.append((ops.PreparedAppend(k, v, sk, sv, slots_t, stream=side),
                     ops.PreparedDecode(out, q, k, v, tables_t, lens_t, maxL, w.scale, w.partition_size, ws,
                                        new_key=None if args.separate else sk,
                                        new_value=None if args.separate else sv,
                                        host_context_lens=None if args.no_order else lens,
                                        write_cache=not args.overlap)))
    torch.cuda.synchronize()
    main_stream = torch.cuda.current_stream()

    def step(i):
        app, dec = reps[i % R]
        if args.separate:
            app()
        elif args.overlap:
            # The append may run beside this step's decode (which takes the new tokens from the
            # input rows); the next step's decode reads them from the cache, so it waits for it.
            side.wait_stream(main_stream)
            app()
            dec.partitions()
            dec.reduce()
            main_stream.wait_stream(side)
            return
        dec.partitions()
        dec.reduce()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly K steps bracketed by synchronisation (one GPU: the barrier is a no-op).
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Per-kernel average launch durations: K back-to-back launches of one kernel between two HIP
    # events recorded on the launch stream (the library enqueues on torch's current stream).
    def avg_us(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    if args.overlap:
        # Kernel durations alone, both on the main stream.
        reps = [(ops.PreparedAppend(*a._keep), d) for a, d in reps]
    t_app = avg_us(lambda i: reps[i % R][0]()) if args.separate or args.overlap else 0.0
    t_part = avg_us(lambda i: reps[i % R][1].partitions())
    t_red = avg_us(lambda i: reps[i % R][1].reduce())

    # Per-call distribution: an event pair around each of K more steps.
    pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(pe):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in pe)

    def quantile(f):
        return round(per_call[min(len(per_call) - 1, int(f * (len(per_call) - 1) + 0.5))], 3)

    kv = w.kv_bytes()
    qb = w.q_bytes()
    step_bytes = kv + qb
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    part_us = float(t_part)
    achieved = step_bytes / (part_us * 1e-6) / 1e9
    traffic = measured_traffic(args.workload)
    read_probe = measure_read_probe(dev, step_bytes)

    # Achievable streaming bandwidth: a plain device copy of 1 GiB.
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 5 / (time.perf_counter() - c0) / 1e9
    del src, dst

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.B,
            "num_q_heads": w.Hq,
            "num_kv_heads": w.Hkv,
            "head_dim": w.D,
            "block_size": 16,
            "context_lens": f"seeded U[{int(w.lens.min())}..{int(w.lens.max())}] sum {int(w.lens.sum())}"
            if args.workload == "llama" else f"{int(w.lens[0])} each",
            "num_blocks": w.num_blocks,
            "partition_size": w.partition_size,
            "work_order": "natural" if args.no_order else "longest first (host copy of the lengths)",
            "replicas": R,
            "parallelism": "none (one GPU)",
        },
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "seqs_steps_per_s": round(w.B / (wall / args.steps), 1),
        "kv_plus_q_bytes_per_step": step_bytes,
        "step": (("paged_cache_append + paged_attention_decode" if args.separate else
                  "paged_attention_decode_newest with paged_cache_append on a second stream" if args.overlap else
                  "paged_attention_decode_append (append fused into the decode kernel)") +
                 (", single pass" if w.partition_size == 0 else
                  f", {w.partition_size}-token partitions + log-sum-exp reduce")),
        "kernel_us": {"append": round(float(t_app), 3), "decode_partitions": round(part_us, 3),
                      "decode_reduce": round(float(t_red), 3)},
        "per_call_us": {"median": quantile(0.5), "p10": quantile(0.1), "p90": quantile(0.9), "calls": len(per_call),
                        "note": "an event pair around each step; the value above is K back-to-back steps"},
        "host_pool_and_builders_us_per_step": round(host_us, 1),  # median of 50 steps
        "device_copy_probe_gbs": round(copy_gbs, 1),
        "achievable_read": {
            "probe": "paged_probe_stream_read, 16-byte nontemporal loads, 8 in flight per lane, best of 5 grid sizes",
            "gbs": read_probe,
            "pct_of_peak_hbm": {k: round(100 * v / PEAK_HBM_GBS, 2) for k, v in read_probe.items()},
            "decode_kernel_frac_of_achievable_at_step_bytes": round(achieved / read_probe["step_bytes"], 4),
            "step_frac_of_achievable_at_step_bytes": round(value / read_probe["step_bytes"], 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_mfma_kernel" + ("" if args.separate else " (new tokens from the input rows)"
                                              if args.overlap else " (fused append)"),
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / step_bytes, 4) if traffic else None,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        res["cpu_baseline"]["cpu_model"] = cpu_model()
        res["cpu_baseline"]["single_core"] = cpu_baseline_one_core(args)
    extras = set(args.extras.split(","))
    if not args.no_extra and args.workload == "llama":
        del reps
        torch.cuda.empty_cache()
        if "tiny" in extras:
            res["tiny"] = measure_tiny(args, dev)
        if "prefill" in extras:
            res["prefill"] = measure_prefill(args, dev)
        if "prefill_fp8" in extras:
            res["prefill_fp8"] = measure_prefill(args, dev, fp8=True)
        if "long" in extras:
            res["long_context"] = measure_long(args, dev)
            if not args.no_cpu_baseline:
                res["long_context"]["cpu_baseline"] = cpu_baseline(wl.long_context_decode(4), args.cpu_seconds / 2,
                                                                   max_seqs=1)
        if "prefix" in extras:
            res["prefix_cache"] = measure_prefix_cache()
        if "fp8" in extras:
            res["fp8_cache"] = measure_fp8(args, dev, part_us)
        if "mixed" in extras:
            res["mixed_step"] = measure_mixed(args, dev)
    if not args.no_extra and args.workload == "llama" and "trace" in extras:
        res["trace"] = measure_trace(dev)
        med = res["trace"].pop("_median_step_lens")
        if not args.no_cpu_baseline:
            # The oracle on 8 sequences of the trace's median-batch step, its GB/s extrapolated to the
            # trace's total decode bytes (running it on every step would take hours).
            w_med = wl.custom_decode(3, med, 32, 8, 128, "bf16")
            cb = cpu_baseline(w_med, args.cpu_seconds / 4, max_seqs=8)
            total_s = res["trace"]["decode_kv_plus_q_bytes"] / (cb["value"] * 1e9)
            cb["sample"] = f"median-batch step of the trace ({len(med)} sequences): " + cb["sample"]
            cb["extrapolated_trace_decode_s"] = round(total_s, 1)
            cb["extrapolated_seqs_steps_per_s"] = round(res["trace"]["seq_steps"] / total_s, 1)
            res["trace"]["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

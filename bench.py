#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one pass of the whole decode path over one batch: slot mapping of
the new tokens, the cache write, then decode.  Default (--mode fused):
pa_decode_step, where the balanced split-KV kernel also derives each new
token's slot and writes its K/V, followed by the reduce.  Other modes run
pa_slot_mapping + pa_cache_write and then balanced, fixed-partition split-KV
(+ reduce) or single-pass decode.  Inputs are seeded synthetic
workloads already resident in HBM.  Timed steps rotate over --rotate copies
of the pool so repeated reads cannot be served by the 256 MB MALL or L2.

Prints ONE JSON line.  ``value`` is KV GB/s: the KV bytes the step must read
(exactly context_len tokens per sequence, K and V) over the step time.
``roofline`` rates the dominant kernel (the decode partition kernel) against
HBM peak with its algorithmic bytes over its event-timed duration.
``cpu_baseline`` is the float64 CPU oracle timed on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode KV GB/s (% of HBM peak) + seqs/s at Llama-2-13B layer shape"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "c1": "tiny paged decode 25/47/12 tokens, 4/4 heads, D64, B16",
    "c2": "Llama-2-13B layer decode: 32 seqs ctx U[1,2048], 40/40 heads, D128, B16, 4000-block pool",
    "c3": "GQA Llama-3-8B-like layer decode: 64 seqs ctx lognormal(700,1) in [1,8192], 32/8 heads, D128, B16",
    "c4": "prefix sharing + COW: 16 prompts x 4 samples, 1024+r shared, tails U[0,512], 40/40 heads, D128, B16",
    "c5_b32": "long-context split-KV: 8 seqs ctx U[32768,131072], 64/8 heads, D128, B32",
    "c5_b64": "long-context split-KV: 8 seqs ctx U[32768,131072], 64/8 heads, D128, B64",
    "c2_spec4": "speculative verify, 4 query tokens per seq: Llama-2-13B layer, 32 seqs "
                "ctx U[4,2048], 40/40 heads, D128, B16",
    "c3_spec4": "speculative verify, 4 query tokens per seq: GQA 32/8 heads, 64 seqs ctx "
                "lognormal(700,1) in [4,8192], D128, B16",
}


def kv_bytes(w) -> int:
    """Algorithmic KV bytes of one decode: K and V rows of exactly
    context_len tokens per sequence."""
    return int(w.context_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_size * 2


def split_kernel_bytes(w) -> int:
    """Algorithmic bytes of one split-KV partition-kernel launch: KV rows, the
    query, the block-table entries read, and the partition states written."""
    S, H, D = w.query.shape
    B, P = w.block_size, w.partition_size
    n = w.context_lens.astype(np.int64)
    table = int(((n + B - 1) // B).sum()) * 4
    parts = int(((n + P - 1) // P).sum()) * H * (D + 2) * 4
    return kv_bytes(w) + S * H * D * 2 + table + parts


PAIR_COST = 64      # flat units the balanced split charges per (sequence, kv head)


def balanced_split_ranges(w, grid: int) -> int:
    """Ranges of the balanced decode that belong to (sequence, kv head)
    pairs cut across several workgroups: each stores one partial state per
    query head, which the pair's last workgroup reads back to merge.  Same
    slicing as the kernel: a pair spans PAIR_COST units, then its length
    padded to 16; equal 16-aligned slices of that space."""
    M = w.max_blocks_per_seq * w.block_size
    n = np.minimum(w.context_lens.astype(np.int64), M)
    pad = np.where(n > 0, (n + 15) // 16 * 16, 0)
    span = np.where(pad > 0, pad + PAIR_COST, 0)
    Hkv = w.num_kv_heads
    total = int(span.sum()) * Hkv
    if total == 0:
        return 0
    C = -(-total // grid)
    C = (C + 15) // 16 * 16
    prefix = np.concatenate([[0], np.cumsum(span)[:-1]])
    count = 0
    for i in range(w.num_seqs):
        if n[i] <= 0:
            continue
        for kvh in range(Hkv):
            F = int(prefix[i]) * Hkv + kvh * int(span[i]) + PAIR_COST
            k = (F + int(n[i]) - 1) // C - F // C + 1
            if k > 1:
                count += k
    return count


def balanced_kernel_bytes(w, grid: int, fused: bool) -> int:
    """Algorithmic bytes of one balanced-kernel launch: KV rows, query, table
    entries, output, partial states of cut pairs (written, then read by the
    merging workgroup) and, for the fused step, this step's K/V rows (read
    and written) and the slots."""
    S, H, D = w.query.shape
    n = w.context_lens.astype(np.int64)
    table = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
    parts = 2 * balanced_split_ranges(w, grid) * w.group * (D + 2) * 4
    extra = (2 * 2 * S * w.num_kv_heads * D * 2 + S * 4) if fused else 0
    return kv_bytes(w) + 2 * S * H * D * 2 + table + parts + extra


def single_kernel_bytes(w) -> int:
    S, H, D = w.query.shape
    n = w.context_lens.astype(np.int64)
    table = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
    return kv_bytes(w) + 2 * S * H * D * 2 + table


def cpu_baseline(w, gpu_out=None, min_s: float = 10.0, max_s: float = 30.0):
    """The oracle (unchanged) on the host: cache write of the step's tokens
    plus float64 decode of the whole batch, repeated until >= min_s.  The
    first pass's outputs are also compared with ``gpu_out`` (one of the timed
    GPU steps) when it is given."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:                                   # pragma: no cover
        threadpool_limits = None
    import oracle
    kc = w.pool_init[0].copy()
    vc = w.pool_init[1].copy()
    oracle.apply_phases(kc, vc, list(w.history), w.block_size)
    ctx = threadpool_limits(1) if threadpool_limits else None
    reps, seqs = 0, 0
    first = {}
    t0 = time.perf_counter()
    try:
        while True:
            oracle.apply_phases(kc, vc, [w.step_copies, w.step_write], w.block_size)
            for i in range(w.num_seqs):
                o = oracle.decode(w.query[i:i + 1], kc, vc, w.block_tables[i:i + 1],
                                  w.context_lens[i:i + 1], w.scale)
                if reps == 0:
                    first[i] = o[0]
                seqs += 1
                if time.perf_counter() - t0 > max_s:
                    break
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_s or el > max_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    el = time.perf_counter() - t0
    frac = seqs / w.num_seqs
    parity = None
    if gpu_out is not None and first:
        idx = sorted(first)
        ref = np.stack([first[i] for i in idx])
        got = np.asarray(gpu_out, np.float64)[idx]
        err = np.abs(got - ref)
        parity = {"seqs_checked": len(idx), "max_abs_err": float(err.max()),
                  "within_tolerance": bool(((err <= 2e-3) | (err <= 1e-2 * np.abs(ref))).all())}
    return parity, {
        "value": round(seqs / el, 3), "unit": "seqs/s", "cores": 1, "kind": "oracle",
        "kv_gbs_equiv": round(kv_bytes(w) * frac / el / 1e9, 4),
        "seconds": round(el, 2),
        "sample": (f"{seqs} sequence decodes ({frac:.2f} passes over the {w.num_seqs}-seq "
                   f"batch, cache write of its new tokens per pass), float64 NumPy, "
                   f"1 BLAS thread"),
    }


KERNEL_SOURCES = ["paged_kv_cache_120_amd/csrc/decode.hip",
                  "paged_kv_cache_120_amd/csrc/common.h",
                  "paged_kv_cache_120_amd/csrc/decode.h"]


def kernel_source_hash(root: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(args, root: str):
    """HBM bytes per launch of the decode kernel from the committed counter
    summary for this workload and mode, if it was taken on the current
    kernel sources (else None)."""
    path = os.path.join(root, "profiles",
                        f"decode_{args.config}_{args.mode}_traffic.txt")
    if not os.path.exists(path):
        return None
    t = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                t[k.strip()] = v.strip()
    if t.get("kernel_source_sha256_16") != kernel_source_hash(root) or \
            t.get("partition_size") != str(args.partition):
        return None
    try:
        return int(float(t["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def load_counters(args, root: str):
    """Per-launch hardware counters of the decode kernel (L2 hit rate, LDS
    bank conflicts, matrix-core and vector instructions) from the committed
    summary for this workload and mode, if it was taken on the current
    kernel sources (else None)."""
    path = os.path.join(root, "profiles",
                        f"decode_{args.config}_{args.mode}_counters.txt")
    if not os.path.exists(path):
        return None
    t = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                t[k.strip()] = v.strip()
    if t.pop("kernel_source_sha256_16", None) != kernel_source_hash(root):
        return None
    out = {}
    for k, v in t.items():
        try:
            out[k] = float(v)
        except ValueError:
            continue
    return out or None


PROBE_BYTES = 4 << 30        # streaming-read probe buffer (well past the 256 MB MALL)


def stream_probe(dev, launches: int = 20) -> dict:
    """Read rate of one plain sequential pass over a 4 GiB buffer
    (pa_stream_read, 16-byte non-temporal loads), timed with events on the
    current stream at 2, 4 and 8 workgroups per CU; the fastest is the
    device's streaming-read ceiling in this run."""
    import torch
    import paged_kv_cache_120_amd as pa
    buf = torch.zeros(PROBE_BYTES, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(4 * 8 * cus, dtype=torch.int32, device=dev)
    best = None
    for grid in (2 * cus, 4 * cus, 8 * cus):
        for _ in range(3):
            pa.pa_stream_read(buf, sink, grid)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(launches):
            pa.pa_stream_read(buf, sink, grid)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        if best is None or ms < best[1]:
            best = (grid, ms)
    del buf, sink
    grid, ms = best
    gbs = PROBE_BYTES / (ms * 1e-3) / 1e9
    return {"kernel": "stream_read_kernel", "bytes": PROBE_BYTES, "grid": grid,
            "us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


HOST_LINK_PEAK_GBS = 64.0     # PCIe 5.0 x16, one direction (nominal)


def swap_bench(args, w, dev) -> int:
    """Swap (pa_swap_blocks) of every block the batch's tables reference:
    device pool -> pinned host pool, then back into the device pool, each
    timed over --steps launches with HIP events on the launch stream.  The
    last swap-in is checked bit-exact against the device pool it came from."""
    import torch
    import paged_kv_cache_120_amd as pa
    from paged_kv_cache_120_amd import runner
    st = runner.upload(w, dev)
    runner.apply_history(w, st)
    torch.cuda.synchronize()
    B = w.block_size
    used = sorted({int(b) for i, n in enumerate(w.context_lens)
                   for b in w.block_tables[i, :(int(n) + B - 1) // B]})
    nu = len(used)
    blk = B * w.num_kv_heads * w.head_size * 2                  # bytes per block half
    host = torch.empty((2, nu) + tuple(st.pool.shape[2:]), dtype=torch.float16,
                       pin_memory=True)
    back = torch.empty_like(st.pool)
    dev_ids = torch.tensor(used, dtype=torch.int32, device=dev)
    host_ids = torch.arange(nu, dtype=torch.int32, device=dev)

    def timed(fn):
        for _ in range(min(args.warmup, 3)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_out = timed(lambda: pa.pa_swap_blocks(st.pool[0], st.pool[1], host[0], host[1],
                                             dev_ids, host_ids))
    ms_in = timed(lambda: pa.pa_swap_blocks(host[0], host[1], back[0], back[1],
                                            host_ids, dev_ids))
    idx = dev_ids.long()
    exact = torch.equal(back[:, idx].view(torch.int16), st.pool[:, idx].view(torch.int16))
    nbytes = 2 * nu * blk
    gbs_out = nbytes / (ms_out * 1e-3) / 1e9
    gbs_in = nbytes / (ms_in * 1e-3) / 1e9
    rec = {
        "metric": "paged KV block swap GB/s (device <-> pinned host)",
        "value": round(2 * nbytes / ((ms_out + ms_in) * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_out + ms_in, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config,
                   "blocks": nu, "bytes_each_way": nbytes},
        "swap_out_gbs": round(gbs_out, 2), "swap_in_gbs": round(gbs_in, 2),
        "swap_out_ms": round(ms_out, 4), "swap_in_ms": round(ms_in, 4),
        "round_trip_bit_exact": exact,
        "roofline": {"bound": "host-link", "achieved": round(max(gbs_out, gbs_in), 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(max(gbs_out, gbs_in) / HOST_LINK_PEAK_GBS, 4),
                     "traffic": None, "kernel": "swap_blocks_kernel"},
    }
    print(json.dumps(rec), flush=True)
    return 0


def multi_kernel_bytes(w) -> int:
    """Algorithmic bytes of one pa_decode_multi: the K/V of exactly
    context_len tokens per sequence (once), the query rows read and output
    rows written, the table entries, and the per-(row, head, partition)
    states written by the partitions and read by the reduce."""
    Q, H, D = w.query.shape
    n = w.context_lens.astype(np.int64)
    cu = w.info["cu_seqlens_q"]
    P = w.partition_size
    table = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
    parts = 0
    for i in range(w.num_seqs):
        T = int(cu[i + 1] - cu[i])
        pos = int(n[i]) - T + np.arange(T)
        parts += int((pos // P + 1).sum())
    return kv_bytes(w) + 2 * Q * H * D * 2 + table + 2 * parts * H * (D + 2) * 4


def multi_bench(args, w, dev) -> int:
    """Steps of several query tokens per sequence: slot mapping + cache write
    of every sequence's chunk, then pa_decode_multi_balanced (one kernel)
    when each sequence's rows x heads fit 16 columns, else pa_decode_multi
    (partitions + reduce); the partition path's step is reported beside."""
    import torch
    import paged_kv_cache_120_amd as pa
    from paged_kv_cache_120_amd import runner
    base = runner.upload_multi(w, dev)
    runner.apply_history(w, base)
    steps = [base] + [runner.upload_multi(w, dev, pool=base.pool.clone())
                      for _ in range(1, max(1, args.rotate))]
    torch.cuda.synchronize()
    R = len(steps)

    def full(st):
        runner.write_step(st)
        runner.multi_step(st)

    def timed(fn):
        for i in range(args.warmup):
            fn(steps[i % R])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(steps[i % R])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_step = timed(full)
    kms = timed(runner.multi_step)
    balanced = steps[0].multi_grid > 0
    ms_part = timed(lambda st: (runner.write_step(st), runner.multi_step(st, balanced=False)))
    full(steps[(args.steps - 1) % R])
    torch.cuda.synchronize()
    Q = int(w.query.shape[0])
    kvb = kv_bytes(w)
    if balanced:
        # the balanced kernel: K/V once, query rows in, outputs out, table,
        # and the states of cut pairs (written, read back) for the rows x
        # heads in use
        n = w.context_lens.astype(np.int64)
        table = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
        cols = Q / w.num_seqs * w.group
        kb = int(kvb + 2 * Q * w.num_heads * w.head_size * 2 + table
                 + 2 * balanced_split_ranges(w, steps[0].multi_grid) * cols
                 * (w.head_size + 2) * 4)
        kname = "balanced_kernel (multi-token rows)"
    else:
        kb = multi_kernel_bytes(w)
        kname = "multi_kernel + multi_reduce_kernel"
    achieved = kb / (kms * 1e-3) / 1e9
    rec = {
        "metric": "paged multi-token (speculative verify) KV GB/s + query tokens/s",
        "value": round(kvb / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config,
                   "num_seqs": w.num_seqs, "query_tokens": Q, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size, "partition_size": w.partition_size,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "rotated_pool_copies": R, "seed": w.seed},
        "accumulate": "f32", "kv_bytes_per_step": kvb,
        "query_tokens_per_s": round(Q / (ms_step * 1e-3), 1),
        "partition_path_step_ms": round(ms_part, 5),
        "pct_hbm_peak": round(100 * kvb / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": kname,
                     "kernel_ms": round(kms, 5), "algorithmic_bytes": kb},
    }
    if not args.no_cpu_baseline:
        import oracle
        gpu = steps[(args.steps - 1) % R].out.cpu().numpy().astype(np.float64)
        kc, vc = w.pool_init[0].copy(), w.pool_init[1].copy()
        oracle.apply_phases(kc, vc, list(w.history), w.block_size)
        cu = w.info["cu_seqlens_q"]
        try:
            from threadpoolctl import threadpool_limits
            ctx = threadpool_limits(1)
        except Exception:                               # pragma: no cover
            ctx = None
        t0 = time.perf_counter()
        done, rows = 0, 0
        while time.perf_counter() - t0 < 10.0 and done < w.num_seqs:
            oracle.apply_phases(kc, vc, [w.step_write], w.block_size)
            i = done
            o = oracle.decode_multi(w.query[cu[i]:cu[i + 1]], kc, vc, w.block_tables[i:i + 1],
                                    np.array([0, cu[i + 1] - cu[i]], np.int32),
                                    w.context_lens[i:i + 1], w.scale)
            err = np.abs(gpu[cu[i]:cu[i + 1]] - o)
            ok = bool(((err <= 2e-3) | (err <= 1e-2 * np.abs(o))).all())
            rec.setdefault("parity", {"rows_checked": 0, "within_tolerance": True})
            rec["parity"]["rows_checked"] += int(cu[i + 1] - cu[i])
            rec["parity"]["within_tolerance"] &= ok
            rows += int(cu[i + 1] - cu[i])
            done += 1
        el = time.perf_counter() - t0
        if ctx is not None:
            ctx.__exit__(None, None, None)
        rec["cpu_baseline"] = {"value": round(rows / el, 3), "unit": "query tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{done} sequences' query chunks ({rows} rows), "
                                         f"float64 NumPy, 1 BLAS thread"}
    print(json.dumps(rec), flush=True)
    return 0


def fp8_scales(w):
    """Per-tensor scales mapping the largest |K| and |V| the workload writes
    to 448, the largest finite e4m3 magnitude."""
    rows = [p for p in w.history if hasattr(p, "seq")] + [w.step_write]
    ka = max(float(np.abs(p.key.astype(np.float32)).max(initial=0)) for p in rows)
    va = max(float(np.abs(p.value.astype(np.float32)).max(initial=0)) for p in rows)
    return ka / 448.0, va / 448.0


def fp8_bench(args, w, dev) -> int:
    """Decode over an fp8 (e4m3) pool: COW copies, slot mapping,
    pa_cache_write_fp8 of the new tokens, then pa_decode_balanced_fp8; the
    one-kernel pa_decode_step_fp8 step is timed too (fused_step_ms)."""
    import torch
    from paged_kv_cache_120_amd import runner
    ks, vs = fp8_scales(w)
    base = runner.upload_fp8(w, ks, vs, dev)
    runner.apply_history_fp8(w, base)
    steps = [base]
    for _ in range(1, max(1, args.rotate)):
        st = runner.upload_fp8(w, ks, vs, dev)
        st.pool = base.pool.clone()
        steps.append(st)
    torch.cuda.synchronize()
    R = len(steps)

    def timed(fn):
        for i in range(args.warmup):
            fn(steps[i % R])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(steps[i % R])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # the step as two launches (fp8 cache write, then the decode) is timed;
    # the one-kernel step (pa_decode_step_fp8) is reported beside it
    ms_step = timed(lambda st: runner.fp8_step(st, fused=False))
    ms_fused = timed(runner.fp8_step)
    kms = timed(runner.fp8_decode)
    runner.fp8_step(steps[(args.steps - 1) % R], fused=False)
    torch.cuda.synchronize()
    kvb = kv_bytes(w) // 2                         # one byte per element
    S, H, D = w.query.shape
    kb = balanced_kernel_bytes(w, steps[0].grid, False) - kv_bytes(w) // 2
    achieved = kb / (kms * 1e-3) / 1e9
    value = kvb / (ms_step * 1e-3) / 1e9
    rec = {
        "metric": "paged decode over an fp8 (e4m3) KV cache: KV GB/s + seqs/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 math on fp8 (e4m3) KV",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config,
                   "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "k_scale": ks, "v_scale": vs, "rotated_pool_copies": R,
                   "seed": w.seed, "balanced_grid": steps[0].grid},
        "accumulate": "f32", "kv_bytes_per_step": kvb,
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "fused_step_ms": round(ms_fused, 5),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "balanced_kernel (fp8 KV)",
                     "kernel_ms": round(kms, 5), "algorithmic_bytes": kb},
    }
    if not args.no_cpu_baseline:
        import oracle
        gpu = steps[(args.steps - 1) % R].out.cpu().numpy().astype(np.float64)
        kc = (w.pool_init[0] & 0xFF).astype(np.uint8)
        vc = (w.pool_init[1] & 0xFF).astype(np.uint8)
        oracle.apply_phases_fp8(kc, vc, list(w.history), w.block_size, ks, vs)
        try:
            from threadpoolctl import threadpool_limits
            ctx = threadpool_limits(1)
        except Exception:                               # pragma: no cover
            ctx = None
        t0 = time.perf_counter()
        done, ok = 0, True
        while time.perf_counter() - t0 < 10.0 and done < w.num_seqs:
            oracle.apply_phases_fp8(kc, vc, [w.step_copies, w.step_write], w.block_size,
                                    ks, vs)
            i = done
            o = oracle.decode_fp8(w.query[i:i + 1], kc, vc, w.block_tables[i:i + 1],
                                  w.context_lens[i:i + 1], w.scale, ks, vs)[0]
            err = np.abs(gpu[i] - o)
            ok &= bool(((err <= 2e-3) | (err <= 1e-2 * np.abs(o))).all())
            done += 1
        el = time.perf_counter() - t0
        if ctx is not None:
            ctx.__exit__(None, None, None)
        rec["parity"] = {"seqs_checked": done, "within_tolerance": ok}
        rec["cpu_baseline"] = {"value": round(done / el, 3), "unit": "seqs/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{done} sequence decodes over the fp8 pool (cache "
                                         f"write of the step's tokens each), float64 "
                                         f"NumPy, 1 BLAS thread"}
    print(json.dumps(rec), flush=True)
    return 0


def prefix_kernel_bytes(w, groups) -> int:
    """Algorithmic bytes of one pa_decode_shared_prefix: K/V of each group's
    shared partitions once, the rest of every sequence's context once, the
    query and output, and the per-(sequence, head, partition) states written
    and read back by the reduce."""
    S, H, D = w.query.shape
    P = w.partition_size
    n = w.context_lens.astype(np.int64)
    off, mem, blk = groups
    shared = np.zeros(S, np.int64)
    row = 2 * w.num_kv_heads * D * 2
    kv = 0
    for j in range(len(blk)):
        t = int(blk[j]) * w.block_size // P * P
        ms = mem[off[j]:off[j + 1]]
        kv += min(t, int(n[ms].max())) * row
        for m in ms:
            shared[m] = min(t, int(n[m]))
    kv += int((n - shared).sum()) * row
    parts = int(((n + P - 1) // P).sum())
    return kv + 2 * S * H * D * 2 + 2 * parts * H * (D + 2) * 4


def prefix_bench(args, w, dev) -> int:
    """Decode with shared prefixes read once per group: COW copies + slot
    mapping + cache write, then pa_decode_shared_prefix."""
    import torch
    from paged_kv_cache_120_amd import runner
    base = runner.upload_prefix(w, dev)
    runner.apply_history(w, base)
    steps = [base] + [runner.upload_prefix(w, dev, pool=base.pool.clone())
                      for _ in range(1, max(1, args.rotate))]
    torch.cuda.synchronize()
    R = len(steps)

    def timed(fn):
        for i in range(args.warmup):
            fn(steps[i % R])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(steps[i % R])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_step = timed(runner.prefix_step)
    kms = timed(runner.prefix_decode)
    runner.prefix_step(steps[(args.steps - 1) % R])
    torch.cuda.synchronize()
    groups = runner.prefix_groups(w.block_tables, w.context_lens, w.block_size)
    kvb = kv_bytes(w)
    kb = prefix_kernel_bytes(w, groups)
    achieved = kb / (kms * 1e-3) / 1e9
    rec = {
        "metric": "paged decode with shared prefixes: logical KV GB/s + seqs/s",
        "value": round(kvb / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config,
                   "num_seqs": w.num_seqs, "groups": int(len(groups[2])),
                   "shared_blocks": [int(x) for x in groups[2][:4]],
                   "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "head_size": w.head_size, "block_size": w.block_size,
                   "partition_size": w.partition_size,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "rotated_pool_copies": R, "seed": w.seed},
        "accumulate": "f32", "kv_bytes_per_step_logical": kvb,
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "prefix_kernel + partition_kernel + reduce_kernel",
                     "kernel_ms": round(kms, 5), "algorithmic_bytes": kb},
    }
    if not args.no_cpu_baseline:
        parity, cpu = cpu_baseline(w, steps[(args.steps - 1) % R].out.cpu().numpy())
        rec["parity"], rec["cpu_baseline"] = parity, cpu
    print(json.dumps(rec), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="fused",
                    choices=["fused", "balanced", "splitk", "single", "swap", "multi",
                             "fp8", "prefix"],
                    help="fused: pa_decode_step (append + balanced decode, one kernel); "
                         "balanced/splitk/single: slot mapping + cache write + that decode; "
                         "swap: pa_swap_blocks of the batch's blocks to pinned host memory "
                         "and back (its own JSON line); multi: cache write of each "
                         "sequence's query chunk + pa_decode_multi (the *_spec4 configs); "
                         "fp8: fp8 cache write + pa_decode_balanced_fp8 over an e4m3 "
                         "pool, the one-kernel pa_decode_step_fp8 beside it (its own "
                         "JSON line); prefix: writes + "
                         "pa_decode_shared_prefix (c4; its own JSON line)")
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--partition", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", type=int, default=0, metavar="PAIRS",
                    help="after timing, copy PAIRS unreferenced blocks with "
                         "pa_copy_blocks (known bytes) to calibrate HBM counters")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(decode shards by sequence or by KV head with no exchange between "
              "GPUs). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import workloads
    from paged_kv_cache_120_amd import runner

    w = workloads.make(args.config)
    w.partition_size = args.partition
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "swap":
        return swap_bench(args, w, dev)
    if args.mode == "fp8":
        return fp8_bench(args, w, dev)
    if args.mode == "prefix":
        return prefix_bench(args, w, dev)
    if args.mode == "multi" or "cu_seqlens_q" in w.info:
        if args.mode != "multi" or "cu_seqlens_q" not in w.info:
            print("--mode multi goes with a multi-token config (c2_spec4, c3_spec4)",
                  file=sys.stderr)
            return 2
        return multi_bench(args, w, dev)

    steps = []
    base = runner.upload(w, dev)
    runner.apply_history(w, base)
    torch.cuda.synchronize()
    steps.append(base)
    for _ in range(1, max(1, args.rotate)):
        st = runner.upload(w, dev, pool=base.pool.clone())
        steps.append(st)
    torch.cuda.synchronize()

    R = len(steps)
    for i in range(args.warmup):
        runner.full_step(steps[i % R], mode=args.mode)
    torch.cuda.synchronize()

    # pass 1: whole steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        runner.full_step(steps[i % R], mode=args.mode)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # pass 2: the dominant kernel alone, launched back to back over the same
    # rotated inputs, between one pair of events on the launch stream
    import paged_kv_cache_120_amd as pa

    def dominant(st):
        if args.mode == "splitk":
            pa.pa_decode_splitk(st.query, st.key_cache, st.value_cache, st.block_tables,
                                st.context_lens, st.scale, st.partition_size, st.workspace)
        else:
            runner.decode_step(st, "fused_only" if args.mode == "fused" else args.mode)

    for i in range(min(args.warmup, 4)):
        dominant(steps[i % R])
    e2 = torch.cuda.Event(enable_timing=True)
    e3 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e2.record()
    for i in range(args.steps):
        dominant(steps[i % R])
    e3.record()
    torch.cuda.synchronize()
    kms = e2.elapsed_time(e3) / args.steps
    # leave the outputs of a full step for the parity check
    runner.full_step(steps[(args.steps - 1) % R], mode=args.mode)
    torch.cuda.synchronize()

    calib = None
    if args.calibrate:
        # a plain copy of known size for scaling HBM counters: pa_copy_blocks
        # of K contiguous blocks onto the next K in a scratch pool of this
        # layer's block shape (K and V halves), outside the timed region
        k = int(args.calibrate)
        cal = torch.zeros((2, 2 * k) + tuple(steps[0].pool.shape[2:]),
                          dtype=torch.float16, device=dev)
        src = torch.arange(0, k, dtype=torch.int32, device=dev)
        dst = torch.arange(k, 2 * k, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        pa.pa_copy_blocks(cal[0], cal[1], src, dst)
        torch.cuda.synchronize()
        blk = w.block_size * w.num_kv_heads * w.head_size * 2
        calib = {"kernel": "copy_blocks_kernel", "pairs": k,
                 "read_bytes": int(2 * k * blk), "write_bytes": int(2 * k * blk)}
        del cal

    kvb = kv_bytes(w)
    if args.mode == "splitk":
        kb, kname = split_kernel_bytes(w), "partition_kernel (split-KV)"
    elif args.mode == "single":
        kb, kname = single_kernel_bytes(w), "partition_kernel (single pass)"
    else:
        kb = balanced_kernel_bytes(w, steps[0].grid, args.mode == "fused")
        kname = "balanced_kernel" + (" (fused append)" if args.mode == "fused" else "")
    if args.mode == "single":
        kname = "partition_kernel (single pass)"
    achieved = kb / (kms * 1e-3) / 1e9
    value = kvb / (ms_step * 1e-3) / 1e9

    gpu_out = steps[(args.steps - 1) % R].out.cpu().numpy()
    traffic = load_traffic(args, ROOT)
    probe = stream_probe(dev)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.config], "name": args.config,
            "num_seqs": w.num_seqs, "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
            "block_size": w.block_size, "num_blocks": w.num_blocks,
            "total_context_tokens": int(w.context_lens.sum()),
            "decode": args.mode, "partition_size": args.partition,
            "rotated_pool_copies": R, "seed": w.seed,
            "balanced_grid": steps[0].grid,
        },
        "accumulate": "f32",
        "kv_bytes_per_step": kvb,
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "pct_stream_probe": round(100 * value / probe["gbs"], 2),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": kname,
            "kernel_ms": round(kms, 5), "algorithmic_bytes": kb,
            "frac_of_stream_probe": round(achieved / probe["gbs"], 4),
        },
        "stream_probe": probe,
    }
    counters = load_counters(args, ROOT)
    if counters:
        rec["counters"] = counters
    if calib:
        rec["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        rec["parity"], rec["cpu_baseline"] = cpu_baseline(w, gpu_out)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

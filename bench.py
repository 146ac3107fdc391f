#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one pass of the whole decode path over one batch: slot mapping of
the new tokens, the cache write, then decode.  Default (--mode fused):
pa_decode_step, where the balanced split-KV kernel also derives each new
token's slot and writes its K/V.  Other modes run pa_slot_mapping +
pa_cache_write and then balanced, fixed-partition split-KV (+ reduce) or
single-pass decode.  Inputs are seeded synthetic workloads already resident
in HBM.  Timed steps rotate over --rotate copies of the pool so repeated
reads cannot be served by the 256 MB MALL or L2.

Prints ONE JSON line.  ``value`` is KV GB/s of the headline workload (the
Llama-2-13B layer, c2): the KV bytes the step must read (exactly
context_len tokens per sequence, K and V) over the step time.  ``roofline``
rates the dominant kernel against HBM peak with the method's bytes over its
event-timed duration; the partial states that cut (sequence, kv head) pairs
hand between workgroups are reported beside, as ``handoff_bytes``, and are
not counted as algorithmic.  With the default configuration the line also
carries ``gqa_c3`` (the GQA decode workload, same measurements and parity
on every sequence), ``long_c5`` (long-context decode in the fixed 512-token
split-K form the workload names, beside the one-kernel form),
``paging_overhead`` (the same decodes on a contiguous identity block table)
and ``context`` (the pages' own system-level figures).  ``cpu_baseline`` is
the float64 CPU oracle timed on the machine's host cores (all of them, and one),
before the GPU is touched.
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
    "c3_chunk512": "chunked prefill, the last 512 tokens of each seq as the chunk: GQA 32/8 "
                   "heads, 16 seqs ctx U[512,4096], D128, B16",
}
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix throughput


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


PAIR_COST = 128      # flat units the balanced split charges per (sequence, kv head)
FULL_PAIR_COST = 160  # the same for the 16-column multi-token form


def multi_full_form(w, max_q: int) -> bool:
    """Whether the balanced multi-token kernel takes its 16-column form:
    max_q * g query columns beyond what one narrow pass holds (4 at head
    size 128 with g <= 4, else 8)."""
    narrow = 4 if (w.head_size == 128 and w.group <= 4) else 8
    return max_q * w.group > narrow


def balanced_split_ranges(w, grid: int, pair_cost: int = PAIR_COST) -> int:
    """Ranges of the balanced decode that belong to (sequence, kv head)
    pairs cut across several workgroups: each stores one partial state per
    query head, which the pair's last workgroup reads back to merge.  Same
    slicing as the kernel: a pair spans pair_cost units, then its length
    padded to 16; equal 16-aligned slices of that space (one column tile per
    pair)."""
    M = w.max_blocks_per_seq * w.block_size
    n = np.minimum(w.context_lens.astype(np.int64), M)
    pad = np.where(n > 0, (n + 15) // 16 * 16, 0)
    span = np.where(pad > 0, pad + pair_cost, 0)
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
            F = int(prefix[i]) * Hkv + kvh * int(span[i]) + pair_cost
            k = (F + int(n[i]) - 1) // C - F // C + 1
            if k > 1:
                count += k
    return count


def balanced_kernel_bytes(w, grid: int, fused: bool) -> int:
    """Algorithmic bytes of one balanced-kernel launch, the method's own:
    KV rows of exactly context_len tokens, query, table entries, output and,
    for the fused step, this step's K/V rows (read and written) and the
    slots.  The partial states of cut pairs are the kernel's, not the
    method's: see balanced_handoff_bytes."""
    S, H, D = w.query.shape
    n = w.context_lens.astype(np.int64)
    table = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
    extra = (2 * 2 * S * w.num_kv_heads * D * 2 + S * 4) if fused else 0
    return kv_bytes(w) + 2 * S * H * D * 2 + table + extra


def decode_pair_cost(w, fp8: bool = False) -> int:
    """The balanced decode's flat units per pair: 192 for the fp16 g = 4
    matrix-core body at head size 128, else PAIR_COST."""
    return 192 if (not fp8 and w.group == 4 and w.head_size == 128) else PAIR_COST


def balanced_handoff_bytes(w, grid: int, fp8: bool = False) -> int:
    """Bytes of the partial states that cut (sequence, kv head) pairs hand
    between workgroups in one balanced-kernel launch: each range of a cut
    pair writes g (max, sum, out[D]) fp32 states and the merging range reads
    them back."""
    return (2 * balanced_split_ranges(w, grid, decode_pair_cost(w, fp8)) * w.group
            * (w.head_size + 2) * 4)


def single_kernel_bytes(w) -> int:
    S, H, D = w.query.shape
    n = w.context_lens.astype(np.int64)
    table = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
    return kv_bytes(w) + 2 * S * H * D * 2 + table


def _parity(gpu_out, ref) -> dict:
    """Elementwise tolerance check of GPU outputs against the oracle."""
    got = np.asarray(gpu_out, np.float64)
    err = np.abs(got - ref)
    return {"seqs_checked": int(ref.shape[0]), "max_abs_err": float(err.max()),
            "within_tolerance": bool(((err <= 2e-3) | (err <= 1e-2 * np.abs(ref))).all())}


def cpu_baseline(w, gpu_out=None, min_s: float = 10.0, max_s: float = 30.0):
    """The oracle (unchanged) on one host core: cache write of the step's
    tokens plus float64 decode of the whole batch, repeated until >= min_s.
    The first pass's outputs are also compared with ``gpu_out`` (one of the
    timed GPU steps) when it is given.  Used by the secondary modes, which
    run it after the GPU work."""
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
        parity = _parity(np.asarray(gpu_out)[idx], np.stack([first[i] for i in idx]))
    return parity, {
        "value": round(seqs / el, 3), "unit": "seqs/s", "cores": 1, "kind": "oracle",
        "kv_gbs_equiv": round(kv_bytes(w) * frac / el / 1e9, 4),
        "seconds": round(el, 2),
        "sample": (f"{seqs} sequence decodes ({frac:.2f} passes over the {w.num_seqs}-seq "
                   f"batch, cache write of its new tokens per pass), float64 NumPy, "
                   f"1 BLAS thread"),
    }


# State the forked oracle workers read (set in the parent before the fork).
_ORACLE = {}


def _oracle_worker(job):
    """One worker of the host-core oracle baseline: starting at sequence
    ``first``, decode the batch's sequences in turn -- each pass begins with
    the cache write of the step's new tokens -- until ``seconds`` have
    passed.  Returns (decodes done, KV bytes read, {seq: first output})."""
    first, seconds = job
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:                                   # pragma: no cover
        pass
    import oracle
    w, kc, vc = _ORACLE["w"], _ORACLE["kc"], _ORACLE["vc"]
    row = 2 * w.num_kv_heads * w.head_size * 2
    done, nbytes, outs = 0, 0, {}
    t0 = time.perf_counter()
    i = first % w.num_seqs
    while True:
        if i == first % w.num_seqs:
            oracle.apply_phases(kc, vc, [w.step_copies, w.step_write], w.block_size)
        o = oracle.decode(w.query[i:i + 1], kc, vc, w.block_tables[i:i + 1],
                          w.context_lens[i:i + 1], w.scale)
        outs.setdefault(i, o[0])
        done += 1
        nbytes += int(w.context_lens[i]) * row
        i = (i + 1) % w.num_seqs
        if time.perf_counter() - t0 >= seconds:
            break
    return done, nbytes, outs


def host_cores() -> dict:
    """Host cores this process may use: the affinity mask, os.cpu_count(),
    and the workers used (the affinity count, at most 16: one GPU's share of
    the host)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:                              # pragma: no cover
        aff = os.cpu_count() or 1
    return {"sched_getaffinity": aff, "os_cpu_count": os.cpu_count(),
            "workers": max(1, min(aff, 16))}


def cpu_baseline_cores(w, seconds: float = 10.0, single_seconds: float = 5.0):
    """The oracle (unchanged) timed on the host: first on one core, then on
    every usable core (a process pool over sequences, one BLAS thread per
    worker).  Must run before the GPU is initialised: the workers are
    forked.  Returns (oracle outputs of every sequence, record)."""
    import multiprocessing as mp
    import oracle
    kc = w.pool_init[0].copy()
    vc = w.pool_init[1].copy()
    oracle.apply_phases(kc, vc, list(w.history), w.block_size)
    _ORACLE.update(w=w, kc=kc, vc=vc)
    cores = host_cores()
    ctx = mp.get_context("fork")
    # one core (in a worker, so the parent keeps its thread settings)
    with ctx.Pool(1) as pool:
        t0 = time.perf_counter()
        d1, b1, outs = pool.map(_oracle_worker, [(0, single_seconds)])[0]
        el1 = time.perf_counter() - t0
    n = cores["workers"]
    with ctx.Pool(n) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_worker, [(k * w.num_seqs // n, seconds) for k in range(n)])
        eln = time.perf_counter() - t0
    _ORACLE.clear()
    dn = sum(r[0] for r in res)
    bn = sum(r[1] for r in res)
    for r in res:
        for i, o in r[2].items():
            outs.setdefault(i, o)
    missing = [i for i in range(w.num_seqs) if i not in outs]
    for i in missing:                                   # rarely: a very short run
        outs[i] = oracle.decode(w.query[i:i + 1], kc, vc, w.block_tables[i:i + 1],
                                w.context_lens[i:i + 1], w.scale)[0]
    ref = np.stack([outs[i] for i in range(w.num_seqs)])
    rec = {
        "value": round(dn / eln, 3), "unit": "seqs/s", "cores": n, "kind": "oracle",
        "kv_gbs_equiv": round(bn / eln / 1e9, 4), "seconds": round(eln, 2),
        "single_core_value": round(d1 / el1, 3),
        "single_core_kv_gbs_equiv": round(b1 / el1 / 1e9, 4),
        "sched_getaffinity": cores["sched_getaffinity"],
        "os_cpu_count": cores["os_cpu_count"],
        "sample": (f"{dn} sequence decodes of the {w.num_seqs}-seq batch over {n} worker "
                   f"processes (each pass starting with the cache write of the step's new "
                   f"tokens), float64 NumPy, one BLAS thread per worker, ~{seconds:.0f} s; "
                   f"single core: {d1} decodes in {el1:.1f} s"),
    }
    return ref, rec


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


def _summary(path: str) -> dict:
    t = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                t[k.strip()] = v.strip()
    return t


def load_traffic(config: str, mode: str, partition: int, root: str):
    """HBM bytes per launch of the decode kernel, from the committed
    rocprofv3 counter summary (FETCH_SIZE / WRITE_SIZE scaled by a copy of
    known size) for this workload and mode, if it was taken on the current
    kernel sources (else None).  Returns {"bytes", "source"}."""
    rel = f"profiles/decode_{config}_{mode}_traffic.txt"
    path = os.path.join(root, rel)
    if not os.path.exists(path):
        return None
    t = _summary(path)
    if t.get("kernel_source_sha256_16") != kernel_source_hash(root) or \
            t.get("partition_size") != str(partition):
        return None
    try:
        return {"bytes": int(float(t["hbm_bytes_per_launch"])),
                "source": f"{rel} (rocprofv3 --pmc on these kernel sources)"}
    except (KeyError, ValueError):
        return None


def load_counters(config: str, mode: str, root: str):
    """Per-launch hardware counters of the decode kernel (L2 hit rate, LDS
    bank conflicts, matrix-core and vector instructions) from the committed
    rocprofv3 summary for this workload and mode, if it was taken on the
    current kernel sources (else None)."""
    rel = f"profiles/decode_{config}_{mode}_counters.txt"
    path = os.path.join(root, rel)
    if not os.path.exists(path):
        return None
    t = _summary(path)
    if t.pop("kernel_source_sha256_16", None) != kernel_source_hash(root):
        return None
    out = {}
    for k, v in t.items():
        try:
            out[k] = float(v)
        except ValueError:
            continue
    if out:
        out["source"] = f"{rel} (rocprofv3 --pmc on these kernel sources)"
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


def stream_probe_sized(dev, nbytes: int, launches: int = 20) -> dict:
    """Read rate of one plain sequential pass over nbytes (rounded up to 16),
    the byte count of one decode launch: the same launch start, ramp and
    tail at that size, with no paging, softmax or handoff.  Successive
    launches read up to 4 disjoint regions in turn (as many as fit in 4 GiB)
    so the 256 MB MALL cannot serve a repeat; best of 1, 2, 4 and 8
    workgroups per CU, timed with events on the current stream."""
    import torch
    import paged_kv_cache_120_amd as pa
    n = (int(nbytes) + 15) // 16 * 16
    k = max(1, min(4, PROBE_BYTES // n))
    buf = torch.zeros(k * n, dtype=torch.uint8, device=dev)
    regions = [buf[i * n:(i + 1) * n] for i in range(k)]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(4 * 8 * cus, dtype=torch.int32, device=dev)
    best = None
    for grid in (cus, 2 * cus, 4 * cus, 8 * cus):
        for i in range(3):
            pa.pa_stream_read(regions[i % k], sink, grid)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(launches):
            pa.pa_stream_read(regions[i % k], sink, grid)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        if best is None or ms < best[1]:
            best = (grid, ms)
    del regions, buf, sink
    torch.cuda.empty_cache()
    grid, ms = best
    gbs = n / (ms * 1e-3) / 1e9
    return {"bytes": n, "regions": k, "grid": grid, "us": round(ms * 1e3, 2),
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def add_same_size_read(rec: dict, dev) -> None:
    """Put a plain read of the dominant kernel's algorithmic bytes beside
    its roofline: the ceiling a kernel moving that many bytes reaches here."""
    rf = rec["roofline"]
    sp = stream_probe_sized(dev, rf["algorithmic_bytes"])
    rf["same_size_read"] = sp
    rf["frac_of_same_size_read"] = round(rf["achieved"] / sp["gbs"], 4)


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


def prefill_flops(w) -> float:
    """Matrix flops of causal attention over the chunk rows: 2*D for the
    score and 2*D for the weighted value of every (row, head, visible key);
    row j of a T-row chunk over n keys sees n - T + j + 1 of them."""
    cu = w.info["cu_seqlens_q"]
    T = np.diff(cu).astype(np.int64)
    n = w.context_lens.astype(np.int64)
    vis = np.where(T > 0, (n - T) * T + T * (T + 1) // 2, 0)
    return 4.0 * w.head_size * w.num_heads * float(vis.sum())


def prefill_bench(args, w, dev) -> int:
    """Chunked prefill steps: slot mapping + cache write of every sequence's
    chunk, then pa_prefill (128 rows x heads per pass over the keys); the
    pa_decode_multi step over the same rows is timed beside it."""
    import torch
    import paged_kv_cache_120_amd as pa
    from paged_kv_cache_120_amd import runner
    base = runner.upload_multi(w, dev)
    runner.apply_history(w, base)
    steps = [base] + [runner.upload_multi(w, dev, pool=base.pool.clone())
                      for _ in range(1, max(1, args.rotate))]
    torch.cuda.synchronize()
    R = len(steps)

    def attend(st):
        pa.pa_prefill(st.out, st.query, st.key_cache, st.value_cache, st.block_tables,
                      st.cu_seqlens_q, st.context_lens, st.max_q, st.scale)

    def timed(fn, steps_n):
        for i in range(args.warmup):
            fn(steps[i % R])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps_n):
            fn(steps[i % R])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps_n

    ms_step = timed(lambda st: (runner.write_step(st), attend(st)), args.steps)
    kms = timed(attend, args.steps)
    ms_multi = timed(lambda st: (runner.write_step(st), runner.multi_step(st, balanced=False)),
                     max(5, args.steps // 10))
    last = steps[(args.steps - 1) % R]
    runner.write_step(last)
    attend(last)
    torch.cuda.synchronize()
    Q = int(w.query.shape[0])
    fl = prefill_flops(w)
    achieved = fl / (kms * 1e-3) / 1e12
    rec = {
        "metric": "paged chunked prefill TFLOP/s + query tokens/s",
        "value": round(fl / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config,
                   "num_seqs": w.num_seqs, "query_tokens": Q, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size,
                   "total_context_tokens": int(w.context_lens.sum()),
                   "rotated_pool_copies": R, "seed": w.seed},
        "accumulate": "f32", "flops_per_step": fl,
        "query_tokens_per_s": round(Q / (ms_step * 1e-3), 1),
        "decode_multi_step_ms": round(ms_multi, 5),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_kernel", "kernel_ms": round(kms, 5),
                     "algorithmic_flops": fl, "kv_bytes": kv_bytes(w)},
    }
    if not args.no_cpu_baseline:
        import oracle
        gpu = last.out.cpu().numpy().astype(np.float64)
        kc, vc = w.pool_init[0].copy(), w.pool_init[1].copy()
        oracle.apply_phases(kc, vc, list(w.history) + [w.step_write], w.block_size)
        cu = w.info["cu_seqlens_q"]
        try:
            from threadpoolctl import threadpool_limits
            ctx = threadpool_limits(1)
        except Exception:                               # pragma: no cover
            ctx = None
        # a bounded sample: the first 32 rows of each sequence's chunk, as
        # many sequences as about 10 s allow
        t0 = time.perf_counter()
        done, rows, ok_all = 0, 0, True
        while time.perf_counter() - t0 < 10.0 and done < w.num_seqs:
            i = done
            T = int(cu[i + 1] - cu[i])
            k = min(T, 32)
            # rows 0..k-1 of a T-row chunk over n keys: as the first k rows
            # of a k-row chunk over n - T + k keys
            o = oracle.decode_multi(w.query[cu[i]:cu[i] + k], kc, vc, w.block_tables[i:i + 1],
                                    np.array([0, k], np.int32),
                                    np.array([w.context_lens[i] - T + k], np.int32), w.scale)
            err = np.abs(gpu[cu[i]:cu[i] + k] - o)
            ok_all &= bool(((err <= 2e-3) | (err <= 1e-2 * np.abs(o))).all())
            rows += k
            done += 1
        el = time.perf_counter() - t0
        if ctx is not None:
            ctx.__exit__(None, None, None)
        rec["parity"] = {"rows_checked": rows, "within_tolerance": ok_all}
        rec["cpu_baseline"] = {"value": round(rows / el, 3), "unit": "query tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the first {min(32, int(np.diff(cu).max()))} rows of "
                                         f"{done} sequences' chunks ({rows} rows x "
                                         f"{w.num_heads} heads), float64 NumPy, 1 BLAS thread"}
    print(json.dumps(rec), flush=True)
    return 0


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
        kb = int(kvb + 2 * Q * w.num_heads * w.head_size * 2 + table)
        pc = FULL_PAIR_COST if multi_full_form(w, steps[0].max_q) else PAIR_COST
        handoff = int(2 * balanced_split_ranges(w, steps[0].multi_grid, pc) * cols
                      * (w.head_size + 2) * 4)
        kname = "balanced_kernel (multi-token rows)"
    else:
        kb = multi_kernel_bytes(w)
        handoff = 0
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
                     "kernel_ms": round(kms, 5), "algorithmic_bytes": kb,
                     "handoff_bytes": handoff},
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
    handoff = balanced_handoff_bytes(w, steps[0].grid, fp8=True)
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
                     "kernel_ms": round(kms, 5), "algorithmic_bytes": kb,
                     "handoff_bytes": handoff},
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


CONTEXT = {
    "note": "the pages' own system-level figures, quoted as context; none is a target "
            "and none was measured here",
    "kv_utilisation": "contiguous allocation 20-40% -> paged about 96% (PagedAttention: "
                      "KV Cache的虚拟内存, 内存碎片化与GPU浪费 and 一图解析, after Kwon et al.)",
    "indirection_overhead": "block-table indirection costs a single-digit percent "
                            "(same page, 一图解析); measured here: paging_overhead",
    "concurrent_requests": "LLaMA-13B on an A100 80GB, input 1024 / output 256: 8 -> 24 "
                           "concurrent requests (PagedAttention原理（下）, §4.4 table)",
}


def _timed(steps, fn, n: int, warm: int) -> float:
    """Mean ms of fn over n launches on the rotated steps (after warm
    untimed ones), between two events on the current stream."""
    import torch
    R = len(steps)
    for i in range(warm):
        fn(steps[i % R])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(steps[i % R])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def upload_rotated(w, dev, rotate: int):
    """The workload on the device with its history replayed, plus
    rotate - 1 copies of the pool (sharing the other inputs' values)."""
    import torch
    from paged_kv_cache_120_amd import runner
    base = runner.upload(w, dev)
    runner.apply_history(w, base)
    torch.cuda.synchronize()
    steps = [base] + [runner.upload(w, dev, pool=base.pool.clone())
                      for _ in range(1, max(1, rotate))]
    torch.cuda.synchronize()
    return steps


def dominant_call(mode: str):
    """The dominant kernel of a step of this mode, launched alone."""
    import paged_kv_cache_120_amd as pa
    from paged_kv_cache_120_amd import runner

    def f(st):
        if mode == "splitk":
            pa.pa_decode_splitk(st.query, st.key_cache, st.value_cache, st.block_tables,
                                st.context_lens, st.scale, st.partition_size, st.workspace)
        else:
            runner.decode_step(st, "fused_only" if mode == "fused" else mode)
    return f


def decode_measure(w, steps, mode: str, n: int, warm: int) -> dict:
    """Whole steps, then the dominant kernel alone, over the rotated steps;
    leaves the outputs of one full step in steps[(n - 1) % R].out."""
    import torch
    from paged_kv_cache_120_amd import runner
    ms = _timed(steps, lambda st: runner.full_step(st, mode=mode), n, warm)
    kms = _timed(steps, dominant_call(mode), n, min(warm, 4))
    last = steps[(n - 1) % len(steps)]
    runner.full_step(last, mode=mode)
    torch.cuda.synchronize()
    return {"ms_step": ms, "kms": kms, "out": last.out.cpu().numpy()}


def decode_record(w, mode: str, grid: int, ms_step: float, kms: float) -> dict:
    """Step rate, KV rate and the dominant kernel's roofline for one decode
    workload.  ``algorithmic_bytes`` are the method's bytes (frac uses only
    these); the balanced kernel's partial-state handoff is reported apart."""
    kvb = kv_bytes(w)
    handoff = 0
    if mode == "splitk":
        kb, kname = split_kernel_bytes(w), "partition_kernel (split-KV)"
    elif mode == "single":
        kb, kname = single_kernel_bytes(w), "partition_kernel (single pass)"
    else:
        kb = balanced_kernel_bytes(w, grid, mode == "fused")
        handoff = balanced_handoff_bytes(w, grid)
        kname = "balanced_kernel" + (" (fused append)" if mode == "fused" else "")
    achieved = kb / (kms * 1e-3) / 1e9
    value = kvb / (ms_step * 1e-3) / 1e9
    return {
        "ms_per_step": round(ms_step, 5), "kv_bytes_per_step": kvb,
        "kv_gbs": round(value, 2), "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": kname, "kernel_ms": round(kms, 5),
                     "algorithmic_bytes": kb, "handoff_bytes": handoff},
    }


def contiguous_steps(w, steps, dev):
    """The same batch on an identity block table: sequence i's logical
    blocks are physical blocks off_i, off_i + 1, ... (sequences laid end to
    end), holding the same K/V bits as the paged pool.  One contiguous pool
    per rotated step."""
    import dataclasses
    import torch
    B, M = w.block_size, w.max_blocks_per_seq
    n = np.minimum(np.maximum(w.context_lens.astype(np.int64), 0), M * B)
    nb = (n + B - 1) // B
    off = np.concatenate([[0], np.cumsum(nb)[:-1]])
    bt = np.zeros_like(w.block_tables)
    src, dst = [], []
    for i in range(w.num_seqs):
        k = int(nb[i])
        bt[i, :k] = off[i] + np.arange(k)
        src.append(w.block_tables[i, :k])
        dst.append(off[i] + np.arange(k))
    src_t = torch.from_numpy(np.concatenate(src).astype(np.int64)).to(dev)
    dst_t = torch.from_numpy(np.concatenate(dst).astype(np.int64)).to(dev)
    total = max(int(nb.sum()), w.num_blocks)
    bt_dev = torch.from_numpy(bt).to(dev)
    out = []
    for st in steps:
        pool = torch.zeros((2, total) + tuple(st.pool.shape[2:]), dtype=st.pool.dtype,
                           device=dev)
        pool[:, dst_t] = st.pool[:, src_t]
        wr = dataclasses.replace(st.write, table=bt_dev,
                                 slots=torch.empty_like(st.write.slots))
        out.append(dataclasses.replace(st, pool=pool, block_tables=bt_dev, write=wr,
                                       out=torch.empty_like(st.out),
                                       bal_workspace=torch.zeros_like(st.bal_workspace)))
    torch.cuda.synchronize()
    return out


def paging_overhead(w, steps, dev, n: int) -> dict:
    """The fused step's kernel on the workload's scattered block table and on
    an identity table with the same K/V bits (alternated, best of two runs
    each); outputs must agree bit for bit."""
    import torch
    from paged_kv_cache_120_amd import runner
    contig = contiguous_steps(w, steps, dev)
    f = dominant_call("fused")
    paged_ms, contig_ms = [], []
    for _ in range(2):
        paged_ms.append(_timed(steps, f, n, 4))
        contig_ms.append(_timed(contig, f, n, 4))
    f(steps[0])
    f(contig[0])
    torch.cuda.synchronize()
    same = bool(torch.equal(steps[0].out.view(torch.int16), contig[0].out.view(torch.int16)))
    p, c = min(paged_ms), min(contig_ms)
    del contig
    torch.cuda.empty_cache()
    return {"paged_kernel_ms": round(p, 5), "contiguous_kernel_ms": round(c, 5),
            "overhead_pct": round(100 * (p - c) / c, 2), "outputs_bit_identical": same,
            "contiguous": "identity block table: each sequence's blocks consecutive, "
                          "sequences end to end, same K/V bits and kernel"}


def long_context_record(name: str, args, dev) -> dict:
    """Long-context decode in the form the workload names (fixed 512-token
    split-K partitions + reduce, with the cache write) beside the one-kernel
    fused step."""
    import torch
    import workloads
    w = workloads.make(name)
    w.partition_size = 512
    steps = upload_rotated(w, dev, args.rotate)
    n = max(10, args.steps // 4)
    sk = decode_measure(w, steps, "splitk", n, min(args.warmup, 5))
    fu = decode_measure(w, steps, "fused", n, min(args.warmup, 5))
    grid = steps[0].grid
    del steps
    torch.cuda.empty_cache()
    fused = decode_record(w, "fused", grid, fu["ms_step"], fu["kms"])
    add_same_size_read(fused, dev)
    return {"workload": WORKLOADS[name], "num_seqs": w.num_seqs,
            "total_context_tokens": int(w.context_lens.sum()), "steps": n,
            "splitk_512": decode_record(w, "splitk", grid, sk["ms_step"], sk["kms"]),
            "fused": fused}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="fused",
                    choices=["fused", "balanced", "splitk", "single", "swap", "multi",
                             "fp8", "prefix", "prefill"],
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
    ap.add_argument("--no-extras", action="store_true",
                    help="only the --config workload (no gqa_c3, long_c5, paging_overhead)")
    ap.add_argument("--calibrate", type=int, default=0, metavar="PAIRS",
                    help="after timing, copy PAIRS unreferenced blocks with "
                         "pa_copy_blocks (known bytes) to calibrate HBM counters")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(decode shards by sequence or by KV head with no exchange between "
              "GPUs). Run with --gpus 1.", file=sys.stderr)
        return 2

    import workloads

    w = workloads.make(args.config)
    w.partition_size = args.partition
    simple = args.mode in ("swap", "fp8", "prefix", "multi") or "cu_seqlens_q" in w.info
    extras = (not simple and not args.no_extras and args.config == "c2"
              and args.mode == "fused")
    w3 = None
    if extras:
        w3 = workloads.make("c3")
        w3.partition_size = args.partition

    # host-core oracle baselines first: their workers are forked, which must
    # happen before this process touches the GPU
    ref, cpu, ref3 = None, None, None
    if not simple and not args.no_cpu_baseline:
        ref, cpu = cpu_baseline_cores(w)
    if w3 is not None:
        import oracle
        kc3, vc3 = w3.pool_init[0].copy(), w3.pool_init[1].copy()
        oracle.apply_phases(kc3, vc3, list(w3.history) + [w3.step_copies, w3.step_write],
                            w3.block_size)
        ref3 = oracle.decode(w3.query, kc3, vc3, w3.block_tables, w3.context_lens, w3.scale)
        del kc3, vc3

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "swap":
        return swap_bench(args, w, dev)
    if args.mode == "fp8":
        return fp8_bench(args, w, dev)
    if args.mode == "prefix":
        return prefix_bench(args, w, dev)
    if args.mode == "prefill":
        if "cu_seqlens_q" not in w.info:
            print("--mode prefill goes with a multi-token config (c3_chunk512)",
                  file=sys.stderr)
            return 2
        return prefill_bench(args, w, dev)
    if args.mode == "multi" or "cu_seqlens_q" in w.info:
        if args.mode != "multi" or "cu_seqlens_q" not in w.info:
            print("--mode multi goes with a multi-token config (c2_spec4, c3_spec4)",
                  file=sys.stderr)
            return 2
        return multi_bench(args, w, dev)

    from paged_kv_cache_120_amd import runner
    import paged_kv_cache_120_amd as pa
    steps = upload_rotated(w, dev, args.rotate)
    R = len(steps)
    for i in range(args.warmup):
        runner.full_step(steps[i % R], mode=args.mode)
    torch.cuda.synchronize()

    # the timed region: exactly --steps whole steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        runner.full_step(steps[i % R], mode=args.mode)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # the dominant kernel alone, launched back to back over the same rotated
    # inputs, between one pair of events on the launch stream
    kms = _timed(steps, dominant_call(args.mode), args.steps, min(args.warmup, 4))
    # leave the outputs of a full step for the parity check
    runner.full_step(steps[(args.steps - 1) % R], mode=args.mode)
    torch.cuda.synchronize()
    gpu_out = steps[(args.steps - 1) % R].out.cpu().numpy()

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

    main_rec = decode_record(w, args.mode, steps[0].grid, ms_step, kms)
    traffic = load_traffic(args.config, args.mode, args.partition, ROOT)
    if traffic is not None:
        main_rec["roofline"]["traffic"] = traffic["bytes"]
        main_rec["roofline"]["traffic_source"] = traffic["source"]
    probe = stream_probe(dev)
    main_rec["roofline"]["frac_of_stream_probe"] = round(
        main_rec["roofline"]["achieved"] / probe["gbs"], 4)
    add_same_size_read(main_rec, dev)

    rec = {
        "metric": METRIC,
        "value": main_rec["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_step"],
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
        "kv_bytes_per_step": main_rec["kv_bytes_per_step"],
        "seqs_per_s": main_rec["seqs_per_s"],
        "pct_hbm_peak": main_rec["pct_hbm_peak"],
        "pct_stream_probe": round(100 * main_rec["kv_gbs"] / probe["gbs"], 2),
        "roofline": main_rec["roofline"],
        "stream_probe": probe,
    }
    counters = load_counters(args.config, args.mode, ROOT)
    if counters:
        rec["counters_from_profile"] = counters
    if calib:
        rec["copy_calibration"] = calib
    if ref is not None:
        rec["parity"] = _parity(gpu_out, ref)
    if extras:
        rec["paging_overhead"] = {"c2": paging_overhead(w, steps, dev, max(20, args.steps // 2))}
    del steps
    torch.cuda.empty_cache()

    if extras:
        # the GQA decode workload, measured the same way
        s3 = upload_rotated(w3, dev, args.rotate)
        m3 = decode_measure(w3, s3, "fused", args.steps, args.warmup)
        r3 = decode_record(w3, "fused", s3[0].grid, m3["ms_step"], m3["kms"])
        t3 = load_traffic("c3", "fused", args.partition, ROOT)
        if t3 is not None:
            r3["roofline"]["traffic"] = t3["bytes"]
            r3["roofline"]["traffic_source"] = t3["source"]
        r3["roofline"]["frac_of_stream_probe"] = round(r3["roofline"]["achieved"] / probe["gbs"], 4)
        add_same_size_read(r3, dev)
        c3c = load_counters("c3", "fused", ROOT)
        gq = {"workload": WORKLOADS["c3"], "num_seqs": w3.num_seqs,
              "num_heads": w3.num_heads, "num_kv_heads": w3.num_kv_heads,
              "total_context_tokens": int(w3.context_lens.sum()), "seed": w3.seed,
              "balanced_grid": s3[0].grid, "decode": "fused", "steps": args.steps, **r3,
              "parity": _parity(m3["out"], ref3)}
        if c3c:
            gq["counters_from_profile"] = c3c
        rec["gqa_c3"] = gq
        rec["paging_overhead"]["c3"] = paging_overhead(w3, s3, dev, max(20, args.steps // 2))
        del s3
        torch.cuda.empty_cache()
        rec["long_c5"] = {n: long_context_record(n, args, dev) for n in ("c5_b32", "c5_b64")}
        rec["context"] = CONTEXT
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Drive one decode step through the library on device tensors.

A step is: copy-on-write block copies (if any), the slot mapping of the new
tokens, the cache write, then decode -- single-pass (``pa_decode``), split
(``pa_decode_splitk`` + ``pa_decode_reduce``) or balanced
(``pa_decode_balanced``); or, mode "fused", copies then ``pa_decode_step``
(slot mapping, cache write and balanced decode in one kernel).  With several
query tokens per sequence (``upload_multi``), ``multi_step`` runs
``pa_decode_multi`` after the same writes.  With an fp8 pool
(``upload_fp8``), ``fp8_step`` runs the copies, ``pa_cache_write_fp8`` and
``pa_decode_balanced_fp8``.  ``upload_prefix`` + ``prefix_step`` run the
writes, then ``pa_decode_shared_prefix`` with groups found by
``prefix_groups``.  Inputs are plain arrays (a
workload object with the attributes used below); this module only uploads
them and calls the binding, so every step runs in the library's kernels.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from . import (pa_balanced_grid, pa_balanced_grid_fp8, pa_balanced_workspace_size,
               pa_cache_write, pa_cache_write_fp8, pa_copy_blocks, pa_decode,
               pa_decode_balanced, pa_decode_balanced_fp8, pa_decode_multi,
               pa_decode_step_fp8, pa_decode_multi_balanced, pa_multi_balanced_grid,
               pa_multi_balanced_workspace_size_tiles,
               pa_decode_reduce, pa_decode_shared_prefix, pa_decode_splitk,
               pa_decode_step, pa_multi_workspace_size, pa_prefix_workspace_size,
               pa_prefill, pa_slot_mapping, pa_splitk_workspace_size)


def _t(a, dev, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev)


@dataclasses.dataclass
class DevWrite:
    table: torch.Tensor
    seq: torch.Tensor
    pos: torch.Tensor
    key: torch.Tensor
    value: torch.Tensor
    slots: torch.Tensor


@dataclasses.dataclass
class DevCopy:
    src: torch.Tensor
    dst: torch.Tensor


@dataclasses.dataclass
class DeviceStep:
    block_size: int
    scale: float
    partition_size: int
    pool: torch.Tensor             # fp16 [2, nb, B, H_kv, D]
    query: torch.Tensor            # fp16 [S, H, D]
    block_tables: torch.Tensor     # int32 [S, M]
    context_lens: torch.Tensor     # int32 [S]
    out: torch.Tensor              # fp16 [S, H, D]
    copies: Optional[DevCopy]
    write: DevWrite
    workspace: torch.Tensor        # uint8 split-KV workspace
    grid: int                      # balanced decode workgroups
    bal_workspace: torch.Tensor    # uint8 balanced decode workspace

    @property
    def key_cache(self):
        return self.pool[0]

    @property
    def value_cache(self):
        return self.pool[1]


def _dev_phase(ph, dev):
    if ph is None:
        return None
    if hasattr(ph, "src"):
        return DevCopy(_t(ph.src, dev), _t(ph.dst, dev))
    n = len(ph.pos)
    return DevWrite(_t(ph.table, dev), _t(ph.seq, dev), _t(ph.pos, dev),
                    _t(ph.key, dev), _t(ph.value, dev),
                    torch.empty(n, dtype=torch.int32, device=dev))


def run_phase(ph, pool, block_size: int, stream=None) -> None:
    if ph is None:
        return
    if isinstance(ph, DevCopy):
        pa_copy_blocks(pool[0], pool[1], ph.src, ph.dst, stream=stream)
        return
    pa_slot_mapping(ph.slots, ph.table, ph.seq, ph.pos, block_size, stream=stream)
    pa_cache_write(ph.key, ph.value, pool[0], pool[1], ph.slots, stream=stream)


def upload_multi(w, device: str = "cuda", pool: Optional[torch.Tensor] = None) -> DeviceStep:
    """As upload, for a workload with several query tokens per sequence
    (``w.info["cu_seqlens_q"]``): adds the row offsets, the largest per-
    sequence query count and the multi-token workspace."""
    st = upload(w, device, pool)
    dev = st.pool.device
    cu = w.info["cu_seqlens_q"]
    st.cu_seqlens_q = _t(cu, dev)
    st.max_q = int(max(1, int(np.diff(cu).max(initial=1))))
    # host-side context statistics of the sequences with rows (routing only)
    has_rows = np.diff(cu) > 0
    ctx = w.context_lens[has_rows].astype(np.float64) if has_rows.any() else np.ones(1)
    st.max_context = int(ctx.max())
    st.mean_context = float(ctx.mean())
    Q, H, D = w.query.shape
    nbytes = pa_multi_workspace_size(Q, H, D, w.max_blocks_per_seq, w.block_size,
                                     w.partition_size)
    st.multi_workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st.multi_grid = pa_multi_balanced_grid(H, w.num_kv_heads, D, w.block_size,
                                               st.max_q)
    nb = pa_multi_balanced_workspace_size_tiles(w.num_seqs, H, w.num_kv_heads, D,
                                                max(st.multi_grid, 1), st.max_q)
    st.multi_bal_workspace = torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev)
    return st


PREFILL_ROWS = 128          # rows x heads per workgroup of pa_prefill
PREFILL_MIN_WORKGROUPS = 256
PREFILL_MAX_TAIL = 4.0      # longest context over the mean one


def prefill_preferred(step: DeviceStep) -> bool:
    """pa_prefill (one workgroup walks all the keys of 128 rows x heads)
    for chunks of more than 16 rows x heads per sequence when the launch has
    at least 256 workgroups and no context is much longer than the mean
    (that workgroup would finish last); otherwise pa_decode_multi, whose
    prefill body splits the keys into partitions and folds them after.
    Measured on MI355X (us, pa_prefill vs pa_decode_multi): 512-token chunks
    of 16 sequences ctx U[512, 4096] 293 vs 1745; 2048 rows of one sequence
    390 vs 559; 8 rows x 64 sequences of 512 keys 36 vs 48; 64 rows of the
    Llama-2-13B layout 159 vs 276; 16 rows x 64 sequences with lognormal
    contexts up to 8192 220 vs 134; 512 rows of one sequence of 4096 keys
    (128 workgroups) 133 vs 76; 64-row chunks of 6 sequences 49 vs 34."""
    g = step.query.shape[1] // step.key_cache.shape[2]
    rows = step.max_q * g
    if rows <= 16:
        return False
    tiles = -(-rows // PREFILL_ROWS)
    wgs = step.block_tables.shape[0] * step.key_cache.shape[2] * tiles
    mean = max(getattr(step, "mean_context", 0.0), 1.0)
    tail = getattr(step, "max_context", 0) / mean
    return wgs >= PREFILL_MIN_WORKGROUPS and tail <= PREFILL_MAX_TAIL


def multi_step(step: DeviceStep, stream=None, balanced=None, prefill=None) -> None:
    """Attention of the step's query rows (their K/V already written):
    pa_prefill when ``prefill_preferred`` (or ``prefill``) says so;
    otherwise pa_decode_multi_balanced when every sequence's rows x heads
    fit one 16-column tile (or ``balanced`` says so), else pa_decode_multi
    (key partitions, then a per-row fold; its prefill body above 16 rows x
    heads).  An explicit ``balanced`` selects between the two decode
    forms."""
    if prefill is None:
        prefill = balanced is None and prefill_preferred(step)
    if prefill:
        pa_prefill(step.out, step.query, step.key_cache, step.value_cache,
                   step.block_tables, step.cu_seqlens_q, step.context_lens,
                   step.max_q, step.scale, stream=stream)
        return
    if balanced is None:
        g = step.query.shape[1] // step.key_cache.shape[2]
        balanced = step.multi_grid > 0 and step.max_q * g <= 16
    if balanced:
        pa_decode_multi_balanced(step.out, step.query, step.key_cache, step.value_cache,
                                 step.block_tables, step.cu_seqlens_q, step.context_lens,
                                 step.max_q, step.scale, step.multi_grid,
                                 step.multi_bal_workspace, stream=stream)
        return
    pa_decode_multi(step.out, step.query, step.key_cache, step.value_cache,
                    step.block_tables, step.cu_seqlens_q, step.context_lens,
                    step.max_q, step.scale, step.partition_size,
                    step.multi_workspace, stream=stream)


def upload(w, device: str = "cuda", pool: Optional[torch.Tensor] = None) -> DeviceStep:
    """Device copies of a workload's pool (initial garbage), decode inputs and
    step phases.  ``pool`` reuses an existing device pool tensor."""
    dev = torch.device(device)
    if pool is None:
        pool = _t(w.pool_init.view(np.float16), dev)
    S, H, D = w.query.shape
    ws = pa_splitk_workspace_size(S, H, D, w.max_blocks_per_seq, w.block_size,
                                  w.partition_size)
    with torch.cuda.device(dev):
        grid = pa_balanced_grid(H, w.num_kv_heads, D, w.block_size)
    if grid <= 0:
        raise RuntimeError("pa_balanced_grid failed")
    bws = pa_balanced_workspace_size(S, H, w.num_kv_heads, D, grid)
    return DeviceStep(
        block_size=w.block_size, scale=w.scale, partition_size=w.partition_size,
        pool=pool, query=_t(w.query, dev), block_tables=_t(w.block_tables, dev),
        context_lens=_t(w.context_lens, dev),
        out=torch.empty((S, H, D), dtype=torch.float16, device=dev),
        copies=_dev_phase(w.step_copies, dev), write=_dev_phase(w.step_write, dev),
        workspace=torch.empty(max(ws, 16), dtype=torch.uint8, device=dev),
        grid=grid,
        bal_workspace=torch.zeros(max(bws, 16), dtype=torch.uint8, device=dev))


def apply_history(w, step: DeviceStep, stream=None) -> None:
    """Bring the device pool to the pre-step state (prefill writes, COW)."""
    for ph in w.history:
        d = _dev_phase(ph, step.pool.device)
        run_phase(d, step.pool, w.block_size, stream=stream)
        del d


def write_step(step: DeviceStep, stream=None) -> None:
    run_phase(step.copies, step.pool, step.block_size, stream=stream)
    run_phase(step.write, step.pool, step.block_size, stream=stream)


def decode_step(step: DeviceStep, mode: str = "splitk", stream=None) -> None:
    if mode == "single":
        pa_decode(step.out, step.query, step.key_cache, step.value_cache,
                  step.block_tables, step.context_lens, step.scale, stream=stream)
    elif mode == "fused_only":         # pa_decode_step without the COW copies
        wr = step.write
        pa_decode_step(step.out, step.query, wr.key, wr.value, step.key_cache,
                       step.value_cache, step.block_tables, step.context_lens,
                       step.scale, step.grid, step.bal_workspace,
                       slot_mapping=wr.slots, stream=stream)
    elif mode == "balanced":
        pa_decode_balanced(step.out, step.query, step.key_cache, step.value_cache,
                           step.block_tables, step.context_lens, step.scale,
                           step.grid, step.bal_workspace, stream=stream)
    elif mode == "splitk":
        pa_decode_splitk(step.query, step.key_cache, step.value_cache,
                         step.block_tables, step.context_lens, step.scale,
                         step.partition_size, step.workspace, stream=stream)
        pa_decode_reduce(step.out, step.workspace, step.context_lens,
                         step.block_tables.shape[1], step.block_size,
                         step.partition_size, stream=stream)
    else:
        raise ValueError(mode)


def fused_step(step: DeviceStep, stream=None) -> None:
    """COW copies (if any), then pa_decode_step: append + balanced decode."""
    run_phase(step.copies, step.pool, step.block_size, stream=stream)
    decode_step(step, "fused_only", stream=stream)


def full_step(step: DeviceStep, mode: str = "splitk", stream=None) -> None:
    if mode == "fused":
        fused_step(step, stream=stream)
        return
    write_step(step, stream=stream)
    decode_step(step, mode=mode, stream=stream)


def split_views(step: DeviceStep, S: int, H: int, D: int, M: int, B: int, P: int):
    """(max_logits, exp_sums, tmp_out) views of the split-KV workspace."""
    pm = (M * B + P - 1) // P
    rows = S * H * pm
    f = step.workspace[: (2 * rows + rows * D) * 4].view(torch.float32)
    return (f[:rows].view(S, H, pm), f[rows:2 * rows].view(S, H, pm),
            f[2 * rows:].view(S, H, pm, D))


__all__: List[str] = ["DeviceStep", "upload", "apply_history", "write_step",
                      "decode_step", "fused_step", "full_step", "run_phase",
                      "split_views"]


# ---------------------------------------------------------------------------
# fp8 (e4m3) pool
# ---------------------------------------------------------------------------

def _byte_view(half: torch.Tensor) -> torch.Tensor:
    """An fp8 pool half [nb, B, H_kv, D] uint8 seen as fp16 [nb, B, H_kv, D/2]:
    block copies move bytes, so the fp16 copy kernel serves both pools."""
    return half.view(torch.float16)


def run_phase_fp8(ph, pool, block_size: int, k_scale: float, v_scale: float,
                  stream=None) -> None:
    if ph is None:
        return
    if isinstance(ph, DevCopy):
        pa_copy_blocks(_byte_view(pool[0]), _byte_view(pool[1]), ph.src, ph.dst,
                       stream=stream)
        return
    pa_slot_mapping(ph.slots, ph.table, ph.seq, ph.pos, block_size, stream=stream)
    pa_cache_write_fp8(ph.key, ph.value, pool[0], pool[1], ph.slots, k_scale, v_scale,
                       stream=stream)


def upload_fp8(w, k_scale: float, v_scale: float, device: str = "cuda") -> DeviceStep:
    """As upload, with a uint8 pool of e4m3 codes whose initial garbage is
    the low byte of the fp16 garbage; the balanced grid and workspace are
    the fp8 decode's."""
    dev = torch.device(device)
    pool = _t((w.pool_init & 0xFF).astype(np.uint8), dev)
    st = upload(w, device, pool=torch.empty(0, dtype=torch.float16, device=dev))
    st.pool = pool
    S, H, D = w.query.shape
    with torch.cuda.device(dev):
        st.grid = pa_balanced_grid_fp8(H, w.num_kv_heads, D, w.block_size)
    if st.grid <= 0:
        raise RuntimeError("pa_balanced_grid_fp8 failed")
    bws = pa_balanced_workspace_size(S, H, w.num_kv_heads, D, st.grid)
    st.bal_workspace = torch.zeros(max(bws, 16), dtype=torch.uint8, device=dev)
    st.k_scale, st.v_scale = float(k_scale), float(v_scale)
    return st


def apply_history_fp8(w, step: DeviceStep, stream=None) -> None:
    for ph in w.history:
        d = _dev_phase(ph, step.pool.device)
        run_phase_fp8(d, step.pool, w.block_size, step.k_scale, step.v_scale,
                      stream=stream)
        del d


def fp8_decode(step: DeviceStep, stream=None) -> None:
    pa_decode_balanced_fp8(step.out, step.query, step.key_cache, step.value_cache,
                           step.block_tables, step.context_lens, step.scale,
                           step.k_scale, step.v_scale, step.grid, step.bal_workspace,
                           stream=stream)


def fp8_fused(step: DeviceStep, stream=None) -> None:
    """pa_decode_step_fp8: quantised append + decode in one kernel."""
    wr = step.write
    pa_decode_step_fp8(step.out, step.query, wr.key, wr.value, step.key_cache,
                       step.value_cache, step.block_tables, step.context_lens,
                       step.scale, step.k_scale, step.v_scale, step.grid,
                       step.bal_workspace, slot_mapping=wr.slots, stream=stream)


def fp8_step(step: DeviceStep, fused: bool = True, stream=None) -> None:
    """COW copies, then either the fused fp8 step or slot mapping + fp8
    cache write + the fp8 decode."""
    run_phase_fp8(step.copies, step.pool, step.block_size, step.k_scale, step.v_scale,
                  stream=stream)
    if fused:
        fp8_fused(step, stream=stream)
        return
    run_phase_fp8(step.write, step.pool, step.block_size, step.k_scale, step.v_scale,
                  stream=stream)
    fp8_decode(step, stream=stream)


# ---------------------------------------------------------------------------
# shared-prefix decode
# ---------------------------------------------------------------------------

def prefix_groups(block_tables, context_lens, block_size: int):
    """Groups of sequences whose table rows start with the same physical
    blocks (what a scheduler knows from its reference counts): sequences are
    grouped by their first block id; a group's shared block count is the
    length of the members' common row prefix, at most min(n_i) // B full
    blocks.  Returns (offsets, members, blocks) int32 arrays, groups of two
    or more members only."""
    bt = np.asarray(block_tables)
    n = np.asarray(context_lens).astype(np.int64)
    by_first = {}
    for i in range(bt.shape[0]):
        if n[i] >= block_size:
            by_first.setdefault(int(bt[i, 0]), []).append(i)
    offsets, members, blocks = [0], [], []
    for first, mem in sorted(by_first.items()):
        if len(mem) < 2:
            continue
        cap = int(min(n[m] for m in mem) // block_size)
        rows = bt[mem, :cap]
        same = (rows == rows[0]).all(axis=0)
        k = int(np.argmin(same)) if not same.all() else cap
        if k == 0:
            continue
        members += mem
        offsets.append(len(members))
        blocks.append(k)
    return (np.asarray(offsets, np.int32), np.asarray(members, np.int32),
            np.asarray(blocks, np.int32))


def upload_prefix(w, device: str = "cuda", pool: Optional[torch.Tensor] = None,
                  groups=None) -> DeviceStep:
    """As upload, plus the shared-prefix groups of the step's tables (from
    prefix_groups unless given) and the shared-prefix workspace."""
    st = upload(w, device, pool)
    dev = st.pool.device
    if groups is None:
        groups = prefix_groups(w.block_tables, w.context_lens, w.block_size)
    off, mem, blk = groups
    st.grp_offsets, st.grp_members, st.grp_blocks = (_t(off, dev), _t(mem, dev),
                                                     _t(blk, dev))
    st.grp_max_size = int(np.diff(off).max(initial=1)) if len(off) > 1 else 1
    st.grp_max_blocks = int(blk.max(initial=0))
    S, H, D = w.query.shape
    nbytes = pa_prefix_workspace_size(S, H, D, w.max_blocks_per_seq, w.block_size,
                                      w.partition_size)
    st.prefix_workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    return st


def prefix_decode(step: DeviceStep, stream=None) -> None:
    pa_decode_shared_prefix(step.out, step.query, step.key_cache, step.value_cache,
                            step.block_tables, step.context_lens, step.scale,
                            step.partition_size, step.grp_offsets, step.grp_members,
                            step.grp_blocks, step.grp_max_size, step.grp_max_blocks,
                            step.prefix_workspace, stream=stream)


def prefix_step(step: DeviceStep, stream=None) -> None:
    """COW copies, slot mapping and cache write, then the shared-prefix
    decode."""
    write_step(step, stream=stream)
    prefix_decode(step, stream=stream)

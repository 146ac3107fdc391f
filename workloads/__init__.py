"""Seeded synthetic inputs for paged KV-cache decode.

This module only draws random numbers and does block bookkeeping (a free list
with reference counts, the way a scheduler hands out block ids).  It holds none
of the arithmetic the method computes: no slot arithmetic, no gather, no
attention.  Each consumer (the HIP path and the CPU oracle) turns the raw
per-token K/V below into pool contents with its own slot_mapping and cache
write, and runs its own decode.

A workload is a list of phases applied to a pool that starts as garbage:

* ``WritePhase`` -- tokens given by (table row, logical position) with their
  K/V rows; the consumer derives each token's physical slot from ``table``.
* ``CopyPhase``  -- copy-on-write block copies (src -> dst, K and V).

``history`` brings the pool to the state before the decode step; ``step_*``
is the decode step itself (append one token per sequence, then attend over
exactly ``context_lens[i]`` tokens).

Shapes and distributions follow the five decode workloads the method is
measured on: the 25/47/12-token worked example of "PagedAttention：KV Cache的
虚拟内存" (section 具体实例演示), the Llama-2-13B layer shape of the vLLM book
ch.4 "PagedAttention：虚拟内存的启示" (§4.1.1, §4.3.1), a GQA layer, parallel
sampling with a shared prefix and copy-on-write (§4.7.1 of the book; the COW
steps of "PagedAttention原理（下）" §4.3), and long-context split-KV decode.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Union

import numpy as np

__all__ = [
    "WritePhase", "CopyPhase", "Workload", "PRESETS", "make", "preset_names",
    "normal_f16", "garbage_u16",
]

_CHUNK = 1 << 22


# ----------------------------------------------------------------------------
# raw random arrays (deterministic in (seed, tag, shape), independent of threads)
# ----------------------------------------------------------------------------

def _seedseq(seed: int, tag: str) -> np.random.SeedSequence:
    key = tuple(int(b) for b in tag.encode())
    return np.random.SeedSequence(entropy=seed, spawn_key=key)


def _parallel_fill(out_flat: np.ndarray, ss: np.random.SeedSequence, fill) -> None:
    n = out_flat.size
    k = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = ss.spawn(k)

    def work(i: int) -> None:
        a = i * _CHUNK
        b = min(n, a + _CHUNK)
        if a >= b:
            return
        rng = np.random.Generator(np.random.PCG64(kids[i]))
        fill(rng, out_flat[a:b])

    if k == 1:
        work(0)
    else:
        with ThreadPoolExecutor(8) as ex:
            list(ex.map(work, range(k)))


def normal_f16(seed: int, tag: str, shape) -> np.ndarray:
    """N(0,1) drawn in float32 and rounded to fp16 (round to nearest even)."""
    out = np.empty(shape, np.float16)

    def fill(rng, dst):
        dst[...] = rng.standard_normal(dst.size, dtype=np.float32)

    _parallel_fill(out.reshape(-1), _seedseq(seed, tag), fill)
    return out


def garbage_u16(seed: int, tag: str, shape, finite: bool = True) -> np.ndarray:
    """Random fp16 bit patterns.  ``finite`` clears the lowest exponent bit, so
    the exponent field can never be all ones: every value is finite, with
    magnitudes from subnormal up to 65504.  ``finite=False`` keeps Inf/NaN."""
    out = np.empty(shape, np.uint16)

    def fill(rng, dst):
        dst[...] = rng.integers(0, 1 << 16, size=dst.size, dtype=np.uint16)
        if finite:
            dst &= np.uint16(0xFBFF)

    _parallel_fill(out.reshape(-1), _seedseq(seed, tag), fill)
    return out


# ----------------------------------------------------------------------------
# workload containers
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class WritePhase:
    table: np.ndarray       # int32 [rows, M]: block table the positions refer to
    seq: np.ndarray         # int32 [N]: row of ``table`` for each token
    pos: np.ndarray         # int32 [N]: logical position of each token
    key: np.ndarray         # fp16 [N, H_kv, D]
    value: np.ndarray       # fp16 [N, H_kv, D]


@dataclasses.dataclass
class CopyPhase:
    src: np.ndarray         # int32 [C] physical block ids to copy from
    dst: np.ndarray         # int32 [C] physical block ids to copy into


Phase = Union[WritePhase, CopyPhase]


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    partition_size: int
    scale: float                    # float32-representable softmax scale
    context_lens: np.ndarray        # int32 [S], includes the appended token
    block_tables: np.ndarray        # int32 [S, M], final (after any COW)
    query: np.ndarray               # fp16 [S, H, D]
    pool_init: np.ndarray           # uint16 [2, nb, B, H_kv, D] (garbage)
    history: List[Phase]
    step_copies: Optional[CopyPhase]
    step_write: WritePhase
    blocks_used: np.ndarray         # int32 [S] number of table entries in use
    ref_cnt: np.ndarray             # int32 [nb] references held by tables
    info: Dict[str, object]

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def kv_shape(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_size)


# ----------------------------------------------------------------------------
# block bookkeeping (scheduler side)
# ----------------------------------------------------------------------------

class _FreeList:
    """Pops physical ids from a seeded order; tracks reference counts."""

    def __init__(self, order: np.ndarray, num_blocks: int):
        self.order = [int(x) for x in order]
        self.next = 0
        self.ref = np.zeros(num_blocks, np.int32)

    def pop(self) -> int:
        if self.next >= len(self.order):
            raise MemoryError("block pool exhausted")
        b = self.order[self.next]
        self.next += 1
        self.ref[b] += 1
        return b

    def drop(self, b: int) -> None:
        """One reference to block b released (copy-on-write repoints a table
        entry); a block nobody references cannot be released again."""
        if self.ref[b] <= 0:
            raise ValueError(f"reference count of block {b} would go below zero")
        self.ref[b] -= 1


def _ceil_div(a: int, b: int) -> int:
    return (a + b - 1) // b


def _fill_unused(tables: np.ndarray, used: np.ndarray, ref: np.ndarray,
                 rng: np.random.Generator) -> None:
    """Entries past each row's used count point at unreferenced (poisoned)
    blocks: a kernel that reads them gets garbage, never an out-of-range id."""
    spare = np.flatnonzero(ref == 0).astype(np.int32)
    if spare.size == 0:
        spare = np.zeros(1, np.int32)
    S, M = tables.shape
    for i in range(S):
        k = M - int(used[i])
        if k > 0:
            tables[i, used[i]:] = rng.choice(spare, size=k, replace=True)


# ----------------------------------------------------------------------------
# context-length recipes
# ----------------------------------------------------------------------------

def _lens_fixed(values):
    def f(rng, S):
        return np.asarray(values, np.int64)
    return f


def _lens_uniform(lo, hi):
    def f(rng, S):
        return rng.integers(lo, hi + 1, size=S).astype(np.int64)
    return f


def _lens_lognormal(median, sigma, lo, hi):
    def f(rng, S):
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=S)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    return f


# ----------------------------------------------------------------------------
# presets
# ----------------------------------------------------------------------------

# Each preset: shape, lengths recipe, pool policy.  "full" presets are the
# benchmarked decode workloads; "*_small" keep their head shapes at sizes the
# CPU oracle finishes in seconds while still spanning several partitions and a
# ragged last block.
PRESETS: Dict[str, dict] = {
    # 3 requests of 25/47/12 tokens, 64-block pool, 4/4 heads, D 64.
    "c1": dict(S=3, H=4, Hkv=4, D=64, B=16, lens=_lens_fixed([25, 47, 12]),
               pool=("choice_nb", 64), max_context=2048, seed=1001),
    # Llama-2-13B layer: 40/40 heads, D 128, B 16, 4000 blocks, 32 seqs U[1,2048].
    "c2": dict(S=32, H=40, Hkv=40, D=128, B=16, lens=_lens_uniform(1, 2048),
               pool=("freelist_nb", 4000), max_context=2048, seed=1002),
    # GQA 32/8, D 128, B 16, 64 seqs lognormal(median 700, sigma 1) in [1, 8192].
    "c3": dict(S=64, H=32, Hkv=8, D=128, B=16,
               lens=_lens_lognormal(700, 1.0, 1, 8192),
               pool=("choice_scale", 1.25), max_context=8192, seed=1003),
    # 16 prompts x 4 samples sharing a 1024(+r)-token prefix, COW of the partial
    # prefix block, tails U[0,512], one appended token; 40/40 heads, D 128.
    "c4": dict(kind="prefix", prompts=16, samples=4, prefix=1024,
               extra=(1, 15), tail=(0, 512), H=40, Hkv=40, D=128, B=16,
               pool=("freelist_nb", 4000), max_context=2048, seed=1004),
    # Long context: 8 seqs U[32768,131072], 64/8 heads, D 128, B 32 / 64.
    "c5_b32": dict(S=8, H=64, Hkv=8, D=128, B=32,
                   lens=_lens_uniform(32768, 131072),
                   pool=("choice_scale", 1.25), max_context=131072,
                   key_outliers=(0.01, 8.0), seed=1005),
    "c5_b64": dict(S=8, H=64, Hkv=8, D=128, B=64,
                   lens=_lens_uniform(32768, 131072),
                   pool=("choice_scale", 1.25), max_context=131072,
                   key_outliers=(0.01, 8.0), seed=1006),
    # ---- reduced sizes of the same shapes (oracle in seconds) ----
    "c1_page_tables": dict(S=3, H=4, Hkv=4, D=64, B=16,
                           lens=_lens_fixed([25, 47, 12]),
                           pool=("explicit", 64, [[3, 7], [0, 5, 9], [4]]),
                           max_context=2048, seed=1011),
    "c2_small": dict(S=6, H=40, Hkv=40, D=128, B=16, lens=_lens_uniform(1, 2048),
                     pool=("freelist_nb", 1000), max_context=2048, seed=1012),
    "c3_small": dict(S=10, H=32, Hkv=8, D=128, B=16,
                     lens=_lens_lognormal(700, 1.0, 1, 8192),
                     pool=("choice_scale", 1.25), max_context=8192, seed=1013),
    "c4_small": dict(kind="prefix", prompts=2, samples=4, prefix=1024,
                     extra=(1, 15), tail=(0, 512), H=40, Hkv=40, D=128, B=16,
                     pool=("freelist_nb", 600), max_context=2048, seed=1014),
    "c4_r0_small": dict(kind="prefix", prompts=2, samples=4, prefix=1024,
                        extra=(0, 0), tail=(0, 512), H=40, Hkv=40, D=128, B=16,
                        pool=("freelist_nb", 600), max_context=2048, seed=1015),
    "c5_b32_small": dict(S=3, H=64, Hkv=8, D=128, B=32,
                         lens=_lens_uniform(1500, 5000),
                         pool=("choice_scale", 1.25), max_context=131072,
                         key_outliers=(0.01, 8.0), seed=1016),
    "c5_b64_small": dict(S=3, H=64, Hkv=8, D=128, B=64,
                         lens=_lens_uniform(1500, 5000),
                         pool=("choice_scale", 1.25), max_context=131072,
                         key_outliers=(0.01, 8.0), seed=1017),
    # ---- several query tokens per sequence (the last q_len of each) ----
    # speculative verify of 4 draft tokens at the Llama-2-13B and GQA shapes
    "c2_spec4": dict(S=32, H=40, Hkv=40, D=128, B=16, lens=_lens_uniform(4, 2048),
                     pool=("freelist_nb", 4000), max_context=2048, q_len=4, seed=1021),
    "c3_spec4": dict(S=64, H=32, Hkv=8, D=128, B=16,
                     lens=_lens_lognormal(700, 1.0, 4, 8192),
                     pool=("choice_scale", 1.25), max_context=8192, q_len=4, seed=1022),
    # reduced sizes: verify, a 64-token prefill chunk, whole-prompt prefill
    "c1_prefill": dict(S=3, H=4, Hkv=4, D=64, B=16, lens=_lens_fixed([25, 47, 12]),
                       pool=("choice_nb", 64), max_context=2048, q_len=2048, seed=1023),
    "c2_small_spec4": dict(S=6, H=40, Hkv=40, D=128, B=16, lens=_lens_uniform(1, 2048),
                           pool=("freelist_nb", 1000), max_context=2048, q_len=4,
                           seed=1024),
    "c3_small_spec4": dict(S=10, H=32, Hkv=8, D=128, B=16,
                           lens=_lens_lognormal(700, 1.0, 1, 8192),
                           pool=("choice_scale", 1.25), max_context=8192, q_len=4,
                           seed=1025),
    "c3_small_chunk64": dict(S=6, H=32, Hkv=8, D=128, B=16,
                             lens=_lens_uniform(40, 1500),
                             pool=("choice_scale", 1.25), max_context=8192, q_len=64,
                             seed=1026),
    # chunked prefill: a 512-token chunk at the end of each sequence (the
    # whole context when it is shorter), GQA 32/8 heads
    "c3_chunk512": dict(S=16, H=32, Hkv=8, D=128, B=16, lens=_lens_uniform(512, 4096),
                        pool=("choice_scale", 1.25), max_context=8192, q_len=512,
                        seed=1028),
    "c3_small_chunk512": dict(S=3, H=32, Hkv=8, D=128, B=16, lens=_lens_uniform(300, 1500),
                              pool=("choice_scale", 1.25), max_context=8192, q_len=512,
                              seed=1029),
    "c5_b32_small_spec2": dict(S=3, H=64, Hkv=8, D=128, B=32,
                               lens=_lens_uniform(1500, 5000),
                               pool=("choice_scale", 1.25), max_context=131072,
                               key_outliers=(0.01, 8.0), q_len=2, seed=1027),
}


def preset_names() -> List[str]:
    return list(PRESETS)


def _scale_for(D: int) -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


def make(name_or_spec: Union[str, dict], seed: Optional[int] = None,
         garbage: str = "finite", **override) -> Workload:
    """Build a workload from a preset name or an explicit spec dict.

    ``override`` replaces spec entries (e.g. ``lens=[1, 512, 513]`` for edge
    cases, ``S=``, ``H=``...).  ``garbage`` is "finite" (default) or
    "nonfinite" (pool garbage may hold Inf/NaN)."""
    if isinstance(name_or_spec, str):
        name = name_or_spec
        spec = dict(PRESETS[name])
    else:
        name = name_or_spec.get("name", "custom")
        spec = dict(name_or_spec)
    for k, v in override.items():
        if k == "lens" and not callable(v):
            v = _lens_fixed(v)
        spec[k] = v
    if seed is None:
        seed = int(spec.get("seed", 0))
    if spec.get("kind") == "prefix":
        return _make_prefix(name, spec, seed, garbage)
    return _make_plain(name, spec, seed, garbage)


def _make_plain(name: str, spec: dict, seed: int, garbage: str) -> Workload:
    rng = np.random.default_rng(_seedseq(seed, "layout"))
    H, Hkv, D, B = spec["H"], spec["Hkv"], spec["D"], spec["B"]
    assert H % Hkv == 0
    lens = spec["lens"](rng, spec.get("S", 0))
    S = int(lens.size)
    M = _ceil_div(int(spec["max_context"]), B)
    assert int(lens.min(initial=1)) >= 1 and int(lens.max(initial=1)) <= M * B
    used = np.array([_ceil_div(int(n), B) for n in lens], np.int64)
    need = int(used.sum())

    pol = spec["pool"]
    tables = np.zeros((S, M), np.int32)
    if pol[0] == "explicit":
        nb = int(pol[1])
        rows = pol[2]
        ref = np.zeros(nb, np.int32)
        for i, row in enumerate(rows):
            assert len(row) == used[i]
            tables[i, :len(row)] = row
            for b in row:
                ref[b] += 1
    else:
        if pol[0] == "choice_nb":
            nb = int(pol[1])
            order = rng.choice(nb, size=need, replace=False)
        elif pol[0] == "choice_scale":
            nb = int(math.ceil(pol[1] * need))
            order = rng.choice(nb, size=need, replace=False)
        elif pol[0] == "freelist_nb":
            nb = int(pol[1])
            order = rng.permutation(nb)
        else:
            raise ValueError(pol)
        fl = _FreeList(order, nb)
        for i in range(S):
            for j in range(int(used[i])):
                tables[i, j] = fl.pop()
        ref = fl.ref
    _fill_unused(tables, used, ref, rng)

    # history: positions 0..n-1-Tq of every sequence; step: the last Tq
    # positions (Tq = 1 for decode; min(q_len, n) for multi-token queries)
    qn = np.minimum(lens, int(spec.get("q_len", 1))).astype(np.int64)
    hist_seq = np.repeat(np.arange(S, dtype=np.int32), lens - qn)
    hist_pos = np.concatenate([np.arange(n - t, dtype=np.int32) for n, t in zip(lens, qn)]) \
        if S else np.zeros(0, np.int32)
    T = int(hist_seq.size)
    Q = int(qn.sum())
    hk = normal_f16(seed, "hist_key", (T, Hkv, D))
    hv = normal_f16(seed, "hist_value", (T, Hkv, D))
    sk = normal_f16(seed, "step_key", (Q, Hkv, D))
    sv = normal_f16(seed, "step_value", (Q, Hkv, D))
    if "key_outliers" in spec:
        frac, mult = spec["key_outliers"]
        for tag, arr in (("hist_outl", hk), ("step_outl", sk)):
            r = np.random.default_rng(_seedseq(seed, tag))
            mask = r.random(arr.shape[:2]) < frac
            arr[mask] = (arr[mask].astype(np.float32) * np.float32(mult)).astype(np.float16)
    q = normal_f16(seed, "query", (Q, H, D))
    pool = garbage_u16(seed, "pool", (2, nb, B, Hkv, D), finite=(garbage == "finite"))

    step_seq = np.repeat(np.arange(S, dtype=np.int32), qn)
    step_pos = np.concatenate([np.arange(n - t, n, dtype=np.int32) for n, t in zip(lens, qn)]) \
        if S else np.zeros(0, np.int32)
    step = WritePhase(tables, step_seq, step_pos, sk, sv)
    info = {"blocks_needed_total": need}
    if "q_len" in spec:
        info["q_lens"] = qn.astype(np.int32)
        info["cu_seqlens_q"] = np.concatenate([[0], np.cumsum(qn)]).astype(np.int32)
    hist = [WritePhase(tables, hist_seq, hist_pos, hk, hv)]
    return Workload(
        name=name, seed=seed, num_seqs=S, num_heads=H, num_kv_heads=Hkv,
        head_size=D, block_size=B, num_blocks=nb, max_blocks_per_seq=M,
        partition_size=int(spec.get("P", 512)), scale=_scale_for(D),
        context_lens=lens.astype(np.int32), block_tables=tables, query=q,
        pool_init=pool, history=hist, step_copies=None, step_write=step,
        blocks_used=used.astype(np.int32), ref_cnt=ref.astype(np.int32),
        info=info,
    )


def _make_prefix(name: str, spec: dict, seed: int, garbage: str) -> Workload:
    """Parallel sampling over a shared prompt, with copy-on-write.

    Each prompt's blocks are referenced by every sample (ref_cnt = samples).
    A sample's first write into a block whose ref_cnt > 1 copies it to a fresh
    block, repoints that sample's table entry and drops the original's count;
    the last sample left holding the block writes in place."""
    rng = np.random.default_rng(_seedseq(seed, "layout"))
    Pn, n_s = int(spec["prompts"]), int(spec["samples"])
    H, Hkv, D, B = spec["H"], spec["Hkv"], spec["D"], spec["B"]
    M = _ceil_div(int(spec["max_context"]), B)
    nb = int(spec["pool"][1])
    fl = _FreeList(rng.permutation(nb), nb)
    S = Pn * n_s

    ex_lo, ex_hi = spec["extra"]
    tl_lo, tl_hi = spec["tail"]
    L = spec["prefix"] + rng.integers(ex_lo, ex_hi + 1, size=Pn)
    tails = rng.integers(tl_lo, tl_hi + 1, size=S)

    prompt_tables = np.zeros((Pn, M), np.int32)
    prompt_used = np.zeros(Pn, np.int64)
    tables = np.zeros((S, M), np.int32)
    used = np.zeros(S, np.int64)
    for p in range(Pn):
        nbp = _ceil_div(int(L[p]), B)
        for j in range(nbp):
            prompt_tables[p, j] = fl.pop()
        prompt_used[p] = nbp
        for s in range(n_s):
            i = p * n_s + s
            tables[i, :nbp] = prompt_tables[p, :nbp]
            used[i] = nbp
        fl.ref[prompt_tables[p, :nbp]] += n_s - 1   # shared by all samples

    hist_copies: List[tuple] = []
    step_copies: List[tuple] = []

    def prepare_write(i: int, pos: int, copies: list) -> None:
        lb = pos // B
        if lb >= used[i]:                       # first token of a new block
            assert lb == used[i]
            tables[i, lb] = fl.pop()
            used[i] = lb + 1
            return
        blk = int(tables[i, lb])
        if fl.ref[blk] > 1:                     # shared: copy on write
            new = fl.pop()
            copies.append((blk, new))
            tables[i, lb] = new
            fl.drop(blk)

    lens = np.zeros(S, np.int64)
    hist_rows, hist_pos = [], []
    for i in range(S):
        p = i // n_s
        for t in range(int(tails[i])):
            pos = int(L[p]) + t
            prepare_write(i, pos, hist_copies)
            hist_rows.append(i)
            hist_pos.append(pos)
        lens[i] = int(L[p]) + int(tails[i]) + 1
    for i in range(S):                          # decode step: one new token
        prepare_write(i, int(lens[i]) - 1, step_copies)

    _fill_unused(tables, used, fl.ref, rng)
    _fill_unused(prompt_tables, prompt_used, fl.ref, rng)

    pre_seq = np.repeat(np.arange(Pn, dtype=np.int32), L)
    pre_pos = np.concatenate([np.arange(int(x), dtype=np.int32) for x in L])
    pk = normal_f16(seed, "prefix_key", (pre_seq.size, Hkv, D))
    pv = normal_f16(seed, "prefix_value", (pre_seq.size, Hkv, D))
    hist_rows = np.asarray(hist_rows, np.int32)
    hist_pos = np.asarray(hist_pos, np.int32)
    tk = normal_f16(seed, "tail_key", (hist_rows.size, Hkv, D))
    tv = normal_f16(seed, "tail_value", (hist_rows.size, Hkv, D))
    sk = normal_f16(seed, "step_key", (S, Hkv, D))
    sv = normal_f16(seed, "step_value", (S, Hkv, D))
    q = normal_f16(seed, "query", (S, H, D))
    pool = garbage_u16(seed, "pool", (2, nb, B, Hkv, D), finite=(garbage == "finite"))

    def copies(lst):
        a = np.asarray(lst, np.int32).reshape(-1, 2)
        return CopyPhase(a[:, 0].copy(), a[:, 1].copy())

    history: List[Phase] = [WritePhase(prompt_tables, pre_seq, pre_pos, pk, pv)]
    if hist_copies:
        history.append(copies(hist_copies))
    history.append(WritePhase(tables, hist_rows, hist_pos, tk, tv))
    step = WritePhase(tables, np.arange(S, dtype=np.int32),
                      (lens - 1).astype(np.int32), sk, sv)
    return Workload(
        name=name, seed=seed, num_seqs=S, num_heads=H, num_kv_heads=Hkv,
        head_size=D, block_size=B, num_blocks=nb, max_blocks_per_seq=M,
        partition_size=int(spec.get("P", 512)), scale=_scale_for(D),
        context_lens=lens.astype(np.int32), block_tables=tables, query=q,
        pool_init=pool, history=history,
        step_copies=copies(step_copies) if step_copies else None,
        step_write=step, blocks_used=used.astype(np.int32),
        ref_cnt=fl.ref.astype(np.int32),
        info={"prompt_len": L.astype(np.int64), "tails": tails.astype(np.int64),
              "samples": n_s, "prompts": Pn,
              "prompt_tables": prompt_tables, "prompt_used": prompt_used,
              "hist_copies": len(hist_copies), "step_copies": len(step_copies)},
    )

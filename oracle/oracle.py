"""CPU oracle for paged KV-cache decode -- TEST INFRASTRUCTURE ONLY.

Plain, slow and obviously correct.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does, and this module imports nothing from the product (no HIP code, no
binding, no shared helpers).  Floating point is computed in float64 from the
exact fp16 inputs.

Sources (page title, then section):

* [BOOK]  vLLM book ch.4 "PagedAttention：虚拟内存的启示" (yangyitao.com)
* [GUST]  "PagedAttention：KV Cache的虚拟内存" (bittide translation of
          thegustafson.com "Paged Attention")
* [CSDN]  CSDN PageAttention tutorial (nanhubrain.csdn.net), part 三.1
* [P5]    "PagedAttention原理（下）" (5688vip, vLLM推理框架全解析 04)

What is computed (paging does not change the math -- [GUST] 常见误解):
for sequence i and query head h, with kv head ⌊h / g⌋ (g = H / H_kv),
    K_t = key_cache[bt[i, ⌊t/B⌋], t mod B, ⌊h/g⌋, :],   t = 0 .. n_i - 1
    out[i, h] = Σ_t softmax_t(scale · <q[i, h], K_t>) · V_t
The softmax here is the plain two-pass form in float64 (max, then
exp/normalise), deliberately not the streaming form a kernel uses.

Every function below is pinned by tests against numbers the pages print,
closed forms, brute force on tiny inputs and a library attention routine.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kv_cache_shape", "kv_bytes_per_token", "block_bytes", "blocks_needed",
    "slots_reserved", "padding_slots", "slot_mapping", "cache_write",
    "copy_blocks", "swap_blocks", "apply_phases", "gather_kv", "decode", "decode_heads",
    "partials", "merge", "decode_multi", "fp8_e4m3_value", "fp8_e4m3_decode",
    "fp8_e4m3_encode", "fp8_quantize_rows", "cache_write_fp8", "apply_phases_fp8",
    "gather_kv_fp8", "decode_fp8",
]


# ----------------------------------------------------------------------------
# byte and block accounting
# ----------------------------------------------------------------------------

def kv_cache_shape(num_blocks: int, block_size: int, num_kv_heads: int,
                   head_size: int) -> tuple:
    """[BOOK] §4.3.1: the per-layer pool is (2, num_blocks, block_size,
    num_kv_heads, head_size); index 0 of the first axis holds K, 1 holds V."""
    return (2, num_blocks, block_size, num_kv_heads, head_size)


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       dtype_bytes: int) -> int:
    """[BOOK] §4.1.1 equation: K and V, times layers, KV heads, head_dim and
    bytes per element."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def block_bytes(block_size: int, num_kv_heads: int, head_size: int,
                dtype_bytes: int, num_layers: int = 1) -> int:
    """[BOOK] §4.3.1: one block of one layer holds K and V for block_size
    tokens; a "complete block" spans every layer."""
    return 2 * block_size * num_kv_heads * head_size * dtype_bytes * num_layers


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """[GUST] 具体实例演示: a request of n tokens takes ceil(n / B) blocks."""
    n, b = int(num_tokens), int(block_size)
    if n <= 0:
        return 0
    return (n + b - 1) // b


def slots_reserved(context_lens, block_size: int) -> int:
    """[GUST] 具体实例演示: slots held = blocks × B, summed over requests."""
    return sum(blocks_needed(n, block_size) * block_size for n in context_lens)


def padding_slots(num_tokens: int, block_size: int) -> int:
    """Slots of the last block left empty; at most B - 1 ([GUST] 一图解析)."""
    return blocks_needed(num_tokens, block_size) * block_size - int(num_tokens)


# ----------------------------------------------------------------------------
# write path
# ----------------------------------------------------------------------------

def slot_mapping(block_tables, seq, positions, block_size: int) -> np.ndarray:
    """[BOOK] §4.4.3: the token at logical position p of the request in table
    row r goes to logical block p // B at offset p mod B; its physical slot is
    block_table[r, p // B] · B + p mod B.  Written token by token."""
    bt = np.asarray(block_tables)
    out = np.empty(len(positions), np.int32)
    for j in range(len(positions)):
        r = int(seq[j])
        p = int(positions[j])
        logical_block = p // block_size
        offset = p % block_size
        physical_block = int(bt[r, logical_block])
        out[j] = physical_block * block_size + offset
    return out


def cache_write(key_cache: np.ndarray, value_cache: np.ndarray,
                key: np.ndarray, value: np.ndarray, slots) -> None:
    """[BOOK] §4.3.2 and §4.5 (1): each new token's K and V rows are copied to
    key_cache[slot] / value_cache[slot].  A pure copy of fp16 bits: the caches
    are uint16 (or float16) arrays of shape [nb, B, H_kv, D]; the token rows
    are [N, H_kv, D].  A negative slot means "no write"."""
    nb, B, Hkv, D = key_cache.shape
    # the pool seen as one flat array of slots: key_cache[slot] in the text
    kc = key_cache.view(np.uint16).reshape(nb * B, Hkv, D)
    vc = value_cache.view(np.uint16).reshape(nb * B, Hkv, D)
    k = np.asarray(key).view(np.uint16)
    v = np.asarray(value).view(np.uint16)
    for j in range(len(slots)):
        s = int(slots[j])
        if s < 0:
            continue
        kc[s] = k[j]
        vc[s] = v[j]


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray, src, dst) -> None:
    """Copy-on-write block copy ([GUST] COW paragraph; [P5] §4.3 step 3): the
    whole physical block src (K and V) is duplicated into dst."""
    kc = key_cache.view(np.uint16)
    vc = value_cache.view(np.uint16)
    for a, b in zip(src, dst):
        kc[int(b)] = kc[int(a)]
        vc[int(b)] = vc[int(a)]


def swap_blocks(src_key_cache: np.ndarray, src_value_cache: np.ndarray,
                dst_key_cache: np.ndarray, dst_value_cache: np.ndarray,
                src_ids, dst_ids) -> None:
    """Block swap between two pools ([P5] §4.4: the physical blocks of a
    paused request move out to CPU memory and back): block src_ids[k] of the
    source pool (K and V) becomes block dst_ids[k] of the destination pool.
    Pairs with an id outside either pool are skipped."""
    sk, sv = src_key_cache.view(np.uint16), src_value_cache.view(np.uint16)
    dk, dv = dst_key_cache.view(np.uint16), dst_value_cache.view(np.uint16)
    for a, b in zip(src_ids, dst_ids):
        a, b = int(a), int(b)
        if not (0 <= a < sk.shape[0] and 0 <= b < dk.shape[0]):
            continue
        dk[b] = sk[a]
        dv[b] = sv[a]


def apply_phases(key_cache: np.ndarray, value_cache: np.ndarray, phases,
                 block_size: int) -> None:
    """Run a list of write / copy phases (objects with .table/.seq/.pos/.key/
    .value or .src/.dst) in order with the functions above."""
    for ph in phases:
        if ph is None:
            continue
        if hasattr(ph, "src"):
            copy_blocks(key_cache, value_cache, ph.src, ph.dst)
        else:
            s = slot_mapping(ph.table, ph.seq, ph.pos, block_size)
            cache_write(key_cache, value_cache, ph.key, ph.value, s)


# ----------------------------------------------------------------------------
# read path
# ----------------------------------------------------------------------------

def gather_kv(key_cache, value_cache, table_row, n: int):
    """[BOOK] §4.5 and §4.4.1: walk the request's table in logical order; for
    each logical block take the physical block's rows; keep exactly the first
    n tokens (the valid slots only -- [CSDN] 三.1).  Returns float64
    K, V of shape [n, H_kv, D]."""
    kc = np.asarray(key_cache).view(np.float16)
    vc = np.asarray(value_cache).view(np.float16)
    B = kc.shape[1]
    nblk = blocks_needed(n, B)
    ids = [int(table_row[lb]) for lb in range(nblk)]
    for b in ids:
        assert 0 <= b < kc.shape[0], "block id out of range"
    K = np.concatenate([kc[b] for b in ids], axis=0)[:n]
    V = np.concatenate([vc[b] for b in ids], axis=0)[:n]
    return K.astype(np.float64), V.astype(np.float64)


def _two_pass_softmax_attention(q, K, V, scale):
    """q [g, D], K/V [n, D] (float64): x = scale·K q; p = exp(x - max x);
    out = (p V) / Σ p."""
    x = scale * (q @ K.T)                    # [g, n]
    m = x.max(axis=1, keepdims=True)
    p = np.exp(x - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def decode_heads(query, key_cache, value_cache, block_tables, context_lens,
                 scale: float, pairs) -> np.ndarray:
    """Attention output for selected (sequence, query head) pairs, float64
    [len(pairs), D].  Same definition as ``decode``; used to sample outputs of
    workloads too large to compute whole."""
    q = np.asarray(query).view(np.float16)
    H = q.shape[1]
    Hkv = np.asarray(key_cache).shape[2]
    g = H // Hkv
    out = np.empty((len(pairs), q.shape[2]), np.float64)
    cache = {}
    for k, (i, h) in enumerate(pairs):
        i, h = int(i), int(h)
        if i not in cache:
            cache = {i: gather_kv(key_cache, value_cache, block_tables[i],
                                  int(context_lens[i]))}
        K, V = cache[i]
        kvh = h // g
        out[k] = _two_pass_softmax_attention(
            q[i, h:h + 1].astype(np.float64), K[:, kvh], V[:, kvh],
            float(scale))[0]
    return out


def decode(query, key_cache, value_cache, block_tables, context_lens,
           scale: float) -> np.ndarray:
    """Decode attention for every sequence and query head, float64 [S, H, D].

    Query head h reads KV head h // g (g = H / H_kv): consecutive query heads
    share a KV head ([BOOK] §4.5 (3) leaves the mapping to the backend; this is
    the reading taken).  context_lens[i] counts every token attended,
    including the one appended in this step ([BOOK] §4.4.3 and §4.5: write
    first, then read)."""
    q = np.asarray(query).view(np.float16)
    S, H, D = q.shape
    Hkv = np.asarray(key_cache).shape[2]
    assert H % Hkv == 0
    g = H // Hkv
    out = np.empty((S, H, D), np.float64)
    for i in range(S):
        n = int(context_lens[i])
        assert n >= 1, "context_len must be >= 1"
        K, V = gather_kv(key_cache, value_cache, block_tables[i], n)
        for kvh in range(Hkv):
            qs = q[i, kvh * g:(kvh + 1) * g].astype(np.float64)
            out[i, kvh * g:(kvh + 1) * g] = _two_pass_softmax_attention(
                qs, K[:, kvh], V[:, kvh], float(scale))
    return out


# ----------------------------------------------------------------------------
# split-KV: per-partition state and its merge
# ----------------------------------------------------------------------------

def partials(query, key_cache, value_cache, block_tables, context_lens,
             scale: float, partition_size: int, num_partitions: int):
    """Per-partition softmax state.  Partition p of sequence i covers tokens
    [p·P, min((p+1)·P, n_i)).  For each (i, h, p) with tokens:
        m = max_t x_t,  s = Σ_t exp(x_t - m),  O = Σ_t exp(x_t - m) V_t
    (O is not normalised).  Empty partitions get m = -inf, s = 0, O = 0.
    Returns float64 m, s [S, H, Pn] and O [S, H, Pn, D]."""
    q = np.asarray(query).view(np.float16)
    S, H, D = q.shape
    Hkv = np.asarray(key_cache).shape[2]
    g = H // Hkv
    P = int(partition_size)
    m = np.full((S, H, num_partitions), -np.inf)
    s = np.zeros((S, H, num_partitions))
    O = np.zeros((S, H, num_partitions, D))
    for i in range(S):
        n = int(context_lens[i])
        K, V = gather_kv(key_cache, value_cache, block_tables[i], n)
        for h in range(H):
            kvh = h // g
            x = float(scale) * (K[:, kvh] @ q[i, h].astype(np.float64))
            for p in range(num_partitions):
                a, b = p * P, min((p + 1) * P, n)
                if a >= b:
                    continue
                mp = x[a:b].max()
                e = np.exp(x[a:b] - mp)
                m[i, h, p] = mp
                s[i, h, p] = e.sum()
                O[i, h, p] = e @ V[a:b, kvh]
    return m, s, O


def merge(m, s, O, context_lens, partition_size: int) -> np.ndarray:
    """Merge partition states with the online-softmax recurrence of [BOOK] §4.6:
    folding state (m_b, s_b, O_b) into (m_a, s_a, O_a) gives
        m = max(m_a, m_b),
        s = s_a·exp(m_a - m) + s_b·exp(m_b - m),
        O = O_a·exp(m_a - m) + O_b·exp(m_b - m);
    the result is O / s after the last partition.  Only partitions holding
    tokens are folded."""
    S, H, Pn = np.asarray(m).shape
    D = np.asarray(O).shape[-1]
    out = np.empty((S, H, D))
    for i in range(S):
        n = int(context_lens[i])
        used = (n + partition_size - 1) // partition_size
        for h in range(H):
            ma, sa, Oa = m[i, h, 0], s[i, h, 0], O[i, h, 0].copy()
            for p in range(1, used):
                mb, sb, Ob = m[i, h, p], s[i, h, p], O[i, h, p]
                mn = max(ma, mb)
                sa = sa * np.exp(ma - mn) + sb * np.exp(mb - mn)
                Oa = Oa * np.exp(ma - mn) + Ob * np.exp(mb - mn)
                ma = mn
            out[i, h] = Oa / sa
    return out


# ----------------------------------------------------------------------------
# several query tokens per sequence
# ----------------------------------------------------------------------------

def decode_multi(query, key_cache, value_cache, block_tables, cu_seqlens_q,
                 context_lens, scale: float) -> np.ndarray:
    """Attention of several new query tokens per request over the same block
    tables ([BOOK] §4.5 (2): the backend gets the query tokens of every
    request delimited by cu_seqlens_q, the keys per request (seqused_k, here
    context_lens) and block_table).  Sequence i owns query rows
    cu[i] .. cu[i+1]-1, the last T_i = cu[i+1] - cu[i] of its n_i tokens
    (written first, read after -- [BOOK] §4.5 (1)); row r = cu[i] + j is at
    position p = n_i - T_i + j and attends to keys t = 0 .. p only (causal).
    Two-pass softmax per row in float64; returns [Q, H, D]."""
    q = np.asarray(query).view(np.float16)
    Q, H, D = q.shape
    Hkv = np.asarray(key_cache).shape[2]
    g = H // Hkv
    cu = np.asarray(cu_seqlens_q)
    out = np.empty((Q, H, D), np.float64)
    for i in range(len(context_lens)):
        n = int(context_lens[i])
        a, b = int(cu[i]), int(cu[i + 1])
        T = b - a
        if T == 0:
            continue
        assert 1 <= T <= n, "each query token needs its key in the cache"
        K, V = gather_kv(key_cache, value_cache, block_tables[i], n)
        for j in range(T):
            p = n - T + j
            for h in range(H):
                out[a + j, h] = _two_pass_softmax_attention(
                    q[a + j, h:h + 1].astype(np.float64), K[:p + 1, h // g],
                    V[:p + 1, h // g], float(scale))[0]
    return out


# ----------------------------------------------------------------------------
# fp8 (e4m3) KV cache
# ----------------------------------------------------------------------------
# [BOOK] §4.8 lists a lower-precision KV cache among the ways to fit more
# tokens in a KV budget; [CSDN] 三.2 (the KVBlock field table) stores block K/V
# as FP16 or FP8.  The pages fix no FP8 format or scaling; the reading taken
# is the OCP 8-bit floating point format E4M3 ("e4m3fn": sign, 4 exponent
# bits with bias 7, 3 mantissa bits, no infinities, exponent and mantissa
# all ones = NaN, largest finite value 448) with one scale per tensor:
# stored value = decode(code) * scale, code = encode(x / scale).

def fp8_e4m3_value(code: int) -> float:
    """Value of one E4M3 code from the format's definition (NaN for the two
    NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:                                  # subnormal: m/8 * 2^(1-7)
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Elementwise fp8_e4m3_value of a uint8 array, float64."""
    table = np.array([fp8_e4m3_value(c) for c in range(256)], np.float64)
    return table[np.asarray(codes, np.uint8)]


def fp8_e4m3_encode(x) -> np.ndarray:
    """Code of the E4M3 value nearest to each float in x, ties to the code
    with an even mantissa (round to nearest even); magnitudes are first
    clamped to 448, NaN gives the NaN code of its sign.  Comparisons are
    against exact midpoints, so no rounding happens inside."""
    a = np.asarray(x, np.float64)
    mags = np.array([fp8_e4m3_value(c) for c in range(0x7F)])   # 0 .. 448
    neg = np.signbit(a)
    nan = np.isnan(a)
    m = np.minimum(np.abs(np.where(nan, 0.0, a)), 448.0)
    hi = np.searchsorted(mags, m, side="left")                  # first mag >= m
    exact = mags[np.minimum(hi, len(mags) - 1)] == m
    lo = np.maximum(hi - 1, 0)
    mid = (mags[lo] + mags[np.minimum(hi, len(mags) - 1)]) / 2.0
    tie_pick = np.where(lo % 2 == 0, lo, hi)                    # even mantissa
    c = np.where(exact, hi, np.where(m < mid, lo, np.where(m > mid, hi, tie_pick)))
    c = np.where(nan, 0x7F, c).astype(np.uint8)
    return (c | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def fp8_quantize_rows(rows, scale: float) -> np.ndarray:
    """fp16 rows -> codes: x times the fp32 reciprocal of the scale, the
    product rounded to fp32 (the precision the quantised code is decided
    in), then encoded.  The code depends only on x's 16 bits, so it is
    computed once for each of the 65536 fp16 values and looked up."""
    inv = np.float32(1.0) / np.float32(scale)
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = every.astype(np.float32) * inv
    table = fp8_e4m3_encode(prod.astype(np.float64))
    return table[np.asarray(rows).view(np.uint16)]


def cache_write_fp8(key_cache: np.ndarray, value_cache: np.ndarray,
                    key: np.ndarray, value: np.ndarray, slots,
                    k_scale: float, v_scale: float) -> None:
    """As cache_write, into an fp8 pool (uint8 [nb, B, H_kv, D]): the rows
    are quantised with their tensor's scale first."""
    nb, B, Hkv, D = key_cache.shape
    kc = key_cache.reshape(nb * B, Hkv, D)
    vc = value_cache.reshape(nb * B, Hkv, D)
    kq = fp8_quantize_rows(key, k_scale)
    vq = fp8_quantize_rows(value, v_scale)
    for j in range(len(slots)):
        s = int(slots[j])
        if s < 0:
            continue
        kc[s] = kq[j]
        vc[s] = vq[j]


def apply_phases_fp8(key_cache: np.ndarray, value_cache: np.ndarray, phases,
                     block_size: int, k_scale: float, v_scale: float) -> None:
    """apply_phases for an fp8 pool: writes quantise, block copies move the
    one-byte codes."""
    for ph in phases:
        if ph is None:
            continue
        if hasattr(ph, "src"):
            for a, b in zip(ph.src, ph.dst):
                key_cache[int(b)] = key_cache[int(a)]
                value_cache[int(b)] = value_cache[int(a)]
        else:
            s = slot_mapping(ph.table, ph.seq, ph.pos, block_size)
            cache_write_fp8(key_cache, value_cache, ph.key, ph.value, s,
                            k_scale, v_scale)


def gather_kv_fp8(key_cache, value_cache, table_row, n: int, k_scale: float,
                  v_scale: float):
    """gather_kv over an fp8 pool: the first n token rows in logical order,
    dequantised (code value times scale), float64 [n, H_kv, D]."""
    kc = np.asarray(key_cache, np.uint8)
    vc = np.asarray(value_cache, np.uint8)
    B = kc.shape[1]
    ids = [int(table_row[lb]) for lb in range(blocks_needed(n, B))]
    for b in ids:
        assert 0 <= b < kc.shape[0], "block id out of range"
    K = np.concatenate([kc[b] for b in ids], axis=0)[:n]
    V = np.concatenate([vc[b] for b in ids], axis=0)[:n]
    return (fp8_e4m3_decode(K) * float(k_scale),
            fp8_e4m3_decode(V) * float(v_scale))


def decode_fp8(query, key_cache, value_cache, block_tables, context_lens,
               scale: float, k_scale: float, v_scale: float,
               pairs=None) -> np.ndarray:
    """decode over an fp8 pool: attention over the dequantised K and V.
    With ``pairs`` (a list of (sequence, query head)), only those outputs,
    [len(pairs), D]; else every one, [S, H, D]."""
    q = np.asarray(query).view(np.float16)
    S, H, D = q.shape
    Hkv = np.asarray(key_cache).shape[2]
    g = H // Hkv
    todo = pairs if pairs is not None else [(i, h) for i in range(S) for h in range(H)]
    out = np.empty((len(todo), D), np.float64)
    cur, K, V = None, None, None
    for k, (i, h) in enumerate(todo):
        i, h = int(i), int(h)
        if i != cur:
            n = int(context_lens[i])
            assert n >= 1, "context_len must be >= 1"
            K, V = gather_kv_fp8(key_cache, value_cache, block_tables[i], n,
                                 k_scale, v_scale)
            cur = i
        out[k] = _two_pass_softmax_attention(
            q[i, h:h + 1].astype(np.float64), K[:, h // g], V[:, h // g],
            float(scale))[0]
    return out if pairs is not None else out.reshape(S, H, D)

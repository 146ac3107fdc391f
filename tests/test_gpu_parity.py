"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Cache writes, slot mappings and block copies must be bit-exact over the
whole pool; attention outputs must satisfy, elementwise,
|y - r| <= 2e-3  or  |y - r| <= 1e-2 * |r|
(fp16 I/O, fp32 accumulation) against the float64 oracle r."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import oracle_pool

pytestmark = pytest.mark.gpu

ATOL = 2e-3
RTOL = 1e-2


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_120_amd as pa
    from paged_kv_cache_120_amd import runner
    return pa, runner


def assert_attention_close(y, r, what=""):
    y = np.asarray(y, np.float64)
    err = np.abs(y - r)
    ok = (err <= ATOL) | (err <= RTOL * np.abs(r))
    big = np.abs(r) >= 0.2
    rel = (err[big] / np.abs(r[big])).max() if big.any() else 0.0
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    assert ok.all(), (f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; "
                      f"max abs {err.max():.3e}, max rel {rel:.3e}")
    return float(err.max()), float(rel)


def run_gpu(w, mode, stream=None):
    pa, runner = _gpu()
    st = runner.upload(w)
    runner.apply_history(w, st)
    runner.full_step(st, mode=mode)
    torch.cuda.synchronize()
    return st


def check_all(w, mode, full_oracle=True, pairs=None):
    st = run_gpu(w, mode)
    kc, vc = oracle_pool(w, oracle)
    gpool = st.pool.cpu().numpy().view(np.uint16)
    assert (gpool[0] == kc).all(), "key cache differs from the oracle's"
    assert (gpool[1] == vc).all(), "value cache differs from the oracle's"
    ref_slots = oracle.slot_mapping(w.step_write.table, w.step_write.seq,
                                    w.step_write.pos, w.block_size)
    assert (st.write.slots.cpu().numpy() == ref_slots).all()
    out = st.out.cpu().numpy()
    if full_oracle:
        ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
        assert_attention_close(out, ref, f"{w.name}/{mode}")
    else:
        ref = oracle.decode_heads(w.query, kc, vc, w.block_tables, w.context_lens,
                                  w.scale, pairs)
        got = np.stack([out[i, h] for i, h in pairs])
        assert_attention_close(got, ref, f"{w.name}/{mode} sampled")
    return st, kc, vc


SMALL = ["c1", "c1_page_tables", "c2_small", "c3_small", "c4_small", "c4_r0_small",
         "c5_b32_small", "c5_b64_small"]


MODES = ["single", "splitk", "balanced", "fused"]


def decode_only(runner, st, mode):
    """Decode with the step's K/V already written (fused: written again)."""
    if mode == "fused":
        runner.fused_step(st)
    else:
        runner.decode_step(st, mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", SMALL)
def test_parity_small(name, mode):
    print(f"[parity] {name} {mode}", flush=True)
    check_all(workloads.make(name), mode)


@pytest.mark.parametrize("name", ["c3_small", "c5_b32_small", "c2_small"])
def test_split_partials_match_oracle(name):
    print(f"[partials] {name}", flush=True)
    pa, runner = _gpu()
    w = workloads.make(name)
    st = run_gpu(w, "splitk")
    kc, vc = oracle_pool(w, oracle)
    S, H, D = w.query.shape
    M, B, P = w.max_blocks_per_seq, w.block_size, w.partition_size
    gm, gs, go = [t.cpu().numpy().astype(np.float64)
                  for t in runner.split_views(st, S, H, D, M, B, P)]
    pm = gm.shape[2]
    m, s, O = oracle.partials(w.query, kc, vc, w.block_tables, w.context_lens,
                              w.scale, P, pm)
    for i, n in enumerate(w.context_lens):
        used = (int(n) + P - 1) // P
        assert np.allclose(gm[i, :, :used], m[i, :, :used], rtol=1e-5, atol=1e-5)
        assert np.allclose(gs[i, :, :used], s[i, :, :used], rtol=2e-3, atol=1e-5)
        scale = s[i, :, :used, None]
        assert np.allclose(go[i, :, :used] / scale, O[i, :, :used] / scale,
                           rtol=1e-2, atol=2e-3)


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,mode", [("c1", "splitk"), ("c2", "splitk"), ("c2", "single"),
                                       ("c2", "balanced"), ("c3", "splitk"),
                                       ("c3", "balanced"), ("c4", "splitk"),
                                       ("c4", "balanced"), ("c2", "fused"),
                                       ("c3", "fused"), ("c4", "fused")])
def test_parity_full(name, mode):
    print(f"[parity-full] {name} {mode}", flush=True)
    check_all(workloads.make(name), mode)


@pytest.mark.parametrize("mode", ["splitk", "balanced", "fused"])
@pytest.mark.parametrize("name", ["c5_b32", "c5_b64"])
def test_parity_full_long_context(name, mode):
    """Every (sequence, query head) output of the long-context workloads,
    including the pairs the balanced split cuts across the most workgroups."""
    print(f"[parity-full] {name} {mode}", flush=True)
    check_all(workloads.make(name), mode)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

EDGE_LENS = [1, 2, 15, 16, 17, 31, 33, 511, 512, 513, 1023, 1024, 1025, 2047, 2048]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("D,B,H,Hkv", [(128, 16, 32, 8), (64, 64, 16, 2),
                                       (128, 32, 8, 8), (64, 16, 8, 4),
                                       (128, 64, 16, 8), (64, 16, 16, 4)])
def test_edge_lengths(D, B, H, Hkv, mode):
    print(f"[edge] D{D} B{B} H{H}/{Hkv} {mode}", flush=True)
    w = workloads.make("c1", D=D, B=B, H=H, Hkv=Hkv, lens=EDGE_LENS,
                       pool=("choice_scale", 1.3), max_context=2048, seed=D + B + H)
    check_all(w, mode)


@pytest.mark.parametrize("mode", MODES)
def test_full_table(mode):
    """context_len = max_blocks_per_seq * block_size (every entry used)."""
    w = workloads.make("c1", D=128, B=32, H=16, Hkv=4, lens=[640, 1, 640, 639],
                       pool=("choice_scale", 1.0), max_context=640, seed=3)
    assert w.max_blocks_per_seq * w.block_size == 640
    check_all(w, mode)


@pytest.mark.parametrize("mode", MODES)
def test_nonfinite_garbage_is_never_read(mode):
    w = workloads.make("c3_small", garbage="nonfinite")
    check_all(w, mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", ["c3_small", "c5_b32_small"])
def test_weights_near_the_lazy_reference_ceiling(name, mode):
    """The matrix-core bodies round softmax weights to fp16 for P.V.  The
    first 64 keys of every 512-token window score 0; the first batch of each
    of a workgroup's four waves (16 keys each at D = 128) that starts a
    sequence or a 512-token split partition falls there and sets the wave's
    reference to 0.  Every other key scores 62 * scale * log2(e) = 7.9 in
    base 2, just below the point where the reference would move (8), so most
    of the weight is carried by weights of 2^7.9 on values of 1: the fp16
    rounding of the weights is as large, and as uniform in sign, as the
    bound allows.  (Balanced slices start at any 16-token boundary; a slice
    whose first batch scores 7.9 takes that as its reference.)"""
    print(f"[lazy-ceiling] {name} {mode}", flush=True)
    w = workloads.make(name)
    assert w.head_size == 128 and w.partition_size % 512 == 0
    w.query[...] = np.float16(1.0)
    for ph in [p for p in w.history if hasattr(p, "seq")] + [w.step_write]:
        early = ph.pos % 512 < 64
        ph.key[early] = np.float16(0.0)
        ph.key[~early] = np.float16(62.0 / 128.0)     # q.k = 62 (exact in fp16)
        ph.value[~early] = np.float16(1.0)
    s2 = 62.0 * float(w.scale) * np.log2(np.e)
    assert 7.5 < s2 < 8.0
    check_all(w, mode)


@pytest.mark.parametrize("P", [16, 64, 256, 1024, 4096])
def test_splitk_partition_sizes(P):
    w = workloads.make("c3_small")
    w.partition_size = P
    check_all(w, "splitk")


@pytest.mark.parametrize("mode", MODES)
def test_zero_context_gives_zeros(mode):
    pa, runner = _gpu()
    w = workloads.make("c2_small")
    st = runner.upload(w)
    runner.apply_history(w, st)
    runner.write_step(st)
    ctx = w.context_lens.copy()
    ctx[2] = 0
    st.context_lens.copy_(torch.from_numpy(ctx))
    decode_only(runner, st, mode)
    torch.cuda.synchronize()
    out = st.out.cpu().numpy().astype(np.float64)
    assert (out[2] == 0).all()
    kc, vc = oracle_pool(w, oracle)
    keep = [i for i in range(w.num_seqs) if i != 2]
    ref = oracle.decode(w.query[keep], kc, vc, w.block_tables[keep], ctx[keep], w.scale)
    assert_attention_close(out[keep], ref, "zero-context neighbours")


def test_permutation_invariance_bitwise():
    """Relabelling physical blocks leaves the GPU result bit-identical."""
    pa, runner = _gpu()
    w = workloads.make("c3_small")
    outs = []
    for relabel in (False, True):
        st = runner.upload(w)
        runner.apply_history(w, st)
        runner.write_step(st)
        if relabel:
            perm = np.random.default_rng(11).permutation(w.num_blocks)
            inv = torch.from_numpy(np.argsort(perm)).cuda()
            newpool = st.pool[:, inv].contiguous()        # newpool[:, perm[b]] = pool[:, b]
            st.pool = newpool
            st.block_tables = torch.from_numpy(perm[w.block_tables].astype(np.int32)).cuda()
        for mode in MODES:
            decode_only(runner, st, mode)
            torch.cuda.synchronize()
            outs.append(st.out.cpu().numpy().copy())
    k = len(MODES)
    for i in range(k):
        assert (outs[i].view(np.uint16) == outs[k + i].view(np.uint16)).all(), MODES[i]


def test_shared_prefix_equals_private_copies_bitwise():
    pa, runner = _gpu()
    w = workloads.make("c4_small")
    st = run_gpu(w, "splitk")
    shared = st.out.cpu().numpy().copy()
    # private layout built on the device: every sample gets copies of its blocks
    S, M = w.num_seqs, w.max_blocks_per_seq
    total = int(w.blocks_used.sum())
    src, tables = [], np.zeros((S, M), np.int32)
    nxt = 0
    for i in range(S):
        for lb in range(int(w.blocks_used[i])):
            src.append(int(w.block_tables[i, lb]))
            tables[i, lb] = nxt
            nxt += 1
    pool2 = torch.empty((2, total) + tuple(st.pool.shape[2:]), dtype=torch.float16,
                        device="cuda")
    idx = torch.tensor(src, dtype=torch.int64, device="cuda")
    pool2.copy_(st.pool[:, idx])
    st.pool = pool2
    st.block_tables = torch.from_numpy(tables).cuda()
    runner.decode_step(st, "splitk")
    torch.cuda.synchronize()
    assert (st.out.cpu().numpy().view(np.uint16) == shared.view(np.uint16)).all()


def test_fused_step_slot_output_for_empty_sequences():
    pa, runner = _gpu()
    w = workloads.make("c2_small")
    st = runner.upload(w)
    runner.apply_history(w, st)
    ctx = w.context_lens.copy()
    ctx[1] = 0
    st.context_lens.copy_(torch.from_numpy(ctx))
    st.write.slots.fill_(12345)
    runner.fused_step(st)
    torch.cuda.synchronize()
    got = st.write.slots.cpu().numpy()
    ref = oracle.slot_mapping(w.step_write.table, w.step_write.seq, w.step_write.pos,
                              w.block_size)
    assert got[1] == -1
    keep = [i for i in range(w.num_seqs) if i != 1]
    assert (got[keep] == ref[keep]).all()


@pytest.mark.parametrize("grid", [1, 3, 17, 200, 5000])
@pytest.mark.parametrize("name", ["c3_small", "c2_small", "c5_b64_small"])
def test_balanced_any_grid(name, grid):
    """Any workgroup count gives the same answer: a slice may hold many
    (sequence, head) ranges (grid 1) or less than one tile (grid 5000)."""
    print(f"[balanced-grid] {name} grid={grid}", flush=True)
    pa, runner = _gpu()
    w = workloads.make(name)
    st = runner.upload(w)
    runner.apply_history(w, st)
    runner.write_step(st)
    nbytes = pa.pa_balanced_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads,
                                           w.head_size, grid)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(2):        # the second call reuses the counters the first reset
        pa.pa_decode_balanced(st.out, st.query, st.key_cache, st.value_cache,
                              st.block_tables, st.context_lens, st.scale, grid, ws)
    torch.cuda.synchronize()
    hdr = w.num_seqs * w.num_kv_heads
    assert (ws[: hdr * 4].view(torch.int32) == 0).all(), "counters not reset"
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"{name} grid {grid}")


def test_balanced_workspace_reuse_across_shapes():
    """One zero-filled workspace, sized for the largest call, serves decode
    calls of different shapes in any order: the counter header does not move
    with the shape, so a call with more (sequence, kv head) pairs never reads
    an earlier call's partial states as counters."""
    print("[balanced-workspace-reuse]", flush=True)
    pa, runner = _gpu()
    names = ["c3_small", "c2_small", "c5_b32_small", "c1"]
    cases = []
    for name in names:
        w = workloads.make(name)
        st = runner.upload(w)
        runner.apply_history(w, st)
        runner.write_step(st)
        kc, vc = oracle_pool(w, oracle)
        ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
        cases.append((name, w, st, ref))
    need = max(pa.pa_balanced_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads,
                                             w.head_size, st.grid)
               for _, w, st, _ in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    # more pairs after fewer and fewer after more (pairs: 80, 240, 24, 12)
    for name, w, st, ref in cases + cases[::-1]:
        st.out.zero_()
        pa.pa_decode_balanced(st.out, st.query, st.key_cache, st.value_cache,
                              st.block_tables, st.context_lens, st.scale, st.grid, ws)
        torch.cuda.synchronize()
        assert_attention_close(st.out.cpu().numpy(), ref, f"{name} (shared workspace)")
    pairs = max(w.num_seqs * w.num_kv_heads for _, w, _, _ in cases)
    assert (ws[: pairs * 4].view(torch.int32) == 0).all(), "counters not reset"


def test_repeat_calls_deterministic():
    pa, runner = _gpu()
    w = workloads.make("c2_small")
    for mode in MODES:
        st = run_gpu(w, mode)
        a = st.out.cpu().numpy().copy()
        decode_only(runner, st, mode)
        torch.cuda.synchronize()
        assert (a.view(np.uint16) == st.out.cpu().numpy().view(np.uint16)).all(), mode


def test_cache_write_skips_negative_and_out_of_range_slots():
    pa, runner = _gpu()
    nb, B, Hkv, D = 6, 16, 2, 64
    rng = np.random.default_rng(5)
    pool = rng.integers(0, 1 << 16, (2, nb, B, Hkv, D), dtype=np.uint16)
    key = rng.integers(0, 1 << 16, (4, Hkv, D), dtype=np.uint16)
    val = rng.integers(0, 1 << 16, (4, Hkv, D), dtype=np.uint16)
    slots = np.array([3, -1, nb * B, 95], np.int32)
    gp = torch.from_numpy(pool.view(np.float16)).cuda()
    pa.pa_cache_write(torch.from_numpy(key.view(np.float16)).cuda(),
                      torch.from_numpy(val.view(np.float16)).cuda(), gp[0], gp[1],
                      torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kc, vc = pool[0].copy(), pool[1].copy()
    oracle.cache_write(kc, vc, key, val, np.where(slots < nb * B, slots, -1))
    g = gp.cpu().numpy().view(np.uint16)
    assert (g[0] == kc).all() and (g[1] == vc).all()


def test_copy_blocks_parity():
    pa, runner = _gpu()
    nb, B, Hkv, D = 9, 32, 4, 128
    rng = np.random.default_rng(6)
    pool = rng.integers(0, 1 << 16, (2, nb, B, Hkv, D), dtype=np.uint16)
    src = np.array([1, 4, 7, 2], np.int32)
    dst = np.array([0, 5, 8, 99], np.int32)          # last pair out of range: skipped
    gp = torch.from_numpy(pool.view(np.float16)).cuda()
    pa.pa_copy_blocks(gp[0], gp[1], torch.from_numpy(src).cuda(),
                      torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    kc, vc = pool[0].copy(), pool[1].copy()
    oracle.copy_blocks(kc, vc, src[:3], dst[:3])
    g = gp.cpu().numpy().view(np.uint16)
    assert (g[0] == kc).all() and (g[1] == vc).all()


def test_swap_blocks_pinned_host_round_trip_bitwise():
    """Swap ([P5] §4.4) through pa_swap_blocks: the used blocks go to a
    pinned host pool bit-exactly (oracle swap_blocks; an out-of-range pair is
    skipped), come back into a NaN-filled device pool under new ids, and the
    decode over it is bit-identical to the decode over the original pool
    with the tables relabelled."""
    pa, runner = _gpu()
    w = workloads.make("c3_small")
    st = runner.upload(w)
    runner.apply_history(w, st)
    runner.write_step(st)
    torch.cuda.synchronize()
    B = w.block_size
    used = sorted({int(b) for i, n in enumerate(w.context_lens)
                   for b in w.block_tables[i, :(int(n) + B - 1) // B]})
    nu = len(used)
    host = torch.zeros((2, nu + 2) + tuple(st.pool.shape[2:]), dtype=torch.float16,
                       pin_memory=True)
    src = torch.tensor(used + [w.num_blocks + 5], dtype=torch.int32, device="cuda")
    dst = torch.tensor(list(range(nu)) + [nu], dtype=torch.int32, device="cuda")
    pa.pa_swap_blocks(st.pool[0], st.pool[1], host[0], host[1], src, dst)
    torch.cuda.synchronize()
    kc, vc = oracle_pool(w, oracle)
    hk = np.zeros(tuple(host.shape[1:]), np.uint16)
    hv = np.zeros_like(hk)
    oracle.swap_blocks(kc, vc, hk, hv, used + [w.num_blocks + 5], list(range(nu)) + [nu])
    h = host.numpy().view(np.uint16)
    assert (h[0] == hk).all() and (h[1] == hv).all()

    for mode in MODES:
        decode_only(runner, st, mode)
    torch.cuda.synchronize()
    ref = {}
    for mode in MODES:
        decode_only(runner, st, mode)
        torch.cuda.synchronize()
        ref[mode] = st.out.cpu().numpy().view(np.uint16).copy()
    new_ids = [w.num_blocks - 1 - j for j in range(nu)]
    pool2 = torch.full_like(st.pool, float("nan"))
    pa.pa_swap_blocks(host[0], host[1], pool2[0], pool2[1],
                      torch.arange(nu, dtype=torch.int32, device="cuda"),
                      torch.tensor(new_ids, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    relabel = np.arange(w.num_blocks)
    relabel[used] = new_ids
    st.pool = pool2
    st.block_tables = torch.from_numpy(relabel[w.block_tables].astype(np.int32)).cuda()
    for mode in MODES:
        decode_only(runner, st, mode)
        torch.cuda.synchronize()
        assert (st.out.cpu().numpy().view(np.uint16) == ref[mode]).all(), mode


MULTI_SMALL = ["c1_prefill", "c2_small_spec4", "c3_small_spec4", "c3_small_chunk64",
               "c5_b32_small_spec2"]


def run_multi(w, balanced=None):
    pa, runner = _gpu()
    st = runner.upload_multi(w)
    assert not balanced or st.multi_grid > 0
    runner.apply_history(w, st)
    runner.write_step(st)
    runner.multi_step(st, balanced=balanced)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("balanced", [False, True])
@pytest.mark.parametrize("name", MULTI_SMALL + ["c2_spec4", "c3_spec4"])
def test_multi_token_parity(name, balanced):
    """pa_decode_multi and pa_decode_multi_balanced (causal within each
    sequence's query chunk) against oracle.decode_multi on every row and
    head; the pool after the chunk's cache write is bit-exact."""
    print(f"[multi] {name} balanced={balanced}", flush=True)
    w = workloads.make(name)
    st = run_multi(w, balanced)
    kc, vc = oracle_pool(w, oracle)
    g = st.pool.cpu().numpy().view(np.uint16)
    assert (g[0] == kc).all() and (g[1] == vc).all()
    ref = oracle.decode_multi(w.query, kc, vc, w.block_tables, w.info["cu_seqlens_q"],
                              w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"{name}/multi")


@pytest.mark.parametrize("D,B,H,Hkv,T", [(128, 16, 16, 8, 2), (64, 32, 8, 8, 8),
                                         (128, 16, 8, 8, 3), (64, 16, 16, 2, 1),
                                         (128, 64, 64, 8, 1), (128, 32, 32, 8, 5),
                                         (64, 16, 16, 4, 3), (128, 16, 16, 8, 3),
                                         (128, 32, 16, 2, 2)])
@pytest.mark.parametrize("balanced", [False, True])
def test_multi_token_shapes(D, B, H, Hkv, T, balanced):
    """Shapes that run the whole-line body with g*T within its 4 or 8
    columns (partial tiles), the whole-line body with 16 distinct columns
    (balanced, g*T up to 16, some columns unused: g = 4 T = 3 at D = 64,
    g = 2 T = 3, g = 8 T = 2) and the 16-column body (g = 4, T = 5); the
    balanced kernel where rows x heads fit 16 columns."""
    print(f"[multi-shape] D{D} B{B} H{H}/{Hkv} T{T} balanced={balanced}", flush=True)
    w = workloads.make("c2_small_spec4", D=D, B=B, H=H, Hkv=Hkv, q_len=T,
                       seed=D + B + H + T)
    st = run_multi(w, balanced)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode_multi(w.query, kc, vc, w.block_tables, w.info["cu_seqlens_q"],
                              w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"multi D{D} g{H // Hkv} T{T}")


def run_prefill(w):
    pa, runner = _gpu()
    st = runner.upload_multi(w)
    runner.apply_history(w, st)
    runner.write_step(st)
    st.out.fill_(7.0)
    pa.pa_prefill(st.out, st.query, st.key_cache, st.value_cache, st.block_tables,
                  st.cu_seqlens_q, st.context_lens, st.max_q, w.scale)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("name", MULTI_SMALL + ["c3_small_chunk512"])
def test_prefill_parity(name):
    """pa_prefill (128 rows x heads per pass over the keys) against
    oracle.decode_multi on every row and head: chunks of 2-4 rows, 64 and
    512 rows (several row tiles, causal limits inside a key tile), and the
    whole prompt as the chunk."""
    print(f"[prefill] {name}", flush=True)
    w = workloads.make(name)
    st = run_prefill(w)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode_multi(w.query, kc, vc, w.block_tables, w.info["cu_seqlens_q"],
                              w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"{name}/prefill")


@pytest.mark.parametrize("D,B,H,Hkv,T", [(64, 32, 8, 8, 40), (128, 64, 16, 8, 33),
                                         (128, 16, 16, 16, 7), (64, 16, 16, 4, 100),
                                         (128, 32, 32, 8, 1), (128, 16, 16, 8, 70)])
def test_prefill_shapes(D, B, H, Hkv, T):
    """Head sizes 64 and 128, blocks of 16-64, groups of 1, 2, 4 and 8, and
    chunk lengths that leave partial row tiles (T*g not a multiple of 128)."""
    print(f"[prefill-shape] D{D} B{B} H{H}/{Hkv} T{T}", flush=True)
    w = workloads.make("c2_small_spec4", D=D, B=B, H=H, Hkv=Hkv, q_len=T,
                       seed=3 * D + B + H + T)
    st = run_prefill(w)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode_multi(w.query, kc, vc, w.block_tables, w.info["cu_seqlens_q"],
                              w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"prefill D{D} g{H // Hkv} T{T}")


def test_prefill_full_size_sampled_rows():
    """The 512-token-chunk workload at full size through the runner's default
    (pa_prefill), checked on sampled rows of every sequence: the first and
    last 8 rows of each chunk (the fewest and the most visible keys) against
    oracle.decode_multi on those rows alone."""
    pa, runner = _gpu()
    w = workloads.make("c3_chunk512")
    st = runner.upload_multi(w)
    assert runner.prefill_preferred(st)
    runner.apply_history(w, st)
    runner.write_step(st)
    runner.multi_step(st)
    torch.cuda.synchronize()
    out = st.out.cpu().numpy().astype(np.float64)
    kc, vc = oracle_pool(w, oracle)
    cu = w.info["cu_seqlens_q"]
    for i in range(w.num_seqs):
        n, T = int(w.context_lens[i]), int(cu[i + 1] - cu[i])
        for j0 in (0, T - 8):
            # rows j0 .. j0+7 of a T-row chunk over n keys are the 8 rows of
            # an 8-row chunk over n - T + j0 + 8 keys
            ref = oracle.decode_multi(w.query[cu[i] + j0:cu[i] + j0 + 8], kc, vc,
                                      w.block_tables[i:i + 1], np.array([0, 8], np.int32),
                                      np.array([n - T + j0 + 8], np.int32), w.scale)
            assert_attention_close(out[cu[i] + j0:cu[i] + j0 + 8], ref,
                                   f"c3_chunk512 seq {i} rows {j0}..")


@pytest.mark.parametrize("P", [16, 64, 512, 4096])
@pytest.mark.parametrize("name", ["c3_small_chunk64", "c1_prefill", "c3_small_chunk512"])
def test_multi_wide_chunks_split_prefill_body(name, P):
    """pa_decode_multi with more than 16 rows x heads per sequence runs the
    matrix-core prefill body per key partition (128 rows x heads per pass)
    and the row reduce: every row and head against oracle.decode_multi, at
    partition sizes from one block to longer than any context."""
    print(f"[multi-split-prefill] {name} P={P}", flush=True)
    pa, runner = _gpu()
    w = workloads.make(name)
    B = w.block_size
    w.partition_size = max(P, B)
    st = runner.upload_multi(w)
    runner.apply_history(w, st)
    runner.write_step(st)
    st.out.fill_(7.0)
    runner.multi_step(st, balanced=False)
    torch.cuda.synchronize()
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode_multi(w.query, kc, vc, w.block_tables, w.info["cu_seqlens_q"],
                              w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"{name}/split prefill P={P}")


def test_prefill_edge_rows():
    """Rows placed before the first key (T > n) and a sequence of context 0
    get zeros; a sequence without rows writes nothing; repeated calls give
    the same bits; pa_prefill and pa_decode_multi agree within tolerance."""
    pa, runner = _gpu()
    w = workloads.make("c3_small_chunk64")
    st = run_prefill(w)
    first = st.out.clone()
    pa.pa_prefill(st.out, st.query, st.key_cache, st.value_cache, st.block_tables,
                  st.cu_seqlens_q, st.context_lens, st.max_q, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), st.out.view(torch.int16))
    cu = w.info["cu_seqlens_q"]
    ctx = w.context_lens.copy()
    ctx[1] = 0                                  # no keys: its rows are zeros
    T2 = int(cu[3] - cu[2])
    ctx[2] = T2 // 2                            # first T2 - T2//2 rows see no key
    st.context_lens.copy_(torch.from_numpy(ctx))
    st.out.fill_(7.0)
    pa.pa_prefill(st.out, st.query, st.key_cache, st.value_cache, st.block_tables,
                  st.cu_seqlens_q, st.context_lens, st.max_q, w.scale)
    torch.cuda.synchronize()
    out = st.out.cpu().numpy().astype(np.float64)
    assert (out[cu[1]:cu[2]] == 0).all()
    assert (out[cu[2]:cu[2] + T2 - ctx[2]] == 0).all()
    kc, vc = oracle_pool(w, oracle)
    keep = [i for i in range(w.num_seqs) if i not in (1, 2)]
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in keep] +
                          [np.arange(cu[2] + T2 - ctx[2], cu[3])])
    Ts = [int(cu[i + 1] - cu[i]) for i in keep] + [int(ctx[2])]
    cu2 = np.concatenate([[0], np.cumsum(Ts)]).astype(np.int32)
    ref = oracle.decode_multi(w.query[rows], kc, vc, w.block_tables[keep + [2]], cu2,
                              ctx[keep + [2]], w.scale)
    assert_attention_close(out[rows], ref, "prefill edge rows")


@pytest.mark.parametrize("P", [16, 512])
def test_multi_split_prefill_edge_rows(P):
    """pa_decode_multi's split prefill body and its fold: rows of a sequence
    with context 0, and rows placed before the first key (T > n), get zeros;
    the other rows match the oracle; a repeated call gives the same bits."""
    print(f"[multi-split-prefill-edge] P={P}", flush=True)
    pa, runner = _gpu()
    w = workloads.make("c3_small_chunk64")
    w.partition_size = P
    st = runner.upload_multi(w)
    runner.apply_history(w, st)
    runner.write_step(st)
    cu = w.info["cu_seqlens_q"]
    ctx = w.context_lens.copy()
    ctx[1] = 0
    T2 = int(cu[3] - cu[2])
    ctx[2] = T2 // 2                            # first T2 - T2//2 rows see no key
    st.context_lens.copy_(torch.from_numpy(ctx))
    st.out.fill_(7.0)
    runner.multi_step(st, balanced=False)
    torch.cuda.synchronize()
    first = st.out.clone()
    runner.multi_step(st, balanced=False)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), st.out.view(torch.int16))
    out = st.out.cpu().numpy().astype(np.float64)
    assert (out[cu[1]:cu[2]] == 0).all()
    assert (out[cu[2]:cu[2] + T2 - ctx[2]] == 0).all()
    kc, vc = oracle_pool(w, oracle)
    keep = [i for i in range(w.num_seqs) if i not in (1, 2)]
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in keep] +
                          [np.arange(cu[2] + T2 - ctx[2], cu[3])])
    Ts = [int(cu[i + 1] - cu[i]) for i in keep] + [int(ctx[2])]
    cu2 = np.concatenate([[0], np.cumsum(Ts)]).astype(np.int32)
    ref = oracle.decode_multi(w.query[rows], kc, vc, w.block_tables[keep + [2]], cu2,
                              ctx[keep + [2]], w.scale)
    assert_attention_close(out[rows], ref, f"split prefill edge rows P={P}")


def test_multi_and_prefix_repeat_calls_bitwise():
    """The multi-token and shared-prefix decodes give the same bits on
    repeated calls (no atomics in their reductions)."""
    pa, runner = _gpu()
    for bal in (False, True):
        w = workloads.make("c2_small_spec4")
        st = run_multi(w, bal)
        first = st.out.clone()
        for _ in range(3):
            runner.multi_step(st, balanced=bal)
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), st.out.view(torch.int16))
    w = workloads.make("c4_small")
    st = runner.upload_prefix(w)
    runner.apply_history(w, st)
    runner.prefix_step(st)
    torch.cuda.synchronize()
    first = st.out.clone()
    for _ in range(3):
        runner.prefix_decode(st)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), st.out.view(torch.int16))


@pytest.mark.parametrize("grid", [1, 5, 300])
@pytest.mark.parametrize("name", ["c3_small_spec4", "c3_small_chunk64"])
def test_multi_balanced_any_grid_and_empty_sequences(name, grid):
    """The balanced multi-token kernel at grids other than the resident one,
    with a sequence of context 0 (its rows are zeros) and one without rows;
    one column tile per (sequence, kv head) (4 rows x g = 4) and sixteen
    (a 64-row chunk)."""
    print(f"[multi-grid] {name} grid={grid}", flush=True)
    pa, runner = _gpu()
    w = workloads.make(name)
    st = run_multi(w, True)
    cu = w.info["cu_seqlens_q"]
    ctx = w.context_lens.copy()
    ctx[2] = 0
    st.context_lens.copy_(torch.from_numpy(ctx))
    nb = pa.pa_multi_balanced_workspace_size_tiles(w.num_seqs, w.query.shape[1],
                                                   w.num_kv_heads, w.head_size, grid,
                                                   st.max_q)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    st.out.fill_(3.0)
    pa.pa_decode_multi_balanced(st.out, st.query, st.key_cache, st.value_cache,
                                st.block_tables, st.cu_seqlens_q, st.context_lens,
                                st.max_q, w.scale, grid, ws)
    torch.cuda.synchronize()
    out = st.out.cpu().numpy().astype(np.float64)
    assert (out[cu[2]:cu[3]] == 0).all()
    keep_seq = [i for i in range(w.num_seqs) if i != 2]
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in keep_seq])
    T = np.diff(cu)[keep_seq]
    cu2 = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode_multi(w.query[rows], kc, vc, w.block_tables[keep_seq], cu2,
                              ctx[keep_seq], w.scale)
    assert_attention_close(out[rows], ref, f"balanced multi grid={grid}")


def test_multi_token_zero_length_sequence_and_partition_sizes():
    """A sequence with no query rows contributes none and leaves its
    neighbours' rows exact; results agree across partition sizes."""
    pa, runner = _gpu()
    w = workloads.make("c2_small_spec4")
    st = run_multi(w)
    cu = w.info["cu_seqlens_q"]
    keep = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in range(w.num_seqs) if i != 1])
    q2 = w.query[keep]
    T = np.diff(cu).copy()
    T[1] = 0
    cu2 = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode_multi(q2, kc, vc, w.block_tables, cu2, w.context_lens, w.scale)
    for P in (16, 512, 2048):
        out = torch.empty((len(keep),) + tuple(st.out.shape[1:]), dtype=torch.float16,
                          device="cuda")
        ws = torch.empty(pa.pa_multi_workspace_size(len(keep), w.num_heads, w.head_size,
                                                    w.max_blocks_per_seq, w.block_size, P),
                         dtype=torch.uint8, device="cuda")
        pa.pa_decode_multi(out, torch.from_numpy(q2).cuda(), st.key_cache, st.value_cache,
                           st.block_tables, torch.from_numpy(cu2).cuda(), st.context_lens,
                           4, w.scale, P, ws)
        torch.cuda.synchronize()
        assert_attention_close(out.cpu().numpy(), ref, f"zero-length seq, P={P}")


def test_multi_token_one_row_per_sequence_matches_decode():
    """With one query row per sequence pa_decode_multi computes decode: the
    same oracle bar as pa_decode on the decode workload."""
    pa, runner = _gpu()
    w = workloads.make("c3_small")
    st = run_gpu(w, "splitk")
    cu = torch.arange(w.num_seqs + 1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(st.out)
    ws = torch.empty(pa.pa_multi_workspace_size(w.num_seqs, w.num_heads, w.head_size,
                                                w.max_blocks_per_seq, w.block_size, 512),
                     dtype=torch.uint8, device="cuda")
    pa.pa_decode_multi(out, st.query, st.key_cache, st.value_cache, st.block_tables, cu,
                       st.context_lens, 1, w.scale, 512, ws)
    torch.cuda.synchronize()
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
    assert_attention_close(out.cpu().numpy(), ref, "multi with T=1")


def test_slot_mapping_parity_and_guards():
    pa, runner = _gpu()
    rng = np.random.default_rng(8)
    M, B = 12, 16
    table = rng.integers(0, 500, (5, M)).astype(np.int32)
    seq = rng.integers(0, 5, 300).astype(np.int32)
    pos = rng.integers(0, M * B, 300).astype(np.int32)
    seq[:3] = [5, -1, 0]
    pos[2] = M * B
    out = torch.empty(300, dtype=torch.int32, device="cuda")
    pa.pa_slot_mapping(out, torch.from_numpy(table).cuda(), torch.from_numpy(seq).cuda(),
                       torch.from_numpy(pos).cuda(), B)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[:3] == -1).all()
    ref = oracle.slot_mapping(table, seq[3:], pos[3:], B)
    assert (got[3:] == ref).all()


def test_empty_batch_is_noop():
    pa, runner = _gpu()
    z = torch.zeros((0, 8, 128), dtype=torch.float16, device="cuda")
    kc = torch.zeros((4, 16, 2, 128), dtype=torch.float16, device="cuda")
    bt = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    cl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    pa.pa_decode(z, z, kc, kc, bt, cl, 0.1)
    s = torch.zeros((0,), dtype=torch.int32, device="cuda")
    pa.pa_cache_write(z[:, :2], z[:, :2], kc, kc, s)
    torch.cuda.synchronize()

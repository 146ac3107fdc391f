"""Checks of the seeded workload generator (CPU only)."""
import numpy as np
import pytest

import oracle
import workloads


@pytest.mark.parametrize("name", ["c1", "c1_page_tables", "c2_small", "c3_small",
                                  "c4_small", "c4_r0_small", "c5_b32_small",
                                  "c5_b64_small", "c2", "c3"])
def test_tables_counts_and_refcounts(name):
    w = workloads.make(name)
    B, nb = w.block_size, w.num_blocks
    assert w.block_tables.dtype == np.int32 and w.block_tables.shape == (
        w.num_seqs, w.max_blocks_per_seq)
    assert (w.block_tables >= 0).all() and (w.block_tables < nb).all()
    ref = np.zeros(nb, np.int64)
    for i, n in enumerate(w.context_lens):
        k = oracle.blocks_needed(int(n), B)
        assert w.blocks_used[i] == k
        ref += np.bincount(w.block_tables[i, :k], minlength=nb)
    assert (ref == w.ref_cnt).all()
    if "prompts" not in w.info:
        assert ref.max() == 1            # drawn without replacement
    # unused entries point at unreferenced (poisoned) blocks
    for i, n in enumerate(w.context_lens):
        k = oracle.blocks_needed(int(n), B)
        assert (w.ref_cnt[w.block_tables[i, k:]] == 0).all()
    # finite fp16 garbage: no all-ones exponent field (Inf / NaN); checked in
    # chunks so no pool-sized temporary is allocated
    flat = w.pool_init.reshape(-1)
    for i in range(0, flat.size, 1 << 22):
        c = flat[i:i + (1 << 22)]
        assert ((c & np.uint16(0x7C00)) != np.uint16(0x7C00)).all()


def test_worked_example_tables_used_verbatim():
    w = workloads.make("c1_page_tables")
    assert list(w.context_lens) == [25, 47, 12]
    assert list(w.block_tables[0, :2]) == [3, 7]
    assert list(w.block_tables[1, :3]) == [0, 5, 9]
    assert list(w.block_tables[2, :1]) == [4]
    assert w.num_blocks == 64 and (w.ref_cnt == 0).sum() == 58


def test_determinism_and_seed_sensitivity():
    a = workloads.make("c3_small")
    b = workloads.make("c3_small")
    c = workloads.make("c3_small", seed=4242)
    assert (a.block_tables == b.block_tables).all()
    assert (a.query.view(np.uint16) == b.query.view(np.uint16)).all()
    assert (a.pool_init == b.pool_init).all()
    assert not (a.query.view(np.uint16) == c.query.view(np.uint16)).all()


def test_history_plus_step_cover_every_position_once():
    for name in ("c2_small", "c4_small", "c4_r0_small"):
        w = workloads.make(name)
        from tests.helpers import contiguous_kv
        kv = contiguous_kv(w)                # asserts no holes
        assert [len(k) for k, _ in kv] == list(w.context_lens)


def test_prefix_copy_on_write_bookkeeping():
    w = workloads.make("c4_small")
    n_s, Pn = w.info["samples"], w.info["prompts"]
    L = w.info["prompt_len"]
    for p in range(Pn):
        rows = w.block_tables[p * n_s:(p + 1) * n_s]
        full = int(L[p]) // 16
        # full prefix blocks are shared by all samples with ref_cnt = samples
        assert (rows[:, :full] == rows[0, :full]).all()
        assert (w.ref_cnt[rows[0, :full]] == n_s).all()
        # the partial prefix block ends up private to every sample
        part = rows[:, full]
        assert len(set(part.tolist())) == n_s
        assert (w.ref_cnt[part] == 1).all()
        assert int(w.info["prompt_tables"][p, full]) in part.tolist()
    assert w.info["hist_copies"] + w.info["step_copies"] == (n_s - 1) * Pn


def test_prefix_without_partial_block_has_no_copies():
    w = workloads.make("c4_r0_small")
    assert w.info["hist_copies"] + w.info["step_copies"] == 0
    assert (w.info["prompt_len"] % 16 == 0).all()


def test_length_recipes():
    w = workloads.make("c3")
    assert w.context_lens.min() >= 1 and w.context_lens.max() <= 8192
    big = workloads.make("c3", S=4000, garbage="finite", H=4, Hkv=1, D=64,
                         lens=workloads.PRESETS["c3"]["lens"], pool=("choice_scale", 1.25),
                         max_context=8192)
    med = np.median(big.context_lens)
    assert 600 < med < 800
    w5 = workloads.make("c5_b32_small")
    assert w5.context_lens.min() >= 1500 and w5.context_lens.max() <= 5000
    w2 = workloads.make("c2")
    assert w2.num_blocks == 4000 and w2.context_lens.max() <= 2048


def test_key_outliers_fraction():
    w = workloads.make("c5_b64_small")
    k = w.history[0].key.astype(np.float32)
    rms = np.sqrt((k ** 2).mean(axis=2))      # per (token, kv head) row
    frac = (rms > 4).mean()
    assert 0.005 < frac < 0.02


def test_nonfinite_garbage_mode():
    w = workloads.make("c1", garbage="nonfinite")
    f = w.pool_init.view(np.float16).astype(np.float32)
    assert not np.isfinite(f).all()


def test_pool_exhaustion_raises_memory_error():
    """The generator's allocator refuses to hand out more blocks than the
    pool holds (the scheduler's allocation failing when no block is free)."""
    with pytest.raises(MemoryError):
        workloads.make("c2_small", pool=("freelist_nb", 40))
    with pytest.raises(MemoryError):
        workloads.make("c4_small", pool=("freelist_nb", 100))


def test_reference_count_cannot_underflow():
    fl = workloads._FreeList(np.arange(4), 4)
    b = fl.pop()
    fl.drop(b)
    assert fl.ref[b] == 0
    with pytest.raises(ValueError):
        fl.drop(b)


@pytest.mark.parametrize("name", ["c4_small", "c4_r0_small", "c4"])
def test_copy_on_write_reference_counts(name):
    """Shared prompt blocks: every full block is held by all samples; the
    partial last block is copied for all but one sample, whose in-place write
    leaves the original with exactly one reference; copies are private."""
    w = workloads.make(name)
    B, n_s, P = w.block_size, w.info["samples"], w.info["prompts"]
    assert (w.ref_cnt >= 0).all()
    copies = [ph for ph in w.history if hasattr(ph, "src")]
    if w.step_copies is not None:
        copies.append(w.step_copies)
    src = np.concatenate([c.src for c in copies]) if copies else np.zeros(0, np.int32)
    dst = np.concatenate([c.dst for c in copies]) if copies else np.zeros(0, np.int32)
    partial = (w.info["prompt_len"] % B) != 0
    assert len(src) == int(partial.sum()) * (n_s - 1)
    assert len(set(dst.tolist())) == len(dst) and (w.ref_cnt[dst] == 1).all()
    pt, pu = w.info["prompt_tables"], w.info["prompt_used"]
    for p in range(P):
        full = int(w.info["prompt_len"][p]) // B
        assert (w.ref_cnt[pt[p, :full]] == n_s).all()
        if partial[p]:
            assert w.ref_cnt[pt[p, pu[p] - 1]] == 1
            assert (src == pt[p, pu[p] - 1]).sum() == n_s - 1

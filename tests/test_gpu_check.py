"""PA_CHECK=1: the decode and cache-write calls validate their device-side
preconditions on the device first and return PA_ERR_CHECK, with nothing
else launched, when one fails (out-of-range table entries, context longer
than the table, out-of-range or duplicate slots).  Valid inputs give the
normal result."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import oracle_pool
from tests.test_gpu_parity import assert_attention_close

pytestmark = pytest.mark.gpu

PA_ERR_CHECK = 7
CONTEXT, TABLE, SLOT_RANGE, DUPLICATE = 1, 2, 4, 8


@pytest.fixture
def checked(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    monkeypatch.setenv("PA_CHECK", "1")
    import paged_kv_cache_120_amd as pa
    from paged_kv_cache_120_amd import runner
    return pa, runner


def _setup(name="c3_small"):
    from paged_kv_cache_120_amd import runner
    w = workloads.make(name)
    st = runner.upload(w)
    runner.apply_history(w, st)
    torch.cuda.synchronize()
    return w, st


def _expect_check(pa, fn, bit):
    with pytest.raises(pa.PaError) as e:
        fn()
    assert e.value.status == PA_ERR_CHECK
    assert pa.pa_last_check() & bit, pa.pa_last_check()


@pytest.mark.parametrize("mode", ["single", "splitk", "balanced", "fused"])
def test_valid_inputs_pass_the_check(checked, mode):
    print(f"[check] valid {mode}", flush=True)
    pa, runner = checked
    w, st = _setup()
    runner.full_step(st, mode=mode)
    torch.cuda.synchronize()
    assert pa.pa_last_check() == 0
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"checked {mode}")


@pytest.mark.parametrize("mode", ["single", "splitk", "balanced", "fused"])
def test_out_of_range_table_entry(checked, mode):
    print(f"[check] table {mode}", flush=True)
    pa, runner = checked
    w, st = _setup()
    i = int(np.argmax(w.context_lens))
    bt = st.block_tables.clone()
    bt[i, 1] = w.num_blocks + 3                   # a block the decode reads
    st.block_tables = bt
    st.out.fill_(7.0)
    pool = st.pool.clone()
    _expect_check(pa, lambda: runner.decode_step(
        st, "fused_only" if mode == "fused" else mode), TABLE)
    torch.cuda.synchronize()
    assert bool((st.out == 7.0).all()), "output written after a failed check"
    assert torch.equal(st.pool.view(torch.int16), pool.view(torch.int16))


def test_context_longer_than_the_table(checked):
    pa, runner = checked
    w, st = _setup()
    cl = st.context_lens.clone()
    cl[0] = w.max_blocks_per_seq * w.block_size + 1
    st.context_lens = cl
    _expect_check(pa, lambda: runner.decode_step(st, "balanced"), CONTEXT)


def test_duplicate_and_out_of_range_slots_in_cache_write(checked):
    print("[check] cache write", flush=True)
    pa, runner = checked
    w, st = _setup()
    wr = st.write
    pa.pa_slot_mapping(wr.slots, wr.table, wr.seq, wr.pos, w.block_size)
    torch.cuda.synchronize()
    pool = st.pool.clone()
    dup = wr.slots.clone()
    dup[1] = dup[0]
    _expect_check(pa, lambda: pa.pa_cache_write(wr.key, wr.value, st.key_cache,
                                                st.value_cache, dup), DUPLICATE)
    far = wr.slots.clone()
    far[2] = w.num_blocks * w.block_size
    _expect_check(pa, lambda: pa.pa_cache_write(wr.key, wr.value, st.key_cache,
                                                st.value_cache, far), SLOT_RANGE)
    torch.cuda.synchronize()
    assert torch.equal(st.pool.view(torch.int16), pool.view(torch.int16))
    skip = wr.slots.clone()
    skip[0] = -1                                  # a skipped token is not a violation
    pa.pa_cache_write(wr.key, wr.value, st.key_cache, st.value_cache, skip)
    torch.cuda.synchronize()


def test_fused_step_into_a_shared_slot(checked):
    """Two sequences whose tables share the block their new token goes to
    (copy-on-write skipped) would both write one slot."""
    print("[check] fused shared slot", flush=True)
    pa, runner = checked
    w, st = _setup()
    bt = st.block_tables.clone()
    cl = st.context_lens.clone()
    bt[1] = bt[0]
    cl[1] = cl[0]
    st.block_tables, st.context_lens = bt, cl
    st.out.fill_(7.0)
    pool = st.pool.clone()
    _expect_check(pa, lambda: runner.decode_step(st, "fused_only"), DUPLICATE)
    torch.cuda.synchronize()
    assert bool((st.out == 7.0).all())
    assert torch.equal(st.pool.view(torch.int16), pool.view(torch.int16))
    # the same tables without the append are fine for a read-only decode
    runner.decode_step(st, "balanced")
    torch.cuda.synchronize()

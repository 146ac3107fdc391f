"""Shared-prefix decode (pa_decode_shared_prefix) on MI355X through the C
ABI, against the CPU oracle: the output must be the plain attention of every
sequence, elementwise |y - r| <= 2e-3 or |y - r| <= 1e-2 * |r|, with the
shared full blocks of each group read once for all its members."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import oracle_pool
from tests.test_gpu_parity import assert_attention_close

pytestmark = pytest.mark.gpu


def _runner():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_120_amd import runner
    return runner


def run_prefix(w, groups=None, max_group_size=None, ctx=None):
    runner = _runner()
    st = runner.upload_prefix(w, groups=groups)
    if max_group_size is not None:
        st.grp_max_size = max_group_size
    runner.apply_history(w, st)
    runner.write_step(st)
    if ctx is not None:
        st.context_lens.copy_(torch.from_numpy(ctx))
    runner.prefix_decode(st)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("name", ["c4_small", "c4_r0_small", "c4"])
def test_shared_prefix_parity(name):
    print(f"[prefix] {name}", flush=True)
    runner = _runner()
    w = workloads.make(name)
    off, mem, blk = runner.prefix_groups(w.block_tables, w.context_lens, w.block_size)
    assert len(blk) == w.info["prompts"] and (blk == 64).all()
    st = run_prefix(w)
    kc, vc = oracle_pool(w, oracle)
    gpool = st.pool.cpu().numpy().view(np.uint16)
    assert (gpool[0] == kc).all() and (gpool[1] == vc).all()
    ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"{name}/shared-prefix")


def test_no_groups_is_split_k_bitwise():
    runner = _runner()
    import paged_kv_cache_120_amd as pa
    w = workloads.make("c4_small")
    empty = (np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32))
    st = run_prefix(w, groups=empty)
    got = st.out.clone()
    runner.decode_step(st, "splitk")
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), st.out.view(torch.int16))


@pytest.mark.parametrize("P", [16, 256, 512, 2048])
def test_partition_sizes_and_members_ending_inside_the_prefix(P):
    """A member whose context ends inside a shared partition keeps its own
    key limit; partition sizes from one block to beyond the prefix."""
    runner = _runner()
    w = workloads.make("c4_small")
    w.partition_size = P
    groups = runner.prefix_groups(w.block_tables, w.context_lens, w.block_size)
    ctx = w.context_lens.copy()
    off, mem, blk = groups
    ctx[mem[1]] = 700          # inside the shared prefix (blocks 0..63)
    ctx[mem[2]] = 1            # a single token
    ctx[mem[off[1] + 1]] = 511
    st = run_prefix(w, groups=groups, ctx=ctx)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode(w.query, kc, vc, w.block_tables, ctx, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"P={P} short members")


def test_group_of_8_heads_more_members_than_one_tile_covers():
    """g = 8: one prefix tile holds 2 members; with max_group_size = 2 the
    other members of each group fall back to per-sequence partitions."""
    runner = _runner()
    w = workloads.make("c4_small", H=64, Hkv=8)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
    for mgs in [4, 2, 1]:
        st = run_prefix(w, max_group_size=mgs)
        assert_attention_close(st.out.cpu().numpy(), ref, f"g8 max_group_size={mgs}")


def test_zero_context_member_and_out_of_range_ids():
    runner = _runner()
    w = workloads.make("c4_small")
    off, mem, blk = runner.prefix_groups(w.block_tables, w.context_lens, w.block_size)
    # an id outside [0, S) inside a group is ignored
    mem2 = np.concatenate([mem[:off[1]], [w.num_seqs + 5], mem[off[1]:]]).astype(np.int32)
    off2 = off.copy()
    off2[1:] += 1
    ctx = w.context_lens.copy()
    ctx[mem[0]] = 0
    st = run_prefix(w, groups=(off2, mem2, blk), ctx=ctx)
    out = st.out.cpu().numpy().astype(np.float64)
    assert (out[mem[0]] == 0).all()
    keep = [i for i in range(w.num_seqs) if i != mem[0]]
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode(w.query[keep], kc, vc, w.block_tables[keep], ctx[keep], w.scale)
    assert_attention_close(out[keep], ref, "zero-context member")


@pytest.mark.parametrize("D,H,Hkv", [(64, 16, 8), (128, 32, 8), (64, 8, 8), (128, 16, 8)])
def test_shared_prefix_shapes(D, H, Hkv):
    """Head sizes 64/128 and groups 1-4: the whole-line prefix body where its
    tile holds a group's members, the 16-column body where it does not."""
    print(f"[prefix-shape] D{D} H{H}/{Hkv}", flush=True)
    w = workloads.make("c4_small", D=D, H=H, Hkv=Hkv)
    st = run_prefix(w)
    kc, vc = oracle_pool(w, oracle)
    ref = oracle.decode(w.query, kc, vc, w.block_tables, w.context_lens, w.scale)
    assert_attention_close(st.out.cpu().numpy(), ref, f"prefix D{D} g{H // Hkv}")

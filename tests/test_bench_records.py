"""bench.py reports committed counter summaries (HBM traffic, L2 hit rate,
LDS conflicts) only while they were taken on the current kernel sources, and
its host-side count of split ranges follows the balanced kernel's slicing
(CPU only)."""
import argparse
import os
import shutil

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _copy_tree(tmp_path):
    for f in bench.KERNEL_SOURCES:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), dst)
    (tmp_path / "profiles").mkdir()
    return tmp_path


def _args(cfg):
    return argparse.Namespace(config=cfg, mode="fused", partition=512)


def test_counters_follow_the_source_hash(tmp_path):
    root = _copy_tree(tmp_path)
    h = bench.kernel_source_hash(str(root))
    (root / "profiles" / "decode_c3_fused_counters.txt").write_text(
        "# comment: ignored\n"
        f"kernel_source_sha256_16: {h}\n"
        "l2_hit_rate_pct: 4.79\nlds_bank_conflict_pct: 49.11\nnote: text\n")
    c = bench.load_counters(_args("c3"), str(root))
    assert c == {"l2_hit_rate_pct": 4.79, "lds_bank_conflict_pct": 49.11}
    # another kernel source: the summary no longer describes it
    with open(root / bench.KERNEL_SOURCES[0], "a") as f:
        f.write("\n// changed\n")
    assert bench.load_counters(_args("c3"), str(root)) is None
    assert bench.load_counters(_args("c2"), str(root)) is None   # no file


def test_traffic_follows_the_source_hash(tmp_path):
    root = _copy_tree(tmp_path)
    h = bench.kernel_source_hash(str(root))
    p = root / "profiles" / "decode_c2_fused_traffic.txt"
    p.write_text(f"kernel_source_sha256_16: {h}\npartition_size: 512\n"
                 "hbm_bytes_per_launch: 793156835\n")
    assert bench.load_traffic(_args("c2"), str(root)) == 793156835
    p.write_text(f"kernel_source_sha256_16: {'0' * 16}\npartition_size: 512\n"
                 "hbm_bytes_per_launch: 793156835\n")
    assert bench.load_traffic(_args("c2"), str(root)) is None


def test_split_ranges_brute_force():
    """Cut pairs counted by walking every 16-token unit of the flat span."""
    class W:
        pass
    rng = np.random.default_rng(7)
    for trial in range(20):
        w = W()
        w.num_seqs = int(rng.integers(1, 9))
        w.num_kv_heads = int(rng.integers(1, 5))
        w.block_size = 16
        w.max_blocks_per_seq = 64
        w.context_lens = rng.integers(0, 1025, size=w.num_seqs).astype(np.int32)
        grid = int(rng.integers(1, 40))
        got = bench.balanced_split_ranges(w, grid)
        # brute force: owner workgroup of every token of every pair
        pc = bench.PAIR_COST
        spans = [((n + 15) // 16 * 16 + pc) if n > 0 else 0 for n in w.context_lens]
        total = sum(spans) * w.num_kv_heads
        if total == 0:
            assert got == 0
            continue
        C = -(-total // grid)
        C = (C + 15) // 16 * 16
        want, flat = 0, 0
        for n, sp in zip(w.context_lens, spans):
            for _ in range(w.num_kv_heads):
                if n > 0:
                    owners = {(flat + pc + t) // C for t in range(int(n))}
                    want += len(owners) if len(owners) > 1 else 0
                flat += sp
        assert got == want, (trial, got, want)

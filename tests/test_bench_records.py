"""bench.py reports committed counter summaries (HBM traffic, L2 hit rate,
LDS conflicts) only while they were taken on the current kernel sources, and
its host-side count of split ranges follows the balanced kernel's slicing
(CPU only)."""
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


def test_counters_follow_the_source_hash(tmp_path):
    root = _copy_tree(tmp_path)
    h = bench.kernel_source_hash(str(root))
    (root / "profiles" / "decode_c3_fused_counters.txt").write_text(
        "# comment: ignored\n"
        f"kernel_source_sha256_16: {h}\n"
        "l2_hit_rate_pct: 4.79\nlds_bank_conflict_pct: 49.11\nnote: text\n")
    c = bench.load_counters("c3", "fused", str(root))
    assert c.pop("source").startswith("profiles/decode_c3_fused_counters.txt")
    assert c == {"l2_hit_rate_pct": 4.79, "lds_bank_conflict_pct": 49.11}
    # another kernel source: the summary no longer describes it
    with open(root / bench.KERNEL_SOURCES[0], "a") as f:
        f.write("\n// changed\n")
    assert bench.load_counters("c3", "fused", str(root)) is None
    assert bench.load_counters("c2", "fused", str(root)) is None   # no file


def test_traffic_follows_the_source_hash(tmp_path):
    root = _copy_tree(tmp_path)
    h = bench.kernel_source_hash(str(root))
    p = root / "profiles" / "decode_c2_fused_traffic.txt"
    p.write_text(f"kernel_source_sha256_16: {h}\npartition_size: 512\n"
                 "hbm_bytes_per_launch: 793156835\n")
    t = bench.load_traffic("c2", "fused", 512, str(root))
    assert t["bytes"] == 793156835 and "rocprofv3" in t["source"]
    assert bench.load_traffic("c2", "fused", 1024, str(root)) is None
    p.write_text(f"kernel_source_sha256_16: {'0' * 16}\npartition_size: 512\n"
                 "hbm_bytes_per_launch: 793156835\n")
    assert bench.load_traffic("c2", "fused", 512, str(root)) is None


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
        pc = (bench.PAIR_COST, bench.FULL_PAIR_COST)[trial % 2]
        got = bench.balanced_split_ranges(w, grid, pc)
        # brute force: owner workgroup of every token of every pair
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


def test_roofline_counts_method_bytes_only():
    """The roofline's algorithmic bytes are the method's (K/V of exactly
    context_len tokens, query, output, table, the appended rows and slots);
    the partial-state handoff of cut pairs is reported apart."""
    import workloads
    w = workloads.make("c3_small")
    S, H, D = w.query.shape
    n = w.context_lens.astype(np.int64)
    kv = int(n.sum()) * 2 * w.num_kv_heads * D * 2
    table = int(((n + w.block_size - 1) // w.block_size).sum()) * 4
    appended = 2 * 2 * S * w.num_kv_heads * D * 2 + S * 4
    assert bench.balanced_kernel_bytes(w, 64, True) == kv + 2 * S * H * D * 2 + table + appended
    assert bench.balanced_kernel_bytes(w, 64, False) == kv + 2 * S * H * D * 2 + table
    ho = bench.balanced_handoff_bytes(w, 64)
    pc = bench.decode_pair_cost(w)
    assert ho == 2 * bench.balanced_split_ranges(w, 64, pc) * w.group * (D + 2) * 4 and ho > 0
    rec = bench.decode_record(w, "fused", 64, 0.01, 0.008)
    rf = rec["roofline"]
    assert rf["handoff_bytes"] == ho
    assert abs(rf["frac"] - rf["algorithmic_bytes"] / 0.008e-3 / 1e9 / 8000.0) < 1e-3


def test_host_cores_are_reported():
    c = bench.host_cores()
    assert c["sched_getaffinity"] >= 1 and 1 <= c["workers"] <= 16


def test_prefill_flops_brute_force():
    """The chunked-prefill flop count equals 4*D*H per visible (row, key)
    pair counted one by one (row j of a T-row chunk over n keys sees keys
    0 .. n - T + j)."""
    import workloads
    for name in ("c3_small_chunk64", "c1_prefill", "c3_small_spec4"):
        w = workloads.make(name)
        cu = w.info["cu_seqlens_q"]
        pairs = 0
        for i in range(w.num_seqs):
            n = int(w.context_lens[i])
            T = int(cu[i + 1] - cu[i])
            for j in range(T):
                pairs += sum(1 for t in range(n) if t <= n - T + j)
        assert bench.prefill_flops(w) == 4.0 * w.head_size * w.num_heads * pairs


def test_prefill_routing_rule():
    """The runner takes pa_prefill for more than 16 rows x heads per
    sequence when the launch has at least 256 workgroups and the longest
    context is at most 4x the mean; otherwise the decode-shaped kernels."""
    from types import SimpleNamespace
    pytest = __import__("pytest")
    runner = pytest.importorskip("paged_kv_cache_120_amd.runner")

    def step(S, H, Hkv, max_q, mx=2048, mean=1024.0):
        return SimpleNamespace(query=np.zeros((S * max_q, H, 1)),
                               key_cache=np.zeros((1, 16, Hkv, 1)),
                               block_tables=np.zeros((S, 1)), max_q=max_q,
                               max_context=mx, mean_context=mean)
    assert runner.prefill_preferred(step(16, 32, 8, 512))        # 2048 workgroups
    assert not runner.prefill_preferred(step(6, 32, 8, 64))      # 96 workgroups
    assert not runner.prefill_preferred(step(64, 32, 8, 4))      # 16 rows x heads
    assert runner.prefill_preferred(step(64, 32, 8, 8))          # 32 rows x heads, 512
    assert not runner.prefill_preferred(step(64, 32, 8, 16, mx=8192, mean=1150.0))
    assert runner.prefill_preferred(step(32, 40, 40, 17))        # g = 1, 1280 workgroups
    assert not runner.prefill_preferred(step(32, 40, 40, 16))

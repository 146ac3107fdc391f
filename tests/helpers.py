"""Test-side glue between the seeded workloads and the oracle / HIP path."""
import numpy as np


def contiguous_kv(w):
    """Per-sequence K/V in logical order, assembled straight from the token
    rows a workload writes (no slots, no pool): list of (K, V) fp16 arrays of
    shape [n_i, H_kv, D]."""
    S, Hkv, D = w.num_seqs, w.num_kv_heads, w.head_size
    Ks = [np.full((int(n), Hkv, D), np.nan, np.float16) for n in w.context_lens]
    Vs = [np.full((int(n), Hkv, D), np.nan, np.float16) for n in w.context_lens]
    phases = [p for p in w.history if hasattr(p, "seq")] + [w.step_write]
    prefix = "prompt_tables" in w.info
    for ph in phases:
        is_prompt = prefix and ph.table is w.info["prompt_tables"]
        for j in range(len(ph.seq)):
            r, p = int(ph.seq[j]), int(ph.pos[j])
            rows = ([r * w.info["samples"] + s for s in range(w.info["samples"])]
                    if is_prompt else [r])
            for i in rows:
                if p < len(Ks[i]):
                    Ks[i][p] = ph.key[j]
                    Vs[i][p] = ph.value[j]
    for K in Ks:
        assert not np.isnan(K.astype(np.float32)).any(), "hole in contiguous K"
    return list(zip(Ks, Vs))


def oracle_pool(w, oracle, include_step=True):
    """Pool after the history (and the decode step's writes) via the oracle."""
    kc = w.pool_init[0].copy()
    vc = w.pool_init[1].copy()
    phases = list(w.history)
    if include_step:
        phases += [w.step_copies, w.step_write]
    oracle.apply_phases(kc, vc, phases, w.block_size)
    return kc, vc

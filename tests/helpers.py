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


def written_amax(w):
    """Largest |K| and |V| over every token row the workload writes."""
    phases = [p for p in w.history if hasattr(p, "seq")] + [w.step_write]
    ka = max(float(np.abs(p.key.astype(np.float32)).max(initial=0)) for p in phases)
    va = max(float(np.abs(p.value.astype(np.float32)).max(initial=0)) for p in phases)
    return ka, va


def fp8_scales(w, kind):
    """Per-tensor scales: "calibrated" maps the largest written magnitude to
    448; "clamped" maps a quarter of it there (the largest values saturate);
    "unit" is 1.0 for both."""
    if kind == "unit":
        return 1.0, 1.0
    ka, va = written_amax(w)
    f = 1.0 if kind == "calibrated" else 0.25
    return ka * f / 448.0, va * f / 448.0


def oracle_pool_fp8(w, oracle, k_scale, v_scale, include_step=True):
    """fp8 pool (uint8 codes) after the history and the step, via the oracle;
    the initial garbage is the low byte of the fp16 garbage."""
    kc = (w.pool_init[0] & 0xFF).astype(np.uint8)
    vc = (w.pool_init[1] & 0xFF).astype(np.uint8)
    phases = list(w.history)
    if include_step:
        phases += [w.step_copies, w.step_write]
    oracle.apply_phases_fp8(kc, vc, phases, w.block_size, k_scale, v_scale)
    return kc, vc

"""FP8 (e4m3) KV cache on MI355X through the C ABI, against the CPU oracle.

The fp8 cache write must match the oracle's codes bit for bit over the whole
pool (the code is decided in fp32 on both sides); the decode must match the
oracle's float64 attention over the dequantised pool within the fp16 path's
tolerance, |y - r| <= 2e-3 or |y - r| <= 1e-2 * |r| elementwise."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.helpers import fp8_scales, oracle_pool_fp8
from tests.test_gpu_parity import EDGE_LENS, assert_attention_close

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_120_amd import runner
    return runner


def check_fp8(w, kind="calibrated", pairs=None, fused=False):
    runner = _gpu()
    ks, vs = fp8_scales(w, kind)
    st = runner.upload_fp8(w, ks, vs)
    runner.apply_history_fp8(w, st)
    runner.fp8_step(st, fused=fused)
    torch.cuda.synchronize()
    kc, vc = oracle_pool_fp8(w, oracle, ks, vs)
    ref_slots = oracle.slot_mapping(w.step_write.table, w.step_write.seq,
                                    w.step_write.pos, w.block_size)
    assert (st.write.slots.cpu().numpy() == ref_slots).all()
    gpool = st.pool.cpu().numpy()
    assert (gpool[0] == kc).all(), f"fp8 key cache differs in {(gpool[0] != kc).sum()} bytes"
    assert (gpool[1] == vc).all(), f"fp8 value cache differs in {(gpool[1] != vc).sum()} bytes"
    out = st.out.cpu().numpy()
    ref = oracle.decode_fp8(w.query, kc, vc, w.block_tables, w.context_lens, w.scale,
                            ks, vs, pairs=pairs)
    got = out if pairs is None else np.stack([out[i, h] for i, h in pairs])
    assert_attention_close(got, ref, f"{w.name}/fp8/{kind}")
    return st


SMALL = ["c1", "c2_small", "c3_small", "c4_small", "c5_b32_small", "c5_b64_small"]


@pytest.mark.parametrize("kind", ["calibrated", "clamped", "unit"])
@pytest.mark.parametrize("name", SMALL)
def test_fp8_parity_small(name, kind):
    print(f"[fp8] {name} {kind}", flush=True)
    check_fp8(workloads.make(name), kind)


@pytest.mark.parametrize("name", SMALL)
def test_fp8_fused_step_parity_small(name):
    """pa_decode_step_fp8: the quantised append lands bit-exactly and the
    attention uses it."""
    print(f"[fp8-fused] {name}", flush=True)
    check_fp8(workloads.make(name), "calibrated", fused=True)


@pytest.mark.parametrize("D,B,H,Hkv", [(128, 16, 32, 8), (64, 64, 16, 2),
                                       (128, 32, 8, 8), (64, 16, 8, 4),
                                       (128, 64, 16, 8), (64, 16, 16, 4)])
@pytest.mark.parametrize("fused", [False, True])
def test_fp8_edge_lengths(D, B, H, Hkv, fused):
    print(f"[fp8-edge] D{D} B{B} H{H}/{Hkv} fused={fused}", flush=True)
    w = workloads.make("c1", D=D, B=B, H=H, Hkv=Hkv, lens=EDGE_LENS,
                       pool=("choice_scale", 1.3), max_context=2048, seed=D + B + H)
    check_fp8(w, fused=fused)


@pytest.mark.parametrize("name,fused", [("c2", False), ("c3", False), ("c2", True),
                                        ("c3", True)])
def test_fp8_parity_full(name, fused):
    """Every (sequence, query head) output of the full workloads."""
    print(f"[fp8-full] {name} fused={fused}", flush=True)
    check_fp8(workloads.make(name), fused=fused)


def test_fp8_zero_context_and_any_grid():
    runner = _gpu()
    import paged_kv_cache_120_amd as pa
    w = workloads.make("c3_small")
    ks, vs = fp8_scales(w, "calibrated")
    st = runner.upload_fp8(w, ks, vs)
    runner.apply_history_fp8(w, st)
    runner.run_phase_fp8(st.write, st.pool, st.block_size, ks, vs)
    kc, vc = oracle_pool_fp8(w, oracle, ks, vs)
    ctx = w.context_lens.copy()
    ctx[1] = 0
    st.context_lens.copy_(torch.from_numpy(ctx))
    keep = [i for i in range(w.num_seqs) if i != 1]
    ref = oracle.decode_fp8(w.query[keep], kc, vc, w.block_tables[keep], ctx[keep],
                            w.scale, ks, vs)
    S, H, D = w.query.shape
    for grid in [1, 7, 300, st.grid]:
        bws = pa.pa_balanced_workspace_size(S, H, w.num_kv_heads, D, grid)
        ws = torch.zeros(bws, dtype=torch.uint8, device=st.pool.device)
        st.out.fill_(7.0)
        pa.pa_decode_balanced_fp8(st.out, st.query, st.key_cache, st.value_cache,
                                  st.block_tables, st.context_lens, st.scale, ks, vs,
                                  grid, ws)
        torch.cuda.synchronize()
        out = st.out.cpu().numpy().astype(np.float64)
        assert (out[1] == 0).all()
        assert_attention_close(out[keep], ref, f"fp8 grid {grid}")


def test_fp8_pool_accepts_float8_dtype_and_halves_the_bytes():
    runner = _gpu()
    w = workloads.make("c2_small")
    ks, vs = fp8_scales(w, "calibrated")
    st = runner.upload_fp8(w, ks, vs)
    runner.apply_history_fp8(w, st)
    runner.run_phase_fp8(st.write, st.pool, st.block_size, ks, vs)
    st.pool = st.pool.view(torch.float8_e4m3fn)
    runner.fp8_decode(st)
    torch.cuda.synchronize()
    assert st.pool.element_size() == 1
    kc, vc = oracle_pool_fp8(w, oracle, ks, vs)
    ref = oracle.decode_fp8(w.query, kc, vc, w.block_tables, w.context_lens, w.scale,
                            ks, vs)
    assert_attention_close(st.out.cpu().numpy(), ref, "float8_e4m3fn pool")

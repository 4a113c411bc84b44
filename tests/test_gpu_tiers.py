"""GPU: the consumer of the compact miss list (a second weight pool computes the rows routed to
absent experts; moe_combine_tiers adds them in row order).  On every compact case, and on each
FFN path the shapes allow:

* the two-tier output matches the oracle's all-resident layer (the stated tolerances);
* it equals, bit for bit, the GPU layer over one pool holding every expert on the same path
  (same rows per expert, same per-row arithmetic, same sum order);
* the pool tier computes exactly the resident tier's miss rows.
"""
import dataclasses
import sys

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu

CASES = {
    "compact": gen.config("compact_mxfp4", T=53, H=512, E=40, I=160, k=6, resident=13),
    "compact_t1": gen.config("compact_mxfp4", T=1, H=256, E=16, I=128, k=4, resident=5),
    "compact_gemm": gen.config("compact_mxfp4", T=300, H=512, E=12, I=256, k=4, resident=5),
    "compact_multigroup": gen.config("compact_mxfp4", T=700, H=256, E=48, I=128, k=5, resident=17),
    "compact_max_e_k": gen.config("compact_mxfp4", T=2, H=128, E=1024, I=128, k=64, resident=700),
    "compact_fp8": gen.config("prefill_fp8_zipf", T=64, H=256, E=24, I=128, k=4, resident=9),
    # bf16 weights with router weights (logits computed on the GPU)
    "compact_bf16": gen.config("decode_bf16", T=96, H=512, E=24, I=256, k=4, resident=9),
}


def _gemm_ok(cfg, mode):
    if cfg.wdtype == "bf16":
        return mode == "A" and cfg.H % 64 == 0 and cfg.I % 64 == 0
    return cfg.H % 128 == 0 and cfg.I % 128 == 0 and (mode == "A" or (cfg.H <= 4096 and cfg.I <= 4096))


@pytest.fixture(scope="module", params=list(CASES))
def tier_case(request):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpu_cases import GpuCase
    from oracle import moe_oracle as O
    cfg = CASES[request.param]
    inp = gen.make_inputs(cfg)
    pool_map, pool = gen.make_pool_map(cfg)
    pool_inp = dataclasses.replace(inp, cfg=cfg.replace(resident=int(pool.size)), slot_map=pool_map,
                                   slot_expert=pool, weights=gen.stack_weights(cfg, pool))
    full_w = gen.stack_weights(cfg, range(cfg.E))
    full_inp = dataclasses.replace(inp, cfg=cfg.replace(resident=None), slot_map=None,
                                   slot_expert=np.arange(cfg.E, dtype=np.int32), weights=full_w)
    ref = O.layer(inp.x, cfg.xdtype, full_w, cfg.wdtype, cfg.H, cfg.I, cfg.E, cfg.k, cfg.score, cfg.renorm,
                  w_router=inp.w_router, logits=inp.logits)
    return request.param, cfg, GpuCase(inp), GpuCase(pool_inp), GpuCase(full_inp), ref


@pytest.mark.parametrize("path,mode", [("gemv", "A"), ("gemm", "A"), ("gemv", "B"), ("gemm", "B")])
def test_two_tiers_equal_one_pool(tier_case, path, mode):
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import assert_fp_close
    name, cfg, ga, gb, gf, ref = tier_case
    if path == "gemm" and not _gemm_ok(cfg, mode):
        pytest.skip("shape outside the matrix-core path")
    print(f"[gpu-tiers] case={name} path={path} mode={mode} T={cfg.T} E={cfg.E} k={cfg.k} S={cfg.S}", flush=True)
    sys.stdout.flush()
    p = moe.MOE_PATH_GEMV if path == "gemv" else moe.MOE_PATH_GEMM
    m = moe.MOE_MODE_A if mode == "A" else moe.MOE_MODE_B
    # tier a: the resident slots (routing, permutation, misses, FFN)
    ra = ga.route_permute()
    ya = ga.expert_ffn(ra["perm"], ra["slot_offsets"], path=p, mode=m)
    # tier b: the pool of absent experts, permuted with its own map from the same routing
    rb = gb.permute(ra["topk_idx"], ra["topk_w"])
    yb = gb.expert_ffn(rb["perm"], rb["slot_offsets"], path=p, mode=m)
    out = ga.combine_tiers(ya, ra["inv_perm"], yb, rb["inv_perm"], ra["topk_w"])
    # the pool tier's rows are exactly the resident tier's misses
    assert np.array_equal(np.sort(rb["perm"]), np.nonzero(ra["inv_perm"] < 0)[0])
    assert rb["perm"].size == ra["miss_count"]
    # one pool with every expert, same path and mode
    rf = gf.route_permute()
    assert np.array_equal(rf["topk_idx"], ra["topk_idx"]) and np.array_equal(rf["topk_w"], ra["topk_w"])
    yf = gf.expert_ffn(rf["perm"], rf["slot_offsets"], path=p, mode=m)
    one = gf.combine(yf, rf["inv_perm"], rf["topk_w"])
    assert np.array_equal(out, one), f"{name}: two tiers differ from one pool in {np.sum(out != one)} elements"
    if mode == "A":
        # logits computed on the GPU (router weights) may flip near-ties: those tokens are left out
        from gpu_cases import routing_mismatches
        keep = np.ones(cfg.T, bool)
        keep[list(routing_mismatches(ra["topk_idx"], ref))] = False
        assert_fp_close(out[keep], ref["out"][keep], f"{name} two-tier layer ({path})")


@pytest.mark.parametrize("mode", ["A", "B"])
def test_two_tiers_full_size(mode):
    """The compact workload at its stated size (T = 4096, 110 of 384 experts resident, MXFP4, Zipf
    routing; the matrix-core path AUTO takes): the resident tier plus the pool of the 274 absent
    experts equals the layer over one pool of all 384 experts bit for bit (the MoET hybrid table's
    identity row: compact calls plus the rows computed elsewhere reproduce the all-resident path)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import GpuCase
    cfg = gen.config("compact_mxfp4", T=4096)
    print(f"[gpu-tiers] full size T={cfg.T} E={cfg.E} S={cfg.S} mode {mode}: generating", flush=True)
    full_w = gen.stack_weights(cfg, range(cfg.E))
    inp = gen.make_inputs(cfg, with_weights=False)
    pick = lambda ex: {k_: (None if v is None else np.ascontiguousarray(v[np.asarray(ex)])) for k_, v in full_w.items()}
    inp.weights = pick(inp.slot_expert)
    pool_map, pool = gen.make_pool_map(cfg)
    pool_inp = dataclasses.replace(inp, cfg=cfg.replace(resident=int(pool.size)), slot_map=pool_map,
                                   slot_expert=pool, weights=pick(pool))
    full_inp = dataclasses.replace(inp, cfg=cfg.replace(resident=None), slot_map=None,
                                   slot_expert=np.arange(cfg.E, dtype=np.int32), weights=full_w)
    ga, gb, gf = GpuCase(inp), GpuCase(pool_inp), GpuCase(full_inp)
    p = moe.MOE_PATH_AUTO
    m = moe.MOE_MODE_A if mode == "A" else moe.MOE_MODE_B
    assert moe.moe_resolve_path(ga.w.desc, cfg.T, cfg.k, p, m) == moe.MOE_PATH_GEMM
    print(f"[gpu-tiers] full size: two tiers", flush=True)
    ra = ga.route_permute()
    ya = ga.expert_ffn(ra["perm"], ra["slot_offsets"], path=p, mode=m)
    rb = gb.permute(ra["topk_idx"], ra["topk_w"])
    yb = gb.expert_ffn(rb["perm"], rb["slot_offsets"], path=p, mode=m)
    out = ga.combine_tiers(ya, ra["inv_perm"], yb, rb["inv_perm"], ra["topk_w"])
    assert np.array_equal(np.sort(rb["perm"]), np.nonzero(ra["inv_perm"] < 0)[0])
    assert rb["perm"].size == ra["miss_count"] and ra["miss_count"] > 10000
    print(f"[gpu-tiers] full size: one pool of {cfg.E} experts", flush=True)
    rf = gf.route_permute()
    assert np.array_equal(rf["topk_idx"], ra["topk_idx"]) and np.array_equal(rf["topk_w"], ra["topk_w"])
    yf = gf.expert_ffn(rf["perm"], rf["slot_offsets"], path=p, mode=m)
    one = gf.combine(yf, rf["inv_perm"], rf["topk_w"])
    assert np.array_equal(out, one), f"two tiers differ from one pool in {np.sum(out != one)} elements"
    print(f"[gpu-tiers] full size mode {mode}: identical ({ra['miss_count']} miss rows)", flush=True)

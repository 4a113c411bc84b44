"""GPU parity: the HIP path through the C ABI against the CPU oracle on seeded inputs.

Shrunken cases finish in the oracle in seconds yet span several work-group tiles with ragged
tails (T, I and H not multiples of the tile sizes, uneven and empty slot groups); every stage is
also checked on its own with the oracle's results as its inputs."""
import sys

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": gen.config("tiny"),
    "f32_sigmoid_norenorm": gen.config("tiny", T=21, score="sigmoid", renorm=False, I=136),
    "bf16_ragged": gen.config("decode_bf16", T=37, H=512, E=24, I=136, k=4),
    "fp8_ragged": gen.config("decode_fp8", T=29, H=384, E=20, I=272, k=3),
    "fp8_zipf": gen.config("prefill_fp8_zipf", T=300, H=256, E=32, I=128, k=8),
    "mxfp4_compact": gen.config("compact_mxfp4", T=53, H=512, E=40, I=160, k=6, resident=13),
    "mxfp4_compact_t1": gen.config("compact_mxfp4", T=1, H=256, E=16, I=128, k=4, resident=5),
    # shapes for the matrix-core path: bf16 weights (H, I multiples of 64) with several M tiles per
    # slot and ragged 32-row blocks; FP8 with a ragged last N tile in both projections (I = 384:
    # three 128-column gate/up tiles; H = 384: a 256- and a 128-column down tile); MXFP4 with 20
    # E8M0 scales per gate/up row (H = 640, copied rather than loaded rotated) and a compact map
    "bf16_gemm": gen.config("decode_bf16", T=70, H=512, E=12, I=192, k=4),
    "fp8_big_groups": gen.config("prefill_fp8_zipf", T=400, H=384, E=8, I=384, k=2),
    "mxfp4_gemm_compact": gen.config("compact_mxfp4", T=200, H=640, E=24, I=384, k=6, resident=9),
    # the matrix-core path with FP8 / MXFP4 weights (K multiples of 128): several M tiles per slot
    "fp8_gemm_groups": gen.config("prefill_fp8_zipf", T=400, H=384, E=4, I=256, k=2),
    "mxfp4_gemm_groups": gen.config("compact_mxfp4", T=300, H=512, E=12, I=256, k=4, resident=5),
    # fused routing + permutation with the small-batch ranking: an odd row count (77, over one
    # wave of rows) with compact misses
    "mxfp4_compact_r77": gen.config("compact_mxfp4", T=11, H=256, E=40, I=128, k=7, resident=11),
    # more than 2048 rows: the permutation runs as several work-groups (ragged last group), with
    # compact misses
    "mxfp4_multigroup_perm": gen.config("compact_mxfp4", T=700, H=256, E=48, I=128, k=5, resident=17),
    # router logits for 3 and 1 tokens with an odd expert count (the last work-group owns one
    # expert row); router bias on the first
    "bf16_router_t3": gen.config("decode_bf16", T=3, H=256, E=13, I=128, k=2),
    "bf16_router_t1": gen.config("decode_bf16", T=1, H=320, E=7, I=64, k=3),
    # the largest expert count and top-k the ABI takes (E = 1024: 16 values per lane in the top-k;
    # k = 64): 128 rows (the last size ranked by direct counts), 192 rows (counter passes in the
    # fused kernel), and a compact map of 700 resident experts out of 1024 with misses
    "max_e_k_r128": gen.config("decode_bf16", T=2, H=128, E=1024, I=64, k=64),
    "max_e_k_r192": gen.config("decode_bf16", T=3, H=128, E=1024, I=64, k=64),
    "max_e_k_compact": gen.config("compact_mxfp4", T=2, H=128, E=1024, I=128, k=64, resident=700),
    # the largest H and I the ABI takes (8192): FP8 GEMM tiles hold 64 block scales per row (their
    # whole scale array), 64 K steps; the router GEMV covers all of H; 64 KiB of staged activations
    "fp8_max_dims": gen.config("decode_fp8", T=3, H=8192, E=2, I=8192, k=1),
    "bf16_max_dims": gen.config("decode_bf16", T=2, H=8192, E=2, I=8192, k=1),
    # either side of the size from which mode A keeps a as a bf16 (hi, lo) pair (H*I >= 2^25):
    # H = 8192, I = 4096 splits; H = 8192, I = 2048 keeps one bf16 a
    "fp8_split_a": gen.config("decode_fp8", T=9, H=8192, E=3, I=4096, k=2),
    "fp8_no_split": gen.config("decode_fp8", T=9, H=8192, E=3, I=2048, k=2),
    # degenerate routing: every expert chosen (k = E), and a single expert (E = k = 1)
    "k_equals_e": gen.config("decode_bf16", T=5, H=256, E=8, I=128, k=8),
    "single_expert": gen.config("decode_bf16", T=7, H=256, E=1, I=64, k=1),
    # down-projection rows of exactly 64 16-byte chunks (16 lanes per row, two rows per step)
    "fp8_down64": gen.config("decode_fp8", T=29, H=256, E=20, I=1024, k=3),
    "bf16_down64": gen.config("decode_bf16", T=6, H=256, E=12, I=512, k=2),
}


def _elem_tol(name, path):
    from gpu_cases import ELEM_TOL
    return ELEM_TOL


def _gemm_capable(cfg):
    step = 64 if cfg.wdtype == "bf16" else 128
    return cfg.wdtype != "f32" and cfg.H % step == 0 and cfg.I % step == 0


def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _banner(name, cfg):
    print(f"[gpu-parity] case={name} T={cfg.T} H={cfg.H} E={cfg.E} I={cfg.I} k={cfg.k} "
          f"w={cfg.wdtype} S={cfg.S}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=list(SMALL))
def small_case(request):
    _gpu()
    from gpu_cases import GpuCase, run_oracle
    cfg = SMALL[request.param]
    inp = gen.make_inputs(cfg, bias=request.param in ("bf16_ragged", "bf16_router_t3"))
    return request.param, inp, GpuCase(inp), run_oracle(inp)


def test_route_stage(small_case):
    from gpu_cases import check_routing
    name, inp, g, ref = small_case
    _banner(name + "/route", inp.cfg)
    idx, w, lo = g.route()
    check_routing(idx, w, ref)
    if lo is not None:
        np.testing.assert_allclose(lo, ref["logits"] if inp.bias is None else ref["logits"] + inp.bias,
                                   rtol=1e-4, atol=1e-5 * np.abs(ref["logits"]).max())


def test_permute_stage(small_case):
    from gpu_cases import check_permute
    name, inp, g, ref = small_case
    _banner(name + "/permute", inp.cfg)
    res = g.permute(ref["topk_idx"], ref["topk_w"])
    check_permute(res, ref)


def test_route_permute_stage(small_case):
    # one launch for T <= 16 (top-k and permutation share a work-group), two or more above
    from gpu_cases import check_permute, check_routing
    name, inp, g, ref = small_case
    _banner(name + "/route_permute", inp.cfg)
    res = g.route_permute()
    flipped = check_routing(res["topk_idx"], res["topk_w"], ref)
    if not flipped:
        check_permute(res, ref)


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_expert_ffn_stage(small_case, path):
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import assert_fp_close
    name, inp, g, ref = small_case
    _banner(f"{name}/expert_ffn/{path}", inp.cfg)
    p = moe.MOE_PATH_GEMV if path == "gemv" else moe.MOE_PATH_GEMM
    if path == "gemm" and not _gemm_capable(inp.cfg):
        with pytest.raises(moe.MoeError) as ei:
            g.expert_ffn(ref["perm"], ref["slot_offsets"], path=p)
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
        return
    y = g.expert_ffn(ref["perm"], ref["slot_offsets"], path=p)
    tol = _elem_tol(name, path)
    assert_fp_close(y, ref["y_perm"], f"{name} y_perm ({path})", elem_tol=tol, scale_tol=tol)


def test_combine_stage(small_case):
    from gpu_cases import assert_fp_close
    name, inp, g, ref = small_case
    _banner(name + "/combine", inp.cfg)
    out = g.combine(ref["y_perm"].astype(np.float32), ref["inv_perm"], ref["topk_w"].astype(np.float32))
    assert_fp_close(out, ref["out"], f"{name} combine")


@pytest.mark.parametrize("path", ["auto", "gemv", "gemm"])
def test_layer(small_case, path):
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import assert_fp_close, check_misses, check_routing
    name, inp, g, ref = small_case
    _banner(f"{name}/layer/{path}", inp.cfg)
    if path == "gemm" and not _gemm_capable(inp.cfg):
        pytest.skip("shape outside the matrix-core path (covered by the UNSUPPORTED check)")
    res = g.layer(path={"auto": moe.MOE_PATH_AUTO, "gemv": moe.MOE_PATH_GEMV, "gemm": moe.MOE_PATH_GEMM}[path])
    flipped = check_routing(res["topk_idx"], res["topk_w"], ref)
    keep = np.array([t not in flipped for t in range(inp.cfg.T)], bool)
    tol = _elem_tol(name, path)
    assert_fp_close(res["out"][keep], ref["out"][keep], f"{name} layer out", elem_tol=tol, scale_tol=tol)
    if not flipped:
        check_misses(res, ref)


def test_layer_is_deterministic(small_case):
    name, inp, g, ref = small_case
    _banner(name + "/determinism", inp.cfg)
    a = g.layer()
    b = g.layer()
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["topk_idx"], b["topk_idx"])


def test_empty_batch():
    _gpu()
    from gpu_cases import GpuCase
    cfg = gen.config("decode_bf16", T=0, H=256, E=16, I=128, k=4)
    inp = gen.make_inputs(cfg)
    g = GpuCase(inp)
    res = g.layer()
    assert res["out"].shape == (0, cfg.H)
    p = g.permute(np.zeros((0, cfg.k), np.int32), np.zeros((0, cfg.k), np.float32))
    assert np.all(p["counts"] == 0) and np.all(p["slot_offsets"] == 0)


def test_all_rows_missing():
    # compact map with no routed expert resident: zero output rows, every row in the miss list
    _gpu()
    from gpu_cases import GpuCase, check_misses, run_oracle
    cfg = gen.config("compact_mxfp4", T=6, H=256, E=16, I=128, k=2, resident=3)
    inp = gen.make_inputs(cfg)
    lg = np.zeros((cfg.T, cfg.E), np.float32)
    resident = np.nonzero(inp.slot_map >= 0)[0]
    lg[:, resident] = -10.0
    inp.logits = lg
    g = GpuCase(inp)
    ref = run_oracle(inp)
    res = g.layer()
    assert np.all(res["out"] == 0)
    check_misses(res, ref)
    assert res["miss_count"] == cfg.T * cfg.k


def test_out_of_range_expert_sets_device_error():
    _gpu()
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import GpuCase
    cfg = gen.config("decode_bf16", T=4, H=256, E=16, I=128, k=2)
    g = GpuCase(gen.make_inputs(cfg))
    idx = np.array([[0, 1], [2, 99], [3, 4], [5, -1]], np.int32)
    with pytest.raises(moe.MoeError) as ei:
        g.permute(idx, np.full((4, 2), 0.5, np.float32))
    assert ei.value.status == moe.MOE_ERR_DEVICE


@pytest.mark.parametrize("T", [5, 40])
def test_exact_ties_resolved_by_expert_id(T):
    # logits on a coarse grid: many exactly equal values; given logits (no GEMV) reach both sides
    # unchanged, so the (logit desc, id asc) order must agree on every token, ties included
    _gpu()
    from gpu_cases import GpuCase, run_oracle
    cfg = gen.config("decode_fp8", T=T, H=256, E=200, I=128, k=8)
    inp = gen.make_inputs(cfg)
    rng = np.random.default_rng(77)
    inp.logits = (rng.integers(0, 6, (T, cfg.E)) * 0.25).astype(np.float32)
    _banner(f"ties/T{T}", cfg)
    g = GpuCase(inp)
    ref = run_oracle(inp)
    res = g.route_permute()
    assert np.array_equal(res["topk_idx"], ref["topk_idx"])
    np.testing.assert_allclose(res["topk_w"], ref["topk_w"], rtol=1e-6)


def _near_tie_logits(T, E, rng):
    """Per token: background logits in [-2, 0) and a cluster of values a few float steps apart
    near 1.0 (0.25 for every fourth token), placed on random experts.  The cluster spans 600
    float steps, so its members often agree in all but the last 9 bits, with a few exact ties;
    the selection must still follow the exact logits (then the lower expert id)."""
    lg = (-2.0 * rng.random((T, E))).astype(np.float32)
    for t in range(T):
        base = np.float32(1.0 if t % 4 else 0.25)
        n = int(rng.integers(2, 14))
        steps = rng.integers(0, 600, n)
        if t % 3 == 0:
            steps[1] = steps[0]                    # one exact tie
        e = rng.choice(E, n, replace=False)
        vals = np.full(n, base, np.float32).view(np.uint32) + steps.astype(np.uint32)
        lg[t, e] = vals.view(np.float32)
        if t % 5 == 1:                             # seven clear winners above a near-tied 8th place
            lg[t, rng.choice(np.setdiff1d(np.arange(E), e), 7, replace=False)] = 3.0 + np.arange(7, dtype=np.float32)
    return lg


@pytest.mark.parametrize("name,T,E,k", [("decode_bf16", 4, 384, 8), ("decode_fp8", 37, 384, 8),
                                        ("decode_fp8", 3, 200, 4), ("compact_mxfp4", 1, 384, 8),
                                        ("decode_fp8", 2, 500, 8)])
def test_near_ties_select_by_exact_logit(name, T, E, k):
    # logits that agree in all but their last bits: the router's top-k, the fused top-k and
    # permutation, and (T <= 4) the two-launch decode layer must all select and order the experts
    # exactly as the oracle does
    _gpu()
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import GpuCase, run_oracle
    cfg = gen.config(name, T=T, H=256, E=E, I=128, k=k, router="uniform",
                     **({"resident": min(E, 120)} if name == "compact_mxfp4" else {}))
    inp = gen.make_inputs(cfg)
    inp.logits = _near_tie_logits(T, E, np.random.default_rng(1000 + T + E))
    _banner(f"near-ties/{name}/T{T}/E{E}/k{k}", cfg)
    g = GpuCase(inp)
    ref = run_oracle(inp)
    idx, w, _ = g.route()
    assert np.array_equal(idx, ref["topk_idx"]), "router top-k"
    np.testing.assert_allclose(w, ref["topk_w"], rtol=1e-6)
    res = g.route_permute()
    assert np.array_equal(res["topk_idx"], ref["topk_idx"]), "route + permute top-k"
    assert np.array_equal(res["topk_w"].view(np.uint32), w.view(np.uint32))
    if T <= 4:
        lay = g.layer(path=moe.MOE_PATH_GEMV, mode=moe.MOE_MODE_A)
        assert np.array_equal(lay["topk_idx"].reshape(T, k), ref["topk_idx"]), "decode layer top-k"
        assert np.array_equal(lay["topk_w"].reshape(T, k).view(np.uint32), w.view(np.uint32))

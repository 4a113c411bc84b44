"""GPU: the two-launch decode layer.  For batches of at most 4 tokens and 32 rows (MXFP4; 8 rows for the other formats) on the GEMV path
(mode A) moe_layer runs the layer in two launches: every work-group of the first selects the
batch's experts itself and computes gate/up for one slot, the second computes the down projection
of every row for a block of output columns and combines in place.  The staged launches (route and
permute, the expert FFN on the GEMV path, combine) compute the same layer in four or five.

The two flows must agree bit for bit -- top-k ids and gates, the compact miss list and the output
-- since each element is formed by the same arithmetic (the routing card of the pages' layer
and the two-tier identity of the MoET hybrid table rest on that); and the layer meets the oracle's
tolerances.  Cases cover every weight format, both activation and output formats, router weights
and given logits, softmax and sigmoid scores, a selection bias, compact maps, slots holding several
rows of the batch, k = 16, E above 512, and the decode shapes at their stated sizes (T = 1)."""
import dataclasses
import sys

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu

CASES = {
    # bf16 weights, router weights (logits computed on the GPU), sigmoid scores
    "bf16_router_T2": (gen.config("decode_bf16", T=2, H=512, E=64, I=256, k=4), False),
    "bf16_T1_f32out": (gen.config("decode_bf16", T=1, H=512, E=40, I=128, k=8, out_dtype="f32"), False),
    "bf16_x_f32": (gen.config("decode_bf16", T=2, H=256, E=24, I=192, k=4, xdtype="f32"), False),
    # FP8 block-scaled weights, given logits; I = 1024 takes the 16-lane down rows
    "fp8_T2": (gen.config("decode_fp8", T=2, H=512, E=48, I=256, k=4), False),
    "fp8_I1024": (gen.config("decode_fp8", T=2, H=256, E=16, I=1024, k=2), False),
    "fp8_bias": (gen.config("decode_fp8", T=4, H=256, E=32, I=128, k=2), True),
    # MXFP4 compact maps (rows routed to absent experts go to the miss list)
    "mxfp4_compact_T1": (gen.config("compact_mxfp4", T=1, H=512, E=96, I=256, k=8, resident=30), False),
    "mxfp4_compact_T4": (gen.config("compact_mxfp4", T=4, H=512, E=96, I=256, k=4, resident=30), False),
    "mxfp4_compact_T4_k8": (gen.config("compact_mxfp4", T=4, H=512, E=96, I=256, k=8, resident=40), False),
    "mxfp4_E600_k16": (gen.config("compact_mxfp4", T=1, H=256, E=600, I=128, k=16, resident=200), False),
    # fp32 weights and activations, softmax scores
    "f32_softmax": (gen.config("tiny", T=2, H=256, E=8, I=128, k=2), False),
    # few experts: slots hold several of the batch's rows
    "shared_slots": (gen.config("decode_fp8", T=4, H=256, E=6, I=128, k=2, score="softmax"), False),
    "k16_T1": (gen.config("compact_mxfp4", T=1, H=256, E=128, I=128, k=16, resident=100), False),
    # the decode shapes at their stated sizes
    "compact_mxfp4_T1_full": (gen.config("compact_mxfp4", T=1), False),
    "compact_mxfp4_T4_full": (gen.config("compact_mxfp4", T=4), False),
    "decode_fp8_T1_full": (gen.config("decode_fp8", T=1), False),
    "decode_bf16_T1_full": (gen.config("decode_bf16", T=1), False),
}


def _staged(g):
    """The layer through the staged launches, GEMV path."""
    import routed_expert_ffn_05_amd as moe
    r = g.route_permute()
    y = g.expert_ffn(r["perm"], r["slot_offsets"], path=moe.MOE_PATH_GEMV, mode=moe.MOE_MODE_A)
    out = g.combine(y, r["inv_perm"], r["topk_w"])
    return r, out


@pytest.mark.parametrize("name", list(CASES))
def test_fused_decode_equals_staged_launches(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import GpuCase, assert_fp_close, check_routing, run_oracle
    cfg, with_bias = CASES[name]
    print(f"[gpu-decode-fused] case={name} T={cfg.T} H={cfg.H} E={cfg.E} I={cfg.I} k={cfg.k} S={cfg.S} "
          f"w={cfg.wdtype} x={cfg.xdtype} out={cfg.out_dtype}", flush=True)
    sys.stdout.flush()
    inp = gen.make_inputs(cfg, bias=with_bias)
    g = GpuCase(inp)
    assert moe.moe_layer_decode_fused(cfg.T, g.route_cfg, g.w.desc, moe.MOE_PATH_GEMV, moe.MOE_MODE_A, g.xdt)
    lay = g.layer(path=moe.MOE_PATH_GEMV, mode=moe.MOE_MODE_A)
    r, out = _staged(g)
    assert np.array_equal(lay["topk_idx"].reshape(cfg.T, cfg.k), r["topk_idx"]), "top-k ids"
    assert np.array_equal(lay["topk_w"].reshape(cfg.T, cfg.k).view(np.uint32), r["topk_w"].view(np.uint32)), "gates"
    if inp.slot_map is not None:
        assert lay["miss_count"] == r["miss_count"], "miss count"
        for f in ("miss_token", "miss_expert"):
            assert np.array_equal(lay[f], r[f]), f
        assert np.array_equal(lay["miss_weight"].view(np.uint32), r["miss_weight"].view(np.uint32)), "miss weights"
    assert np.array_equal(lay["out"], out), f"{name}: {np.sum(lay['out'] != out)} of {out.size} output elements differ"
    # AUTO takes the same flow at these batch sizes where the matrix cores are not chosen
    if moe.moe_resolve_path(g.w.desc, cfg.T, cfg.k, moe.MOE_PATH_AUTO, moe.MOE_MODE_A) == moe.MOE_PATH_GEMV:
        auto = g.layer(path=moe.MOE_PATH_AUTO, mode=moe.MOE_MODE_A)
        assert np.array_equal(auto["out"], lay["out"])
    ref = run_oracle(inp)
    flipped = check_routing(lay["topk_idx"].reshape(cfg.T, cfg.k), lay["topk_w"].reshape(cfg.T, cfg.k), ref)
    keep = np.array([t not in flipped for t in range(cfg.T)], bool)
    assert_fp_close(lay["out"][keep], ref["out"][keep], f"{name} layer")
    if inp.slot_map is not None and not flipped:
        assert lay["miss_count"] == ref["miss_token"].size
        assert np.array_equal(lay["miss_token"], ref["miss_token"])
        assert np.array_equal(lay["miss_expert"], ref["miss_expert"])
    print(f"[gpu-decode-fused] case={name}: identical to the staged launches", flush=True)



def test_out_of_range_slot_map_entry_sets_device_error():
    """A routed expert whose slot_map entry lies outside [-1, S) sets the device error word, as the
    staged permutation does; a valid call writes the word back to zero."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import GpuCase
    cfg = gen.config("compact_mxfp4", T=1, H=256, E=32, I=128, k=4, resident=10)
    inp = gen.make_inputs(cfg)
    lg = np.zeros((1, cfg.E), np.float32)
    lg[0, [5, 6, 7, 8]] = [4.0, 3.0, 2.0, 1.0]       # the four chosen experts
    inp.logits = lg
    good = GpuCase(inp)
    assert moe.moe_layer_decode_fused(cfg.T, good.route_cfg, good.w.desc, moe.MOE_PATH_GEMV, moe.MOE_MODE_A, good.xdt)
    print("[gpu-decode-fused] error word: valid map", flush=True)
    good.layer(path=moe.MOE_PATH_GEMV)              # no error raised: the word was written zero
    for bad_entry in (cfg.S + 3, -7):
        sm = inp.slot_map.copy()
        sm[6] = bad_entry
        inp_bad = dataclasses.replace(inp, slot_map=sm)
        print(f"[gpu-decode-fused] error word: slot_map[6] = {bad_entry}", flush=True)
        with pytest.raises(moe.MoeError) as ei:
            GpuCase(inp_bad, dev_weights=good.w).layer(path=moe.MOE_PATH_GEMV)
        assert ei.value.status == moe.MOE_ERR_DEVICE

"""GPU: the GEMM path's tile order across the XCDs changes placement only.  The scheduler deals
(slot, M tile, N tile) tiles to the eight XCDs in cost-sorted units (the default) or, as its
fallback, in eight contiguous runs of the plain order (MOE_PATH_TILES_CONTIGUOUS or'ed into the
path).  Every
output element is computed by one tile in a fixed reduction order, so both orders must give the
same bits, on skewed routing (a few hot slots of many M tiles), on few slots, and on uniform
routing, for both projections (y) in modes A and B."""
import sys

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu

CASES = [
    # name, config overrides
    ("zipf-384", dict(name="prefill_fp8_zipf", T=600, H=256, I=256, E=384, k=8)),
    ("zipf-few", dict(name="prefill_fp8_zipf", T=1500, H=256, I=128, E=6, k=2)),
    ("uniform", dict(name="decode_fp8", T=700, H=384, I=256, E=48, k=4)),
    ("compact", dict(name="compact_mxfp4", T=1200, H=256, I=256, E=64, k=4, resident=20)),
]


@pytest.mark.parametrize("mode", ["A", "B"])
@pytest.mark.parametrize("case", [c[0] for c in CASES])
def test_tile_orders_give_identical_bits(case, mode):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import GpuCase
    over = dict(dict(CASES)[case])
    cfg = gen.config(over.pop("name"), **over)
    inp = gen.make_inputs(cfg)
    g = GpuCase(inp)
    m = moe.MOE_MODE_A if mode == "A" else moe.MOE_MODE_B
    rp = g.route_permute()
    ys = {}
    for order in ("balanced", "contiguous"):
        print(f"[gpu-tile-order] case={case} mode={mode} order={order} T={cfg.T} E={cfg.E} S={cfg.S}", flush=True)
        sys.stdout.flush()
        path = moe.MOE_PATH_GEMM | (moe.MOE_PATH_TILES_CONTIGUOUS if order == "contiguous" else 0)
        ys[order] = g.expert_ffn(rp["perm"], rp["slot_offsets"], path=path, mode=m)
    a, b = ys["balanced"], ys["contiguous"]
    assert a.shape == b.shape and a.shape[0] == len(rp["perm"])
    assert np.all(np.isfinite(a)), "rows left unwritten (NaN fill) in the balanced order"
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{np.sum(a != b)} of {a.size} values differ"

"""GPU: batch invariance of a fixed FFN path.  A token's layer output must not depend on the batch
it is computed in (the pages claim this for their whole model: the vLLM-Moet README and its
mirror, batch-invariant decoding).  The AUTO path is not invariant (it switches between the GEMV
and the matrix-core path with the batch size); each fixed path is: routing is per token, every
output element of the GEMV and the GEMM is reduced in a fixed order whatever other rows share its
slot or tile, and the combine is per token.

One probe token is placed at several positions of batches from 1 to 300 tokens (other tokens
random); its output row must be the same bits in every batch, for each path and mode -- including
MOE_PATH_INVARIANT, the batch-invariant choice for callers that want the matrix cores wherever the
shape allows: the batches cross AUTO's GEMV/GEMM crossover (T*k = c*S with S = 16: T = 11 for bf16,
8 for FP8, 2 for MXFP4), and INVARIANT stays on one path across all of them."""
import dataclasses
import sys

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu

SIZES = [(1, 0), (2, 1), (5, 3), (16, 15), (17, 0), (40, 21), (300, 299), (300, 128)]  # (T, probe position)


def _batch(cfg, T, pos, pool):
    x = pool[1:T + 1].copy()
    x[pos] = pool[0]
    return x


@pytest.mark.parametrize("path,mode", [("gemv", "A"), ("gemm", "A"), ("gemv", "B"), ("gemm", "B"),
                                       ("invariant", "A"), ("invariant", "B")])
@pytest.mark.parametrize("wd", ["bf16", "fp8", "mxfp4"])
def test_probe_token_output_is_batch_invariant(path, mode, wd):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import GpuCase
    from routed_expert_ffn_05_amd import device as D
    if wd == "bf16" and mode == "B":
        pytest.skip("mode B multiplies FP8 / MXFP4 weights")
    base = gen.config("decode_bf16", T=301, H=256, E=16, I=128, k=4, wdtype=wd, out_dtype="f32")
    inp0 = gen.make_inputs(base)
    pool = inp0.x                                    # 301 tokens: the probe is row 0
    w_dev = D.upload_weights(wd, base.H, base.I, inp0.weights)
    p = {"gemv": moe.MOE_PATH_GEMV, "gemm": moe.MOE_PATH_GEMM, "invariant": moe.MOE_PATH_INVARIANT}[path]
    m = moe.MOE_MODE_A if mode == "A" else moe.MOE_MODE_B
    ref = None
    for T, pos in SIZES:
        print(f"[gpu-invariance] w={wd} path={path} mode={mode} T={T} pos={pos}", flush=True)
        sys.stdout.flush()
        inp = dataclasses.replace(inp0, cfg=base.replace(T=T), x=_batch(base, T, pos, pool))
        res = GpuCase(inp, dev_weights=w_dev).layer(path=p, mode=m)
        row = res["out"][pos]
        if ref is None:
            ref = row
        else:
            assert np.array_equal(row, ref), f"T={T} pos={pos}: {np.sum(row != ref)} of {row.size} differ"

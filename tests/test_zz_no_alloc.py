"""GPU: moe_layer_static (moe_layer on the library's static workspace, for callers that cannot
allocate) gives the same bits as moe_layer on a caller-allocated workspace, on two calls in a row
(the second smaller, so the static workspace still holds the first call's contents), on a compact
MXFP4 layer with misses (matrix-core path) and a bf16 layer with router weights (GEMV path)."""
import sys

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu


def _run(moe, D, torch, inp, static):
    cfg = inp.cfg
    T, H, E, k, S = cfg.T, cfg.H, cfg.E, cfg.k, cfg.S
    R = max(T * k, 1)
    w = D.upload_weights(cfg.wdtype, H, cfg.I, inp.weights)
    rcfg = moe.routing(E, k, cfg.score, cfg.renorm)
    xdt = moe.MOE_BF16 if cfg.xdtype == "bf16" else moe.MOE_F32
    odt = moe.MOE_BF16 if cfg.out_dtype == "bf16" else moe.MOE_F32
    d_x, d_wr, d_lg, d_sm = (D.to_device(a) for a in (inp.x, inp.w_router, inp.logits, inp.slot_map))
    out = torch.full((T, H), -1, dtype=torch.int16 if odt == moe.MOE_BF16 else torch.float32, device="cuda")
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    tw = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
    mc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    mt, me = (torch.full((R,), -1, dtype=torch.int32, device="cuda") for _ in range(2))
    mw = torch.full((R,), -1.0, dtype=torch.float32, device="cuda")
    c = d_sm is not None
    args = (d_x, xdt, T, d_wr, d_lg, None, rcfg, d_sm, w.desc, moe.MOE_PATH_AUTO, moe.MOE_MODE_A, out, odt, idx, tw,
            mc if c else None, mt if c else None, me if c else None, mw if c else None)
    if static:
        moe.moe_layer_static(*args)
    else:
        nb = moe.moe_layer_workspace_size(T, rcfg, w.desc, moe.MOE_PATH_AUTO, moe.MOE_MODE_A, d_wr is not None)
        ws = D.workspace(nb)
        moe.moe_layer(*args, ws, nb)
    torch.cuda.synchronize()
    res = dict(out=D.to_host(out), idx=D.to_host(idx), w=D.to_host(tw))
    if c:
        n = int(D.to_host(mc)[0])
        res.update(n=n, mt=D.to_host(mt)[:n], me=D.to_host(me)[:n], mw=D.to_host(mw)[:n])
    return res


@pytest.mark.parametrize("name", ["compact_mxfp4", "decode_bf16"])
def test_static_workspace_matches_caller_workspace(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from routed_expert_ffn_05_amd import device as D
    if name == "compact_mxfp4":
        shapes = [dict(T=48, H=512, E=32, I=256, k=4, resident=11), dict(T=5, H=512, E=32, I=256, k=4, resident=11)]
    else:
        shapes = [dict(T=9, H=512, E=24, I=256, k=4), dict(T=3, H=512, E=24, I=256, k=4)]
    for call, over in enumerate(shapes):
        cfg = gen.config(name, **over)
        print(f"[gpu-static] {name} call {call}: T={cfg.T} H={cfg.H} E={cfg.E} I={cfg.I} k={cfg.k} S={cfg.S}", flush=True)
        sys.stdout.flush()
        inp = gen.make_inputs(cfg)
        a = _run(moe, D, torch, inp, static=True)
        b = _run(moe, D, torch, inp, static=False)
        for key in b:
            va, vb = np.asarray(a[key]), np.asarray(b[key])
            assert va.shape == vb.shape and va.tobytes() == vb.tobytes(), f"{name} call {call}: {key} differs"
        assert (a["idx"] >= 0).all()

"""GPU: LRU slot refill (moe_refill_slots) against the oracle over a stream of calls.

Starting from empty slots, each call routes a new batch of the compact workload (Zipf logits,
the workload's expert ranking) through moe_route_permute with the current slot map, then refills:
the maps, the last-use stamps and the moves must equal the oracle's after every call, and at the
end every slot must hold its expert's weight bytes exactly (every weight format's segments)."""
import sys

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu

CASES = {
    "mxfp4": gen.config("compact_mxfp4", T=4, H=128, E=48, I=64, k=4, resident=12),
    "fp8": gen.config("prefill_fp8_zipf", T=6, H=256, E=40, I=128, k=3, resident=10),
    "bf16_all_fit": gen.config("prefill_fp8_zipf", T=3, H=128, E=16, I=64, k=2, resident=16, wdtype="bf16"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_refill_stream_matches_oracle(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from oracle import moe_oracle as O
    from routed_expert_ffn_05_amd import device as D
    cfg = CASES[name]
    T, E, k, S = cfg.T, cfg.E, cfg.k, cfg.S
    store = D.upload_weights(cfg.wdtype, cfg.H, cfg.I, gen.stack_weights(cfg, range(E)))
    slots = D.DeviceWeights(cfg.wdtype, S, cfg.H, cfg.I,
                            *[torch.zeros((S,) + tuple(t.shape[1:]), dtype=t.dtype, device="cuda") if t is not None
                              else None for t in (store.w_gu, store.s_gu, store.w_d, store.s_d)])
    sm = np.full(E, -1, np.int32)
    se = np.full(S, -1, np.int32)
    lu = np.full(S, -1, np.int64)
    d_sm, d_se, d_lu = D.to_device(sm), D.to_device(se), D.to_device(lu)
    rcfg = moe.routing(E, k, cfg.score, cfg.renorm)
    R = T * k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(S + 1, dtype=torch.int32, device="cuda")
    perm, inv, mt, me = (torch.empty(R, dtype=torch.int32, device="cuda") for _ in range(4))
    mw = torch.empty(R, dtype=torch.float32, device="cuda")
    mc = torch.zeros(1, dtype=torch.int32, device="cuda")
    nb = moe.moe_route_permute_workspace_size(T, rcfg, S, False)
    ws = D.workspace(nb)
    rws = D.workspace(moe.moe_refill_workspace_size(S))
    hits = rows = 0
    for step in range(24):
        print(f"[gpu-refill] case={name} step={step}", flush=True)
        sys.stdout.flush()
        lg = gen.make_logits(cfg, batch=step)
        moe.moe_route_permute(None, moe.MOE_BF16, T, cfg.H, None, D.to_device(lg), None, rcfg, d_sm, S, idx, w,
                              counts, off, perm, inv, mc, mt, me, mw, ws, nb)
        moe.moe_refill_slots(counts, E, step, d_sm, d_se, d_lu, store.desc, slots.desc, rws, rws.numel())
        torch.cuda.synchronize()
        c = D.to_host(counts)
        assert np.array_equal(c, np.bincount(O.select_topk(lg, k).reshape(-1), minlength=E))
        hits += int(c[sm >= 0].sum())
        rows += int(c.sum())
        sm, se, lu, moves = O.lru_refill(c, step, sm, se, lu)
        assert np.array_equal(D.to_host(d_sm), sm), step
        assert np.array_equal(D.to_host(d_se), se), step
        assert np.array_equal(D.to_host(d_lu), lu), step
        raw = D.to_host(rws)
        n = int(raw[:4].view(np.int32)[0])
        got = raw[256:256 + 8 * n].view(np.int32).reshape(-1, 2).tolist()
        assert got == [list(m) for m in moves], step
    for s, e in enumerate(se):
        if e < 0:
            continue
        for a, b in ((slots.w_gu, store.w_gu), (slots.s_gu, store.s_gu), (slots.w_d, store.w_d), (slots.s_d, store.s_d)):
            if a is not None:
                assert torch.equal(a[s], b[e]), (s, e)
    print(f"[gpu-refill] case={name} hit rate {hits / rows:.3f} over 24 calls", flush=True)

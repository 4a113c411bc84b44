"""Full-size parity: every workload at its stated size, run through the same C-ABI call sequence
that bench.py times (route+permute, gate/up, down, combine on one stream, device-resident inputs),
checked against the oracle: routing, counts, slot offsets, permutation and the compact miss list
in full; the expert-FFN rows and layer outputs of a seeded sample of tokens (the oracle computes
only those tokens' rows, dequantising just the experts they touch)."""
import sys
import time

import numpy as np
import pytest

from synth import gen

pytestmark = pytest.mark.gpu

FULL = [("decode_bf16", None, "A"), ("decode_fp8", None, "A"), ("prefill_fp8_zipf", None, "A"),
        ("compact_mxfp4", 1, "A"), ("compact_mxfp4", 4096, "A"),
        # mode B on the block-scaled matrix cores, against the oracle with the same activation
        # quantisation (the scale-aware bound widened as in the small mode-B cases)
        ("prefill_fp8_zipf", None, "B"), ("compact_mxfp4", 4096, "B")]
N_SAMPLE = 4


def _say(msg):
    print(f"[gpu-full] {msg}", flush=True)
    sys.stdout.flush()


def _run_staged(inp, w, mode):
    """bench.py's timed sequence on device inputs; returns host copies of every result."""
    import torch

    import routed_expert_ffn_05_amd as moe
    from routed_expert_ffn_05_amd import device as D
    cfg = inp.cfg
    T, H, E, k, S = cfg.T, cfg.H, cfg.E, cfg.k, cfg.S
    R = T * k
    dev = "cuda"
    d_x = D.to_device(inp.x)
    d_lg = D.to_device(inp.logits)
    d_wr = D.to_device(inp.w_router)
    d_sm = D.to_device(inp.slot_map)
    xdt = moe.MOE_BF16 if cfg.xdtype == "bf16" else moe.MOE_F32
    odt = moe.MOE_BF16 if cfg.out_dtype == "bf16" else moe.MOE_F32
    rcfg = moe.routing(E, k, cfg.score, cfg.renorm)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(S + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(R, dtype=torch.int32, device=dev)
    inv = torch.empty(R, dtype=torch.int32, device=dev)
    mc = torch.zeros(1, dtype=torch.int32, device=dev)
    mt = torch.empty(R, dtype=torch.int32, device=dev)
    me = torch.empty(R, dtype=torch.int32, device=dev)
    mw = torch.empty(R, dtype=torch.float32, device=dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.int16 if odt == moe.MOE_BF16 else torch.float32, device=dev)
    rp = moe.moe_route_permute_workspace_size(T, rcfg, S, d_wr is not None)
    pws = D.workspace(rp)
    path = moe.MOE_PATH_AUTO
    fb = moe.moe_expert_ffn_workspace_size(w.desc, T, k, path, mode)
    fws = D.workspace(fb)
    c = d_sm is not None
    moe.moe_route_permute(d_x, xdt, T, H, d_wr, d_lg, None, rcfg, d_sm, S, idx, tw, counts, off, perm, inv,
                          mc if c else None, mt if c else None, me if c else None, mw if c else None, pws, rp)
    moe.moe_expert_gate_up(w.desc, d_x, xdt, T, k, perm, off, path, mode, fws, fb)
    moe.moe_expert_down(w.desc, T, k, off, path, mode, y, fws, fb)
    moe.moe_combine(y, inv, tw, T, k, H, out, odt)
    torch.cuda.synchronize()
    moe.moe_check_device_error(pws)
    n_res = int(D.to_host(off)[-1])
    res = dict(topk_idx=D.to_host(idx), topk_w=D.to_host(tw), counts=D.to_host(counts), slot_offsets=D.to_host(off),
               perm=D.to_host(perm)[:n_res], inv_perm=D.to_host(inv), y=y, out=out, odt=odt)
    if c:
        n = int(D.to_host(mc)[0])
        res.update(miss_count=n, miss_token=D.to_host(mt)[:n], miss_expert=D.to_host(me)[:n],
                   miss_weight=D.to_host(mw)[:n])
    return res


@pytest.mark.parametrize("name,T,mode", FULL,
                         ids=[f"{n}" + (f"_T{t}" if t else "") + f"_mode{m}" for n, t, m in FULL])
def test_full_size_layer(name, T, mode):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_05_amd as moe
    from gpu_cases import assert_fp_close, check_permute, check_routing
    from oracle import moe_oracle as O
    from routed_expert_ffn_05_amd import device as D
    cfg = gen.config(name, T=T) if T else gen.config(name)
    _say(f"{name} T={cfg.T} H={cfg.H} E={cfg.E} I={cfg.I} k={cfg.k} S={cfg.S} w={cfg.wdtype} mode {mode}: generating")
    t0 = time.time()
    inp = gen.make_inputs(cfg)
    _say(f"{name}: inputs in {time.time() - t0:.1f}s; uploading")
    w = D.upload_weights(cfg.wdtype, cfg.H, cfg.I, inp.weights)
    res = _run_staged(inp, w, moe.MOE_MODE_A if mode == "A" else moe.MOE_MODE_B)
    _say(f"{name}: GPU layer done; oracle on a sample")
    rng = np.random.default_rng(1234)
    sample = np.sort(rng.choice(cfg.T, size=min(N_SAMPLE, cfg.T), replace=False))
    t0 = time.time()
    ref = O.layer(inp.x, cfg.xdtype, inp.weights, cfg.wdtype, cfg.H, cfg.I, cfg.E, cfg.k, cfg.score, cfg.renorm,
                  w_router=inp.w_router, logits=inp.logits, slot_map=inp.slot_map, S=cfg.S, tokens=sample,
                  act_quant=O.act_quant_mx_e4m3 if mode == "B" else None)
    stol = 8e-2 if mode == "B" else 2e-2
    _say(f"{name}: oracle in {time.time() - t0:.1f}s")
    # routing and permutation, every token
    flipped = check_routing(res["topk_idx"], res["topk_w"], ref)
    if not flipped:
        check_permute(res, ref)
    # sampled tokens: their expert-FFN rows and outputs
    keep = np.array([t not in flipped for t in sample], bool)
    assert keep.any()
    tok = sample[keep]
    pos = ref["inv_perm"].reshape(cfg.T, cfg.k)[tok].reshape(-1)
    pos = pos[pos >= 0]
    if pos.size:
        y_gpu = D.to_host(res["y"][torch.as_tensor(pos, device="cuda").long()]).astype(np.float64)
        assert_fp_close(y_gpu, ref["y_perm"][pos], f"{name} y_perm rows of the sample", scale_tol=stol)
    o = D.to_host(res["out"][torch.as_tensor(tok, device="cuda").long()])
    o = (D.bf16_bits_to_float(o) if res["odt"] == moe.MOE_BF16 else o).astype(np.float64)
    assert_fp_close(o, ref["out"][keep], f"{name} out rows of the sample", scale_tol=stol)
    _say(f"{name}: ok ({len(tok)} sampled tokens, {pos.size} expert rows, {len(flipped)} near-tie flips)")

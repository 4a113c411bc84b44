"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on seeded inputs,
run the oracle on the same inputs, and compare with the stated tolerances.

Integer results (routing indices, counts, offsets, permutation, miss lists) must match exactly,
except the routing of tokens the oracle flags as near-ties (two of the k+1 best scores closer
than 1e-5), which may differ because logits are accumulated in another order.
Floating-point results must satisfy, elementwise and in relative L2:
    |gpu - ref| <= 2e-2 * max(1, |ref|)        ||gpu - ref||_2 <= 5e-3 ||ref||_2
and, since the layer's outputs are often far below 1 in magnitude, a scale-aware elementwise
bound as well:  |gpu - ref| <= 2e-2 * max(|ref|, rms(ref)).
"""
from __future__ import annotations

import numpy as np

import routed_expert_ffn_05_amd as moe
from oracle import moe_oracle as O
from routed_expert_ffn_05_amd import device as D

ELEM_TOL = 2e-2
L2_TOL = 5e-3
# fp32 gates (renormalised scores, also the miss list's weights) against the oracle's fp64 ones:
# a few fp32 roundings (the score, the sum of k scores, one division), so 1e-6 relative; the
# absolute floor only matters for softmax scores far below 1
GATE_RTOL = 1e-6
GATE_ATOL = 1e-12


def assert_fp_close(gpu, ref, what, elem_tol=ELEM_TOL, l2_tol=L2_TOL, scale_tol=ELEM_TOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    err = np.abs(gpu - ref)
    assert np.all(err <= elem_tol * np.maximum(1.0, np.abs(ref))), f"{what}: elementwise bound, max err {err.max()}"
    rms = np.sqrt(np.mean(ref ** 2))
    bound = scale_tol * np.maximum(np.abs(ref), rms)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond {scale_tol:g}*max(|ref|, rms); worst {(err / np.maximum(bound, 1e-300)).max():.3g}x"
    nr = np.linalg.norm(ref)
    if nr > 0:
        rel = np.linalg.norm(gpu - ref) / nr
        assert rel <= l2_tol, f"{what}: relative L2 {rel:.3g} > {l2_tol}"


def run_oracle(inp, tokens=None, act_quant=None):
    cfg = inp.cfg
    return O.layer(inp.x, cfg.xdtype, inp.weights, cfg.wdtype, cfg.H, cfg.I, cfg.E, cfg.k, cfg.score,
                   cfg.renorm, w_router=inp.w_router, logits=inp.logits, bias=inp.bias,
                   slot_map=inp.slot_map, S=cfg.S, tokens=tokens, act_quant=act_quant)


class GpuCase:
    """Device copies of one LayerInputs and the calls to each ABI stage."""

    def __init__(self, inp, dev_weights=None):
        import torch
        self.inp = inp
        c = inp.cfg
        self.cfg = c
        self.x = D.to_device(inp.x)
        self.xdt = moe.MOE_BF16 if c.xdtype == "bf16" else moe.MOE_F32
        self.odt = moe.MOE_BF16 if c.out_dtype == "bf16" else moe.MOE_F32
        self.w_router = D.to_device(inp.w_router)
        self.logits = D.to_device(inp.logits)
        self.bias = D.to_device(inp.bias)
        self.slot_map = D.to_device(inp.slot_map)
        self.w = dev_weights if dev_weights is not None else D.upload_weights(c.wdtype, c.H, c.I, inp.weights)
        self.route_cfg = moe.routing(c.E, c.k, c.score, c.renorm)
        self.torch = torch

    # --- whole layer ---------------------------------------------------------------------
    def layer(self, path=moe.MOE_PATH_AUTO, mode=moe.MOE_MODE_A):
        torch = self.torch
        c = self.cfg
        L = D.Layer(T=c.T, H=c.H, I=c.I, E=c.E, k=c.k, score=c.score, renorm=c.renorm, xdtype=c.xdtype,
                    out_dtype=c.out_dtype, weights=self.w, w_router=self.w_router, slot_map=self.slot_map,
                    bias=self.bias, path=path, mode=mode)
        L(self.x, self.logits)
        torch.cuda.synchronize()
        moe.moe_check_device_error(L.ws)
        out = D.to_host(L.out)
        out = D.bf16_bits_to_float(out) if self.odt == moe.MOE_BF16 else out
        res = dict(out=out.astype(np.float64), topk_idx=D.to_host(L.topk_idx), topk_w=D.to_host(L.topk_w))
        if self.slot_map is not None:
            n = int(D.to_host(L.miss_count)[0])
            res.update(miss_count=n, miss_token=D.to_host(L.miss_token)[:n],
                       miss_expert=D.to_host(L.miss_expert)[:n], miss_weight=D.to_host(L.miss_weight)[:n])
        return res

    # --- stages ----------------------------------------------------------------------------
    def route(self):
        torch = self.torch
        c = self.cfg
        idx = torch.empty((c.T, c.k), dtype=torch.int32, device="cuda")
        w = torch.empty((c.T, c.k), dtype=torch.float32, device="cuda")
        lo = torch.empty((c.T, c.E), dtype=torch.float32, device="cuda") if self.w_router is not None else None
        moe.moe_route(self.x, self.xdt, c.T, c.H, self.w_router, self.logits, self.bias, self.route_cfg, idx, w,
                      lo, None, 0)
        torch.cuda.synchronize()
        return D.to_host(idx), D.to_host(w), (D.to_host(lo) if lo is not None else None)

    def permute(self, topk_idx, topk_w):
        torch = self.torch
        c = self.cfg
        R = c.T * c.k
        t_idx = D.to_device(np.asarray(topk_idx, np.int32))
        t_w = D.to_device(np.asarray(topk_w, np.float32))
        counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
        off = torch.empty(c.S + 1, dtype=torch.int32, device="cuda")
        perm = torch.full((max(R, 1),), -7, dtype=torch.int32, device="cuda")
        inv = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
        mc = torch.zeros(1, dtype=torch.int32, device="cuda")
        mt = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
        me = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
        mw = torch.empty(max(R, 1), dtype=torch.float32, device="cuda")
        ws = D.workspace(moe.moe_permute_workspace_size(c.T, self.route_cfg, c.S))
        moe.moe_permute(t_idx, t_w, c.T, self.route_cfg, self.slot_map, c.S, counts, off, perm, inv, mc, mt, me, mw,
                        ws, ws.numel())
        torch.cuda.synchronize()
        moe.moe_check_device_error(ws)
        n_res = int(D.to_host(off)[-1])
        n_miss = int(D.to_host(mc)[0])
        return dict(counts=D.to_host(counts), slot_offsets=D.to_host(off), perm=D.to_host(perm)[:n_res],
                    inv_perm=D.to_host(inv)[:R], miss_count=n_miss, miss_token=D.to_host(mt)[:n_miss],
                    miss_expert=D.to_host(me)[:n_miss], miss_weight=D.to_host(mw)[:n_miss])

    def route_permute(self):
        torch = self.torch
        c = self.cfg
        R = c.T * c.k
        idx = torch.empty((max(c.T, 1), c.k), dtype=torch.int32, device="cuda")
        w = torch.empty((max(c.T, 1), c.k), dtype=torch.float32, device="cuda")
        counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
        off = torch.empty(c.S + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
        inv = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
        mc = torch.zeros(1, dtype=torch.int32, device="cuda")
        mt = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
        me = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
        mw = torch.empty(max(R, 1), dtype=torch.float32, device="cuda")
        nb = moe.moe_route_permute_workspace_size(c.T, self.route_cfg, c.S, self.w_router is not None)
        ws = D.workspace(nb)
        sm = self.slot_map
        moe.moe_route_permute(self.x, self.xdt, c.T, c.H, self.w_router, self.logits, self.bias, self.route_cfg, sm,
                              c.S, idx, w, counts, off, perm, inv, mc if sm is not None else None,
                              mt if sm is not None else None, me if sm is not None else None,
                              mw if sm is not None else None, ws, nb)
        torch.cuda.synchronize()
        moe.moe_check_device_error(ws)
        n_res = int(D.to_host(off)[-1])
        n_miss = int(D.to_host(mc)[0]) if sm is not None else 0
        res = dict(topk_idx=D.to_host(idx)[: c.T], topk_w=D.to_host(w)[: c.T], counts=D.to_host(counts),
                   slot_offsets=D.to_host(off), perm=D.to_host(perm)[:n_res], inv_perm=D.to_host(inv)[:R])
        if sm is not None:
            res.update(miss_count=n_miss, miss_token=D.to_host(mt)[:n_miss], miss_expert=D.to_host(me)[:n_miss],
                       miss_weight=D.to_host(mw)[:n_miss])
        return res

    def expert_ffn(self, perm, slot_offsets, path=moe.MOE_PATH_AUTO, mode=moe.MOE_MODE_A, want_a=False):
        """y_perm rows of the call; with want_a also the intermediate a the call left in its
        workspace (read through moe_expert_ffn_workspace_layout, as fp64 values)."""
        torch = self.torch
        c = self.cfg
        R = c.T * c.k
        d_perm = D.to_device(np.asarray(perm, np.int32)) if len(perm) else torch.zeros(1, dtype=torch.int32, device="cuda")
        d_off = D.to_device(np.asarray(slot_offsets, np.int32))
        y = torch.full((max(R, 1), c.H), float("nan"), dtype=torch.float32, device="cuda")
        desc = self.w.desc
        nb = moe.moe_expert_ffn_workspace_size(desc, c.T, c.k, path, mode)
        ws = D.workspace(nb)
        moe.moe_expert_ffn(desc, self.x, self.xdt, c.T, c.k, d_perm, d_off, path, mode, y, ws, nb)
        torch.cuda.synchronize()
        y = D.to_host(y)[: len(perm)]
        if not want_a:
            return y
        return y, read_a(ws, moe.moe_expert_ffn_workspace_layout(desc, c.T, c.k, path, mode), len(perm), c.I)


    def combine(self, y_perm, inv_perm, topk_w):
        torch = self.torch
        c = self.cfg
        d_y = D.to_device(np.ascontiguousarray(y_perm, np.float32)) if len(y_perm) else \
            torch.zeros((1, c.H), dtype=torch.float32, device="cuda")
        d_inv = D.to_device(np.asarray(inv_perm, np.int32))
        d_w = D.to_device(np.asarray(topk_w, np.float32))
        out = torch.empty((c.T, c.H), dtype=torch.int16 if self.odt == moe.MOE_BF16 else torch.float32, device="cuda")
        moe.moe_combine(d_y, d_inv, d_w, c.T, c.k, c.H, out, self.odt)
        torch.cuda.synchronize()
        o = D.to_host(out)
        return (D.bf16_bits_to_float(o) if self.odt == moe.MOE_BF16 else o).astype(np.float64)


    def combine_tiers(self, y_a, inv_a, y_b, inv_b, topk_w):
        torch = self.torch
        c = self.cfg

        def rows(y):
            return D.to_device(np.ascontiguousarray(y, np.float32)) if len(y) else \
                torch.zeros((1, c.H), dtype=torch.float32, device="cuda")
        out = torch.empty((c.T, c.H), dtype=torch.int16 if self.odt == moe.MOE_BF16 else torch.float32, device="cuda")
        moe.moe_combine_tiers(rows(y_a), D.to_device(np.asarray(inv_a, np.int32)), rows(y_b),
                              D.to_device(np.asarray(inv_b, np.int32)), D.to_device(np.asarray(topk_w, np.float32)),
                              c.T, c.k, c.H, out, self.odt)
        torch.cuda.synchronize()
        o = D.to_host(out)
        return (D.bf16_bits_to_float(o) if self.odt == moe.MOE_BF16 else o).astype(np.float64)


def read_a(ws, layout, n, I):
    """The intermediate a of n permuted rows from an expert-FFN workspace (a torch uint8 tensor),
    decoded to fp64 by its format (fp32; bf16; bf16 hi + lo; E4M3 codes x 2^(E8M0 - 127))."""
    off_a, off_q, off_s, fmt = layout
    host = D.to_host(ws)
    if fmt == 0:
        return host[off_a:off_a + n * I * 4].view(np.float32).reshape(n, I).astype(np.float64)
    if fmt == 1:
        return O.bf16_to_f64(host[off_a:off_a + n * I * 2].view(np.uint16).reshape(n, I))
    if fmt == 2:
        v = O.bf16_to_f64(host[off_a:off_a + n * 2 * I * 2].view(np.uint16).reshape(n, 2 * I))
        return v[:, :I] + v[:, I:]
    codes = host[off_q:off_q + n * I].reshape(n, I)
    sc = host[off_s:off_s + n * (I // 32)].reshape(n, I // 32).astype(np.int64) - 127
    return O.e4m3fn_to_f64(codes) * np.exp2(np.repeat(sc, 32, axis=1))


def oracle_mode_b_stages(inp, perm, off, positions, a_gpu, threads=1):
    """The oracle's mode-B stages for the permuted rows `positions`, computed slot by slot from its
    own primitives: the fp64 a of each row (from the MX-E4M3-quantised x, as the mirror does), its
    MX-E4M3 quantisation (scale exponents and dequantised values), and the down projection applied
    to the GPU's own quantised a (a_gpu, one row per position).  The quantisation of a is a
    floating-point decision on an integer code: where the oracle's fp64 a and the kernel's fp32 a
    straddle a rounding boundary both codes are correct, so the down projection is checked on the
    GPU's codes and the codes are checked apart (check_mode_b_codes)."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = inp.cfg
    x64 = O.activations_f64(inp.x, cfg.xdtype)
    positions = np.asarray(positions, np.int64)
    slot_of = np.searchsorted(np.asarray(off), positions, side="right") - 1
    res = dict(a64=np.empty((positions.size, cfg.I)), deq=np.empty((positions.size, cfg.I)),
               X=np.empty((positions.size, cfg.I // 32), np.int64), y=np.empty((positions.size, cfg.H)))

    def work(s):
        sel = np.nonzero(slot_of == s)[0]
        wg, wu, wd = O.slot_matrices(inp.weights, cfg.wdtype, int(s), cfg.H, cfg.I)
        xq = O.act_quant_mx_e4m3(x64[np.asarray(perm)[positions[sel]] // cfg.k])
        a64 = O.silu(xq @ wg.T) * (xq @ wu.T)
        X, q = O.act_quant_mx_e4m3_parts(a64)
        res["a64"][sel] = a64
        res["X"][sel] = X
        res["deq"][sel] = np.ldexp(q.reshape(sel.size, -1, 32), X[:, :, None]).reshape(sel.size, cfg.I)
        res["y"][sel] = a_gpu[sel] @ wd.T
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(work, np.unique(slot_of)))
    return res


def check_mode_b_codes(a_gpu, st, what, rel=1e-3, rel_blk=1e-4):
    """The GPU's quantised a against the oracle's exact (fp64) a.  The quantisation is a
    floating-point decision on integer codes, taken by the kernel on its own fp32 a (block-scaled
    matrix-core sums), which differs from the exact a by a little: allowed here up to
    eps = rel*|a| + rel_blk*max|a| over the 32-value block (measured: about 2e-5 of the block
    maximum).  Every GPU value must be the correct MX-E4M3 rounding of some value within eps of the
    exact a: at the block's scale exponent, or one higher or lower where the block maximum itself
    lies within eps_blk of a power of two.  Returns the share of values equal to the oracle's own
    quantisation (information)."""
    a64, X = st["a64"], st["X"]
    n, K = a64.shape
    blk = np.abs(a64).reshape(n, K // 32, 32).max(axis=2)
    eps = rel * np.abs(a64) + np.repeat(rel_blk * blk, 32, axis=1)
    eps_blk = (rel + rel_blk) * blk
    valid = np.zeros(a64.shape, bool)
    for dx in (-1, 0, 1):
        Xc = X + dx
        if dx:  # another scale only where the block maximum's binade is ambiguous
            ok = (np.floor(np.log2(np.maximum(blk - eps_blk, 1e-300))) !=
                  np.floor(np.log2(np.maximum(blk + eps_blk, 1e-300))))
            ok &= blk > 0
            if not ok.any():
                continue
        else:
            ok = np.ones_like(blk, bool)
        sc = np.repeat(Xc, 32, axis=1)
        lo = np.ldexp(O.e4m3fn_round(np.ldexp(a64 - eps, -sc)), sc)
        hi = np.ldexp(O.e4m3fn_round(np.ldexp(a64 + eps, -sc)), sc)
        valid |= np.repeat(ok, 32, axis=1) & (lo <= a_gpu) & (a_gpu <= hi)
    if not valid.all():
        ii = np.argwhere(~valid)[:6]
        ex = "; ".join(f"row {r} col {c}: exact {a64[r, c]:.6g} gpu {a_gpu[r, c]:.6g} oracle {st['deq'][r, c]:.6g} "
                       f"X {X[r, c // 32]} block max {blk[r, c // 32]:.6g}" for r, c in ii)
        raise AssertionError(f"{what}: {(~valid).sum()} quantised a values that no value within the kernel's "
                             f"precision of the exact a rounds to: {ex}")
    return float((a_gpu == st["deq"]).mean()) if a_gpu.size else 1.0


def routing_mismatches(gpu_idx, ref):
    """Tokens whose GPU selection differs from the oracle's; asserts each one is a flagged near-tie."""
    diff = np.nonzero((np.asarray(gpu_idx) != ref["topk_idx"]).any(axis=1))[0]
    unflagged = [int(t) for t in diff if not ref["near_tie"][t]]
    assert not unflagged, f"routing differs on tokens {unflagged[:10]} that are not near-ties"
    return set(int(t) for t in diff)


def check_routing(gpu_idx, gpu_w, ref):
    flipped = routing_mismatches(gpu_idx, ref)
    keep = np.array([t not in flipped for t in range(ref["topk_idx"].shape[0])], bool)
    if keep.any():
        np.testing.assert_allclose(np.asarray(gpu_w, np.float64)[keep], ref["topk_w"][keep], rtol=GATE_RTOL,
                                   atol=GATE_ATOL)
    return flipped


def check_permute(g, ref):
    assert np.array_equal(g["counts"], ref["counts"]), "counts"
    assert np.array_equal(g["slot_offsets"], ref["slot_offsets"]), "slot_offsets"
    assert np.array_equal(g["perm"], ref["perm"]), "perm"
    assert np.array_equal(g["inv_perm"], ref["inv_perm"]), "inv_perm"
    check_misses(g, ref)


def check_misses(g, ref):
    if "miss_token" not in g:
        return
    assert g["miss_count"] == ref["miss_token"].size, "miss_count"
    assert np.array_equal(g["miss_token"], ref["miss_token"]), "miss_token"
    assert np.array_equal(g["miss_expert"], ref["miss_expert"]), "miss_expert"
    np.testing.assert_allclose(g["miss_weight"], ref["miss_weight"], rtol=GATE_RTOL, atol=GATE_ATOL)

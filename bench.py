#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode_bf16]

A step is one pass of the whole layer -- router logits and top-k, permutation, expert gate/up
and down projections, combine -- over one batch of synthetic tokens, with every input resident in
HBM before the timed region starts.  Batches rotate over ``--rotate`` pre-generated activation
(or logit) sets so that consecutive steps route to different experts.  Prints ONE JSON line.

The default workload is the bf16 decode layer: T=4 tokens, hidden 4096, 384 experts, expert
intermediate 1024, top-8 sigmoid routing with renormalised gates.  ``--tiers`` (compact configs)
adds the second tier to every step: the rows routed to absent experts are permuted over a pool
holding those experts, computed there, and combined with the resident rows (moe_combine_tiers),
so the step produces the full layer output.  ``--lru`` (compact configs) refills the slots after every
call with the experts that missed (moe_refill_slots, weights copied from a store of every expert);
``--plan-slots`` places the hot set planned from other batches instead of the seeded map.

The ``roofline`` object describes the dominant kernel (the expert gate/up projection, 2/3 of the
layer's bytes): algorithmic bytes per launch over its average duration, measured with HIP events
recorded on the launch stream around every timed launch (timing-only events, created with
hipEventDisableSystemFence, so that recording them adds no cache writeback between the kernels).  ``cpu_baseline`` times the CPU oracle
on a bounded sample of the same workload.

Profiling helpers (no GPU work of their own):
    python bench.py --copy-probe-mib 512 ...   also launches one plain device copy of known size
    python bench.py --summarize-kernels DIR --out FILE   rocprofv3 --stats CSV -> summary text
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --out FILE   PMC CSVs -> traffic summary
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0}
PROFILES = os.path.join(ROOT, "profiles")
# sources of each gate/up kernel: a recorded traffic figure stands only while their hash matches
GATE_UP_SOURCES = {
    "gemv": ["routed_expert_ffn_05_amd/csrc/gemv_impl.h", "routed_expert_ffn_05_amd/csrc/common.h"],
    "gemm": ["routed_expert_ffn_05_amd/csrc/gemm.hip", "routed_expert_ffn_05_amd/csrc/common.h"],
    "gemm_q": ["routed_expert_ffn_05_amd/csrc/gemm.hip", "routed_expert_ffn_05_amd/csrc/common.h"],
    "decode": ["routed_expert_ffn_05_amd/csrc/gemv_impl.h", "routed_expert_ffn_05_amd/csrc/common.h",
               "routed_expert_ffn_05_amd/csrc/topk.h"],
}
GATE_UP_KERNELS = {"gemv": "gemv::gate_up_kernel", "gemm": "gemm::gemm_kernel", "gemm_q": "gemm::gemm_q_kernel",
                   "decode": "gemv::decode_gate_up_kernel"}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    """Hash of the code in `paths` with comments and whitespace removed, so that a recorded
    counter figure outlives edits of the comments but not of the code."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------------------------

def _csvs(d, pattern):
    return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))


def summarize_kernels(d, out, command):
    rows = []
    for f in _csvs(d, "*kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel statistics", "", f"command: `{command}`", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = name.split("(")[0][:90]
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_per_kernel(d, counter):
    """{kernel short name: [per-dispatch counter values]} from rocprofv3 counter_collection CSVs."""
    res = {}
    for f in _csvs(d, "*counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                name = r.get("Kernel_Name", "").split("(")[0]
                res.setdefault(name, []).append(float(r["Counter_Value"]))
    return res


def summarize_pmc(fetch_dir, write_dir, out, command_fetch, command_write, kind, copy_bytes,
                  bytes_per_launch):
    """PMC summary of the gate/up kernel `kind` (gemv | decode | gemm | gemm_q).  The GEMM template serves
    both projections; its gate/up instances are the ones whose second template argument is true."""
    kernel_key = GATE_UP_KERNELS[kind]
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")

    def pick(dct, key):
        ks = [k for k in dct if key in k and (kind in ("gemv", "decode") or k.rstrip().endswith("true>"))]
        if not ks:
            raise SystemExit(f"no kernel matching {key!r} in {sorted(dct)}")
        return dct[ks[0]]

    # the copy probe: the largest-fetch elementwise copy kernel
    copy_keys = [k for k in fetch if "neg" in k.lower()]
    copy_f = max((max(fetch[k]) for k in copy_keys), default=None)
    copy_wk = [k for k in write if "neg" in k.lower()]
    copy_w = max((max(write[k]) for k in copy_wk), default=None)
    f_factor = copy_bytes / (copy_f * 1024.0) if copy_f else None
    w_factor = copy_bytes / (copy_w * 1024.0) if copy_w else None
    kf = pick(fetch, kernel_key)
    kw = pick(write, kernel_key)
    fetch_b = sum(kf) / len(kf) * 1024.0 * (f_factor or 1.0)
    write_b = sum(kw) / len(kw) * 1024.0 * (w_factor or 1.0)
    what = {"gemv": "GEMV", "decode": "launch of the two-launch decode layer (routing + gate/up)"}.get(kind, "grouped GEMM")
    lines = [f"# HBM traffic of the gate/up {what} (rocprofv3 PMC)", "",
             f"fetch command: `{command_fetch}`", f"write command: `{command_write}`", "",
             f"kernel: `{kernel_key}`, dispatches: {len(kf)} (FETCH_SIZE), {len(kw)} (WRITE_SIZE)",
             f"copy probe: {copy_bytes} bytes; FETCH_SIZE {copy_f} KiB -> factor {f_factor}; "
             f"WRITE_SIZE {copy_w} KiB -> factor {w_factor}",
             f"mean FETCH_SIZE per dispatch (scaled): {fetch_b:.0f} bytes",
             f"mean WRITE_SIZE per dispatch (scaled): {write_b:.0f} bytes",
             f"algorithmic bytes per launch (same run): {bytes_per_launch:.0f}",
             "",
             f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
             f"source_hash: {source_hash(GATE_UP_SOURCES[kind])}"]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_mfma(d, out, command):
    """MFMA counters of the grouped GEMMs (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE): per kernel, the
    matrix work it issued (one MOP = 512 flops), and the share of SIMD cycles its MFMA pipe was
    busy.  GRBM_GUI_ACTIVE is summed over the 8 XCDs, SQ_VALU_MFMA_BUSY_CYCLES over the 1024
    SIMDs, so busy / (1024 * GRBM_GUI_ACTIVE / 8) is the pipe's busy fraction."""
    vals = {}
    for f in _csvs(d, "*counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "").split("(")[0].replace("void ", "")
                vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no counter_collection.csv under {d}")
    lines = ["# MFMA counters of the grouped GEMMs (rocprofv3 PMC)", "", f"command: `{command}`", "",
             "| kernel | dispatches | MOPS bf16 | MOPS f8 | issued TFLOP | active cycles per XCD | MFMA busy |",
             "|---|---|---|---|---|---|---|"]
    for name in sorted(vals):
        v = {c: sum(x) / len(x) for c, x in vals[name].items()}
        n = len(next(iter(vals[name].values())))
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + v.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        cyc = v.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024.0 * cyc) if cyc else float("nan")
        lines.append(f"| {name} | {n} | {v.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0.0):.4g} | "
                     f"{v.get('SQ_INSTS_VALU_MFMA_MOPS_F8', 0.0):.4g} | {mops * 512 / 1e12:.4f} | {cyc:.4g} | {busy:.3f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def recorded_traffic(kind, workload_key):
    """Traffic bytes per launch of gate/up kernel `kind` from the committed PMC summary, None if
    there is none or the kernel's sources changed since."""
    p = os.path.join(PROFILES, f"gate_up_{kind}_{workload_key}_pmc.md")
    if not os.path.exists(p):
        return None
    vals = {}
    for line in open(p):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_hash"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash(GATE_UP_SOURCES[kind]):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------------------------
# timing-only HIP events
# ---------------------------------------------------------------------------------------------

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _hip_runtime():
    """The HIP runtime library this process already has loaded (torch's), opened by its path so
    that the handle is the same instance, never a second runtime."""
    import ctypes
    with open("/proc/self/maps") as fh:
        paths = {ln.split()[-1] for ln in fh if "libamdhip64.so" in ln and ln.split()[-1].startswith("/")}
    if len(paths) != 1:
        raise SystemExit(f"bench: expected one loaded HIP runtime, found {sorted(paths)}")
    hip = ctypes.CDLL(paths.pop())
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


class TimingEvent:
    """A HIP event created with hipEventDisableSystemFence: recording it writes a timestamp when
    the work before it on the stream is done, without the system-scope cache writeback and
    invalidation that a default event performs (on this GPU a default event recorded between two
    kernels adds about 3 us to the step).  Read it only after a device synchronisation."""

    def __init__(self, hip):
        import ctypes
        self.hip, self.h = hip, ctypes.c_void_p()
        rc = hip.hipEventCreateWithFlags(ctypes.byref(self.h), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise SystemExit(f"bench: hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self.hip.hipEventRecord(self.h, stream.cuda_stream)
        if rc != 0:
            raise SystemExit(f"bench: hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise SystemExit(f"bench: hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if getattr(self, "h", None) and self.h.value:
            self.hip.hipEventDestroy(self.h)


# ---------------------------------------------------------------------------------------------
# the benchmark
# ---------------------------------------------------------------------------------------------

def plan_hot_set(cfg, seeded_map, moe, D, torch, np, gen, log, batches=8):
    """Hot-set placement planned on the GPU (moe_accumulate_counts, moe_plan_slots) from the
    routing of `batches` batches of the same workload that are not timed (other seeds), routed
    under the seeded map; returns (slot_map, the experts of slots 0..S-1)."""
    T, H, E, k, S = cfg.T, cfg.H, cfg.E, cfg.k, cfg.S
    dev = "cuda"
    R = T * k
    rcfg = moe.routing(E, k, cfg.score, cfg.renorm)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(S + 1, dtype=torch.int32, device=dev)
    perm, inv, mt, me = (torch.empty(R, dtype=torch.int32, device=dev) for _ in range(4))
    mw = torch.empty(R, dtype=torch.float32, device=dev)
    mc = torch.zeros(1, dtype=torch.int32, device=dev)
    nb = moe.moe_route_permute_workspace_size(T, rcfg, S, False)
    ws = D.workspace(nb)
    d_sm = D.to_device(seeded_map)
    hist = torch.zeros(E, dtype=torch.int64, device=dev)
    for b in range(batches):
        lg = D.to_device(gen.make_logits(cfg, batch=1000 + b))
        moe.moe_route_permute(None, moe.MOE_BF16, T, H, None, lg, None, rcfg, d_sm, S, idx, w, counts, off, perm,
                              inv, mc, mt, me, mw, ws, nb)
        moe.moe_accumulate_counts(counts, E, hist)
    sm = torch.empty(E, dtype=torch.int32, device=dev)
    moe.moe_plan_slots(hist, E, S, sm)
    torch.cuda.synchronize()
    planned = D.to_host(sm)
    h = D.to_host(hist)
    experts = np.empty(S, np.int32)
    experts[planned[planned >= 0]] = np.nonzero(planned >= 0)[0]
    log(f"hot set planned from {batches} batches: resident-row share {h[planned >= 0].sum() / h.sum():.3f} "
        f"(seeded map {h[seeded_map >= 0].sum() / h.sum():.3f})")
    return planned, experts


def graph_timing(args, step, w, stream, out, T, S, H, I, cfg, D, torch, log):
    """Time the layer as replays of one HIP graph of L consecutive layers (launch-bound small
    batches): layer l runs on its own device copy of the weights (same bytes, other addresses, so
    no layer finds another's weights in a cache) and on rotation l.  The replayed output of the last
    layer is checked against the eager step, before and after the timed replays."""
    L = args.graph_layers
    wbytes = w.nbytes_per_slot * S
    ncopy = max(1, min(L, int(64e9 // max(wbytes, 1))))
    copies = [w] + [D.DeviceWeights(w.wdtype, S, H, I, *[t.clone() if t is not None else None
                                                         for t in (w.w_gu, w.s_gu, w.w_d, w.s_d)])
                    for _ in range(ncopy - 1)]
    descs = [c.desc for c in copies]
    step(L - 1, dsc=descs[(L - 1) % ncopy])
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap):
        for l in range(L):
            step(l, dsc=descs[l % ncopy], sp=cap.cuda_stream)
    torch.cuda.synchronize()

    def check(when):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise SystemExit(f"bench: graph replay ({when}) differs from the eager step")
    check("first")
    n = max(2, args.steps // L)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    check("after timing")
    us = ms * 1e3 / L
    log(f"graph: {n} replays of {L} layers ({ncopy} weight copies): {ms * 1e3:.1f} us per replay, "
        f"{us:.2f} us per layer, {T / (us * 1e-6):.0f} tokens/s")
    del g
    return dict(layers=L, weight_copies=ncopy, us_per_layer=us, tokens_per_s=T / (us * 1e-6))


def run(args):
    import numpy as np
    import torch

    import routed_expert_ffn_05_amd as moe
    from routed_expert_ffn_05_amd import device as D
    from synth import gen

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    moe.lib()  # fail loudly without the HIP library
    torch.cuda.set_device(0)
    over = {}
    if args.T is not None:
        over["T"] = args.T
    if args.E is not None:  # e.g. a compute-bound prefill shape: few experts, many rows each
        over["E"] = args.E
    cfg = gen.config(args.config, **over)
    T, H, I, E, k, S = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.S
    t0 = time.time()
    slot_map, slot_expert = gen.make_slot_map(cfg)
    if args.plan_slots:
        if slot_map is None:
            raise SystemExit("--plan-slots needs a compact config (a resident subset of the experts)")
        slot_map, slot_expert = plan_hot_set(cfg, slot_map, moe, D, torch, np, gen, log)
    host_w = gen.stack_weights(cfg, slot_expert)
    log(f"generated {cfg.name} weights ({S} slots) in {time.time() - t0:.1f}s")
    w = D.upload_weights(cfg.wdtype, H, I, host_w)
    if not args.cpu_baseline:
        host_w = None
    lru = bool(args.lru)
    if lru and (slot_map is None or args.tiers or args.graph_layers or args.plan_slots):
        raise SystemExit("--lru needs a compact config and runs alone")
    if lru:
        # the backing store of every expert (the stand-in for the host tier) and the LRU state;
        # the slots start with the seeded experts
        t0 = time.time()
        store = D.upload_weights(cfg.wdtype, H, I, gen.stack_weights(cfg, range(E)))
        log(f"generated the store of all {E} experts in {time.time() - t0:.1f}s")
        w = D.DeviceWeights(cfg.wdtype, S, H, I, *[t.clone() if t is not None else None
                                                    for t in (w.w_gu, w.s_gu, w.w_d, w.s_d)])
        lru_init = (slot_map.copy(), np.asarray(slot_expert, np.int32).copy(), np.full(S, -1, np.int64))
    tiers = bool(args.tiers)
    if tiers and args.graph_layers:
        raise SystemExit("--tiers and --graph-layers are not combined")
    if tiers:
        # the second tier: a pool holding every expert without a resident slot, computing the
        # compact call's miss rows; both tiers are combined in row order
        if slot_map is None:
            raise SystemExit("--tiers needs a compact config (a resident subset of the experts)")
        pool_exp = np.nonzero(slot_map < 0)[0].astype(np.int32)
        if not args.plan_slots:
            _, pool_exp = gen.make_pool_map(cfg)     # the absent experts in the seeded order
        pool_map = np.full(E, -1, np.int32)
        pool_map[pool_exp] = np.arange(pool_exp.size, dtype=np.int32)
        P = int(pool_exp.size)
        t0 = time.time()
        w_pool = D.upload_weights(cfg.wdtype, H, I, gen.stack_weights(cfg, pool_exp))
        log(f"generated the pool tier ({P} experts) in {time.time() - t0:.1f}s")
    rot = []
    for r in range(args.rotate):
        # other activations per rotation; handed-in logits are other batches of the same workload
        # (same expert popularity, other noise)
        rc = cfg.replace(seed=cfg.seed * 1000 + 17 + r) if r else cfg
        x = gen.make_x(rc)
        lg = gen.make_logits(cfg, batch=r) if cfg.router != "weights" else None
        rot.append((x, lg))
    d_x = [D.to_device(x) for x, _ in rot]
    d_lg = [D.to_device(lg) if lg is not None else None for _, lg in rot]
    d_wr = D.to_device(gen.make_router_weights(cfg)) if cfg.router == "weights" else None
    d_sm = D.to_device(slot_map)
    xdt = moe.MOE_BF16 if cfg.xdtype == "bf16" else moe.MOE_F32
    odt = moe.MOE_BF16 if cfg.out_dtype == "bf16" else moe.MOE_F32
    rcfg = moe.routing(E, k, cfg.score, cfg.renorm)
    desc = w.desc
    # weight copies: consecutive steps run on different device copies of the same weights, so that
    # more than 1 GB of distinct weight bytes passes between two uses of one copy (the 256 MB
    # Infinity Cache cannot serve a step from the previous one); the LRU and two-tier modes
    # change or pair the weights and keep one copy
    wbytes = w.nbytes_per_slot * S
    ncopy = args.weight_copies
    if ncopy <= 0:
        ncopy = 1 if wbytes >= 8e9 else max(2, -(-int(1.5e9) // max(wbytes, 1)))
    if args.lru or args.tiers or args.graph_layers:
        ncopy = 1
    ncopy = max(1, min(ncopy, int(48e9 // max(wbytes, 1))))
    wcopies = [w] + [D.DeviceWeights(w.wdtype, S, H, I, *[t.clone() if t is not None else None
                                                          for t in (w.w_gu, w.s_gu, w.w_d, w.s_d)])
                     for _ in range(ncopy - 1)]
    descs = [c.desc for c in wcopies]
    path = {"auto": moe.MOE_PATH_AUTO, "gemv": moe.MOE_PATH_GEMV, "gemm": moe.MOE_PATH_GEMM,
            "invariant": moe.MOE_PATH_INVARIANT}[args.path]
    mode = {"A": moe.MOE_MODE_A, "B": moe.MOE_MODE_B}[args.mode]
    R = T * k
    dev = "cuda"
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
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
    rp_bytes = moe.moe_route_permute_workspace_size(T, rcfg, S, d_wr is not None)
    pws = D.workspace(rp_bytes)
    fbytes = moe.moe_expert_ffn_workspace_size(desc, T, k, path, mode)
    fws = D.workspace(fbytes)
    compact = d_sm is not None
    lru_step = [0]
    if lru:
        if args.rotate < args.warmup + args.steps + 8:
            log("note: --lru over a short rotation revisits batches; use --rotate >= warmup + steps + 8")
        d_se = D.to_device(lru_init[1])
        d_lu = D.to_device(lru_init[2])
        rws = D.workspace(moe.moe_refill_workspace_size(S))
        w_init = [t.clone() if t is not None else None for t in (w.w_gu, w.s_gu, w.w_d, w.s_d)]

        def lru_reset():
            d_sm.copy_(D.to_device(lru_init[0]))
            d_se.copy_(D.to_device(lru_init[1]))
            d_lu.copy_(D.to_device(lru_init[2]))
            for a, b in zip((w.w_gu, w.s_gu, w.w_d, w.s_d), w_init):
                if a is not None:
                    a.copy_(b)
            lru_step[0] = 0
    if tiers:
        d_pm = D.to_device(pool_map)
        desc_b = w_pool.desc
        counts_b = torch.empty(E, dtype=torch.int32, device=dev)
        off_b = torch.empty(P + 1, dtype=torch.int32, device=dev)
        perm_b = torch.empty(R, dtype=torch.int32, device=dev)
        inv_b = torch.empty(R, dtype=torch.int32, device=dev)
        mc_b = torch.zeros(1, dtype=torch.int32, device=dev)
        mt_b = torch.empty(R, dtype=torch.int32, device=dev)
        me_b = torch.empty(R, dtype=torch.int32, device=dev)
        mw_b = torch.empty(R, dtype=torch.float32, device=dev)
        y_b = torch.empty((R, H), dtype=torch.float32, device=dev)
        pb_bytes = moe.moe_permute_workspace_size(T, rcfg, P)
        pws_b = D.workspace(pb_bytes)
        fb_bytes = moe.moe_expert_ffn_workspace_size(desc_b, T, k, path, mode)
        fws_b = D.workspace(fb_bytes)
    # small decode batches: moe_layer's two-launch flow (routing + gate/up, down + combine), after
    # the router logits when router weights are given -- the same calls moe_layer makes
    fused = not (tiers or lru or args.staged) and moe.moe_layer_decode_fused(T, rcfg, desc, path, mode, xdt)
    if fused:
        row_slot = torch.empty(R, dtype=torch.int32, device=dev)
        a_dec = torch.empty((R, I), dtype=torch.float32, device=dev)
        err_w = D.workspace(256)
        lbuf = torch.empty((T, E), dtype=torch.float32, device=dev) if d_wr is not None else None
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i, ev=None, dsc=None, sp=sp):
        # with the LRU every call takes the next batch of the stream, so that no batch comes back
        r = (lru_step[0] if lru else i) % len(rot)
        dsc = descs[i % ncopy] if dsc is None else dsc
        if fused:
            lg = d_lg[r]
            if d_wr is not None:
                moe.moe_route(d_x[r], xdt, T, H, d_wr, None, None, rcfg, None, None, lbuf, None, 0, sp)
                lg = lbuf
            if ev is not None:
                ev[0].record(stream)
            moe.moe_decode_gate_up(d_x[r], xdt, T, lg, None, rcfg, d_sm, dsc, topk_idx, topk_w, row_slot, a_dec,
                                   mc, mt if compact else None, me if compact else None, mw if compact else None,
                                   err_w, sp)
            if ev is not None:
                ev[1].record(stream)
            moe.moe_decode_down_combine(dsc, T, rcfg, row_slot, topk_w, a_dec, out, odt, sp)
            return
        moe.moe_route_permute(d_x[r], xdt, T, H, d_wr, d_lg[r], None, rcfg, d_sm, S, topk_idx, topk_w, counts,
                              off, perm, inv, mc if compact else None, mt if compact else None,
                              me if compact else None, mw if compact else None, pws, rp_bytes, sp)
        if ev is not None:
            ev[0].record(stream)
        moe.moe_expert_gate_up(dsc, d_x[r], xdt, T, k, perm, off, path, mode, fws, fbytes, sp)
        if ev is not None:
            ev[1].record(stream)
        moe.moe_expert_down(dsc, T, k, off, path, mode, y, fws, fbytes, sp)
        if tiers:
            moe.moe_permute(topk_idx, topk_w, T, rcfg, d_pm, P, counts_b, off_b, perm_b, inv_b, mc_b, mt_b, me_b,
                            mw_b, pws_b, pb_bytes, sp)
            moe.moe_expert_ffn(desc_b, d_x[r], xdt, T, k, perm_b, off_b, path, mode, y_b, fws_b, fb_bytes, sp)
            moe.moe_combine_tiers(y, inv, y_b, inv_b, topk_w, T, k, H, out, odt, sp)
        else:
            moe.moe_combine(y, inv, topk_w, T, k, H, out, odt, sp)
        if lru:  # the misses of this call move into slots for the next one
            moe.moe_refill_slots(counts, E, lru_step[0], d_sm, d_se, d_lu, store.desc, desc, rws, rws.numel(), sp)
            lru_step[0] += 1

    # per-rotation routing statistics (outside the timed region)
    per_rot = []
    for r in range(len(rot)):
        step(r)
        torch.cuda.synchronize()
        cnt = np.bincount(topk_idx.cpu().numpy().reshape(-1), minlength=E)[:E] if fused else counts.cpu().numpy()
        if slot_map is not None:
            res = slot_map >= 0
            touched = int(((cnt > 0) & res).sum())
            n_res = int(cnt[res].sum())
            touched_b = int(((cnt > 0) & ~res).sum()) if tiers else 0
        else:
            touched = int((cnt > 0).sum())
            n_res = int(cnt.sum())
            touched_b = 0
        per_rot.append((touched, n_res, touched_b))
    slot_bytes_gu = (w.w_gu.numel() * w.w_gu.element_size() + (0 if w.s_gu is None else w.s_gu.numel() * w.s_gu.element_size())) // S
    slot_bytes_d = (w.w_d.numel() * w.w_d.element_size() + (0 if w.s_d is None else w.s_d.numel() * w.s_d.element_size())) // S
    xb = 2 if cfg.xdtype == "bf16" else 4

    gemm = moe.moe_resolve_path(desc, T, k, path, mode) == moe.MOE_PATH_GEMM

    def gate_up_bytes(r):
        touched, n_res, _ = per_rot[r]
        b = touched * slot_bytes_gu + T * H * xb + n_res * I * (2 if gemm else 4)
        if fused:  # the launch also reads the logits (and the slot map) to route the batch itself
            b += T * E * 4 + (E * 4 if compact else 0)
        return b

    def gate_up_flops(r):
        return per_rot[r][1] * 2.0 * H * 2 * I

    def layer_bytes(r):
        touched, n_res, touched_b = per_rot[r]
        b = (touched + touched_b) * (slot_bytes_gu + slot_bytes_d) + T * H * xb + T * H * (2 if odt == moe.MOE_BF16 else 4)
        b += (E * H * 4) if d_wr is not None else T * E * 4
        return b

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    hip = _hip_runtime()
    # the timed region: `repeats` blocks of K = args.steps steps each, every block bracketed by a
    # device synchronisation and its own pair of events; the reported step time is the median
    # block's.  Step i of the run uses rotation i and weight copy i in turn.
    R = max(1, args.repeats)
    evs = [[(TimingEvent(hip), TimingEvent(hip)) for _ in range(args.steps)] for _ in range(R)]
    block_ms, hosts, walls = [], [], []
    for rr in range(R):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            step(args.warmup + rr * args.steps + i, evs[rr][i])
        end.record(stream)
        hosts.append(time.perf_counter() - wall0)
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - wall0)
        block_ms.append(start.elapsed_time(end))
    med = int(np.argsort(block_ms)[len(block_ms) // 2])
    total_ms = block_ms[med]
    host, wall = hosts[med], walls[med]
    gu_ms = [a.elapsed_time(b) for blk in evs for a, b in blk]
    step_ids = [args.warmup + rr * args.steps + i for rr in range(R) for i in range(args.steps)]
    ms_per_step = total_ms / args.steps
    tokens_per_s = T * args.steps / (total_ms / 1e3)
    gu_bytes = [gate_up_bytes(i % len(rot)) for i in step_ids]
    achieved = sum(gu_bytes) / (sum(gu_ms) / 1e3) / 1e9
    med_ids = [args.warmup + med * args.steps + i for i in range(args.steps)]
    layer_gbs = sum(layer_bytes(i % len(rot)) for i in med_ids) / (total_ms / 1e3) / 1e9
    log(f"{R} x {args.steps} steps: median {ms_per_step * 1e3:.1f} us/step (blocks "
        f"{', '.join(f'{b * 1e3 / args.steps:.1f}' for b in block_ms)}; host enqueue {host * 1e6 / args.steps:.1f} us/step, "
        f"wall {wall * 1e6 / args.steps:.1f} us/step), "
        f"gate/up {np.mean(gu_ms) * 1e3:.1f} us avg, {achieved:.0f} GB/s; layer {layer_gbs:.0f} GB/s; "
        f"path {'gemm' if gemm else 'gemv'}{' (two-launch decode layer)' if fused else ''}; {ncopy} weight copies")

    lru_share = None
    if lru:
        # the LRU is deterministic: replay the same calls from the start, untimed, reading the
        # resident rows (slot_offsets[S]) of each timed call
        lru_reset()
        for r in range(len(rot)):
            step(r)
        for i in range(args.warmup):
            step(i)
        res_rows = 0
        for i in range(args.steps):
            step(i)
            res_rows += int(off[S].item())
        lru_share = res_rows / (args.steps * T * k)
        log(f"LRU: resident-row share over the timed calls {lru_share:.3f}")

    graph = None
    if args.graph_layers:
        graph = graph_timing(args, step, w, stream, out, T, S, H, I, cfg, D, torch, log)
        tokens_per_s = graph["tokens_per_s"]
        ms_per_step = graph["us_per_layer"] / 1e3

    # the staged step is moe_layer's own sequence: check one rotation bit for bit (with two tiers
    # the step goes past moe_layer; their identity with one pool is covered by the GPU tests)
    lay = None if (tiers or lru) else D.Layer(T=T, H=H, I=I, E=E, k=k, score=cfg.score, renorm=cfg.renorm, xdtype=cfg.xdtype,
                  out_dtype=cfg.out_dtype, weights=w, w_router=d_wr, slot_map=d_sm, path=path, mode=mode)
    if lay is not None:
        step(0)
        lay(d_x[0], d_lg[0])
        torch.cuda.synchronize()
        if not torch.equal(lay.out, out):
            raise SystemExit("bench: staged step and moe_layer disagree")
        del lay

    if args.copy_probe_mib:
        # a plain elementwise kernel that reads nb bytes and writes nb bytes (scales the counters)
        nb = args.copy_probe_mib << 20
        a = torch.empty(nb // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        log(f"copy probe: {nb} bytes read and written")

    # a record belongs to one workload: every option that changes the bytes a launch moves is part
    # of its key, so that a variant run finds no record (traffic null) rather than another's
    key = f"{cfg.name}_T{T}"
    if args.E is not None:
        key += f"_E{E}"
    if not gemm and mode == moe.MOE_MODE_B:
        key += "_modeB"
    for flag in ("plan_slots", "lru", "tiers"):
        if getattr(args, flag):
            key += "_" + flag
    kind = ("gemm_q" if mode == moe.MOE_MODE_B else "gemm") if gemm else "decode" if fused else "gemv"
    traffic = recorded_traffic(kind, key)
    tflops = sum(gate_up_flops(i % len(rot)) for i in step_ids) / (sum(gu_ms) / 1e3) / 1e12
    # the whole expert FFN (gate/up + down) of the median block: algorithmic flops over the step
    # time, i.e. with routing, permutation and combine counted as time
    layer_tflops = sum(gate_up_flops(i % len(rot)) * 1.5 for i in med_ids) / (total_ms / 1e3) / 1e12
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": (("moe::gemm::gemm_q_kernel" if mode == moe.MOE_MODE_B else "moe::gemm::gemm_kernel")
                           + " (gate/up)") if gemm else
                          "moe::gemv::decode_gate_up_kernel (routing + gate/up)" if fused else "moe::gemv::gate_up_kernel",
                "bytes_per_launch": round(sum(gu_bytes) / len(gu_bytes)),
                "avg_launch_us": round(float(np.mean(gu_ms)) * 1e3, 2)}
    if traffic is not None:
        # the counters' HBM bytes over the same live launch time: within 10 % of `achieved` when
        # the kernel moves about its algorithmic bytes, above it when it re-reads
        tgbs = traffic / (float(np.mean(gu_ms)) / 1e3) / 1e9
        roofline["traffic_GBs"] = round(tgbs, 1)
        roofline["traffic_vs_algorithmic"] = round(traffic / (sum(gu_bytes) / len(gu_bytes)), 3)
        # the counter rate and the event rate should agree within 10 %; a disagreement flags re-reads
        # (or a record that no longer describes the launch)
        roofline["traffic_agrees"] = bool(abs(tgbs / achieved - 1.0) <= 0.10)
    if gemm:
        # mode A runs bf16 MFMA on decoded weights; mode B the block-scaled f8f6f4 MFMA with E4M3
        # activations, which issues at the FP8 rate whether the weights are E4M3 or E2M1
        mfma_dt = "fp8" if mode == moe.MOE_MODE_B else "bf16"
        roofline["mfma_tflops"] = round(tflops, 1)
        roofline["mfma_dtype"] = mfma_dt
        roofline["mfma_peak"] = MFMA_PEAK_TFLOPS[mfma_dt]
        roofline["mfma_frac"] = round(tflops / MFMA_PEAK_TFLOPS[mfma_dt], 4)
        roofline["mfma_frac_of_bf16_peak"] = round(tflops / MFMA_PEAK_TFLOPS["bf16"], 4)
        roofline["layer_mfma_tflops"] = round(layer_tflops, 1)
        roofline["layer_mfma_frac"] = round(layer_tflops / MFMA_PEAK_TFLOPS[mfma_dt], 4)
    roofline["layer_hbm_frac"] = round(layer_gbs / HBM_PEAK_GBS, 4)

    cpu = None
    if args.cpu_baseline and not tiers:
        if T > 256:  # a prefill batch: the oracle runs the routing of the whole batch and the FFN of a token sample
            cpu = cpu_baseline_sample(cfg, rot, host_w, slot_map, args.cpu_seconds)
        else:
            cpu = cpu_baseline(cfg, rot, host_w, slot_map, args.cpu_seconds)

    rec = {
        "metric": "MoE layer tokens/s",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "repeats": R,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 activations",
                  "mxfp4": "mxfp4 weights, bf16 activations"}[cfg.wdtype],
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": {"workload": f"{cfg.name}: T={T} H={H} E={E} I={I} k={k} S={S} "
                               f"{cfg.score}-renorm weights={cfg.wdtype}"
                               + (f" + pool tier of {P} experts (miss rows computed, both tiers combined)" if tiers else ""),
                   "tokens_per_step": T, "rotations": len(rot), "weight_copies": ncopy,
                   "path": args.path, "mode": args.mode,
                   "layer_algorithmic_GBs": round(layer_gbs, 1),
                   "touched_slots_per_step": round(float(np.mean([p[0] for p in per_rot])), 2),
                   "resident_row_share": round(lru_share if lru else float(np.mean([p[1] for p in per_rot])) / (T * k), 4),
                   "slot_map": ("hot set planned on the GPU from 8 untimed batches" if args.plan_slots
                                else "seeded, then LRU refill after every call" if lru
                                else "seeded" if slot_map is not None else "all resident"),
                   "timing": (f"HIP graph of {graph['layers']} layers ({graph['weight_copies']} weight copies), "
                              f"per-layer time of its replays" if graph else
                              f"eager launches; median of {R} blocks of {args.steps} steps; gate/up timed by fence-free HIP events"),
                   "flow": ("two-launch decode layer (routing + gate/up; down + combine)" if fused else
                            "staged launches (route + permute, gate/up, down, combine)")},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    return rec


def cpu_baseline(cfg, rot, host_w, slot_map, budget_s):
    """Time the CPU oracle (fp64 numpy) on whole batches of the same workload until ~budget_s."""
    from oracle import moe_oracle as O
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    wr = gen.make_router_weights(cfg) if cfg.router == "weights" else None
    n_tok, spent, batches = 0, 0.0, 0
    for i in range(1000):
        x, lg = rot[i % len(rot)]
        t0 = time.perf_counter()
        O.layer(x, cfg.xdtype, host_w, cfg.wdtype, cfg.H, cfg.I, cfg.E, cfg.k, cfg.score, cfg.renorm,
                w_router=wr, logits=lg, slot_map=slot_map, S=cfg.S)
        spent += time.perf_counter() - t0
        n_tok += cfg.T
        batches += 1
        if batches % 10 == 0:
            log(f"cpu oracle batch {batches}: {spent:.1f}s")
        if spent >= budget_s:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), model)
    except OSError:  # pragma: no cover
        pass
    return {"value": round(n_tok / spent, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "cpus_available": len(os.sched_getaffinity(0)),
            "sample": f"{batches} batch(es) x {cfg.T} tokens of the same workload through the whole fp64 "
                      f"oracle layer (routing, permutation, per-slot dequantisation, FFN, combine), "
                      f"{spent:.1f} s"}


def prefill_leg(r):
    """The prefill numbers of a run's record: tokens/s, the gate/up GEMM's matrix-core rate and
    HBM rate (with its counter record), the whole expert FFN's rate over the step time."""
    rf = r["roofline"]
    return {"workload": r["config"]["workload"], "mode": r["config"]["mode"], "value": r["value"],
            "unit": r["unit"], "ms_per_step": r["ms_per_step"], "steps": r["steps"], "repeats": r["repeats"],
            "weight_copies": r["config"]["weight_copies"], "dtype": r["dtype"],
            "mfma_dtype": rf.get("mfma_dtype"), "mfma_peak": rf.get("mfma_peak"),
            "gate_up": {k: rf.get(k) for k in ("kernel", "avg_launch_us", "mfma_tflops", "mfma_frac",
                                               "mfma_frac_of_bf16_peak", "achieved", "frac", "bytes_per_launch",
                                               "traffic", "traffic_vs_algorithmic", "traffic_agrees")},
            "layer_mfma_tflops": rf.get("layer_mfma_tflops"), "layer_mfma_frac": rf.get("layer_mfma_frac"),
            "layer_hbm_frac": rf.get("layer_hbm_frac"), "cpu_baseline": r["cpu_baseline"]}


def cpu_baseline_sample(cfg, rot, host_w, slot_map, budget_s):
    """Time the CPU oracle on a prefill batch, bounded: its routing and permutation of the whole
    batch (timed once), and its expert FFN and combine on a token sample (4 tokens, doubled while
    the budget allows).  Reported as the oracle's per-token rate 1 / (t_route / T + t_ffn / n):
    the routing time spread over the batch plus the sample's FFN time per token."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    x, lg = rot[0]
    args = (x, cfg.xdtype, host_w, cfg.wdtype, cfg.H, cfg.I, cfg.E, cfg.k, cfg.score, cfg.renorm)
    t0 = time.perf_counter()
    O.layer(*args, logits=lg, slot_map=slot_map, S=cfg.S, tokens=np.zeros(0, np.int64))
    t_route = time.perf_counter() - t0
    log(f"cpu oracle: routing and permutation of the {cfg.T}-token batch {t_route:.1f}s")
    rng = np.random.default_rng(12345)
    n, spent = 4, t_route
    while True:
        tokens = np.sort(rng.choice(cfg.T, size=min(n, cfg.T), replace=False))
        t0 = time.perf_counter()
        O.layer(*args, logits=lg, slot_map=slot_map, S=cfg.S, tokens=tokens)
        dt = time.perf_counter() - t0
        spent += dt
        t_ffn = max(dt - t_route, 1e-9)
        log(f"cpu oracle: {tokens.size}-token sample {dt:.1f}s (FFN and combine {t_ffn:.1f}s)")
        if spent + 2 * dt > budget_s or n >= cfg.T:
            break
        n *= 2
    rate = 1.0 / (t_route / cfg.T + t_ffn / tokens.size)
    return {"value": round(rate, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "cpus_available": len(os.sched_getaffinity(0)),
            "sample": f"fp64 oracle on the {cfg.T}-token batch: routing and permutation of all tokens "
                      f"({t_route:.1f} s), expert FFN (per-slot dequantisation of the touched experts) and "
                      f"combine of {tokens.size} sampled tokens ({t_ffn:.1f} s); rate = 1 / (routing time per "
                      f"batch token + FFN time per sampled token)"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            return next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "unknown")
    except OSError:  # pragma: no cover
        return "unknown"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_bf16")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--repeats", type=int, default=5, help="timed blocks of --steps steps; the median is reported")
    ap.add_argument("--weight-copies", type=int, default=0,
                    help="device copies of the weights used in turn (0: enough for 1.5 GB between reuses)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", dest="prefill", action="store_false",
                    help="skip the prefill leg (the 4096-token FP8 batch, modes A and B) of the default run")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "gemm", "invariant"])
    ap.add_argument("--mode", default="A", choices=["A", "B"])
    ap.add_argument("--E", type=int, default=None, help="override the expert count of the config")
    ap.add_argument("--lru", action="store_true",
                    help="compact configs: after every call, refill the slots with the missed experts (LRU)")
    ap.add_argument("--plan-slots", action="store_true",
                    help="compact configs: resident slots from the hot-set planner instead of the seeded map")
    ap.add_argument("--graph-layers", type=int, default=0,
                    help="time the layer as replays of a HIP graph of this many layers (launch-bound batches)")
    ap.add_argument("--staged", action="store_true",
                    help="time the staged launches even where moe_layer takes the two-launch decode layer")
    ap.add_argument("--tiers", action="store_true",
                    help="compact configs: also compute the miss rows from a pool of the absent experts")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--summarize-kernels", default=None)
    ap.add_argument("--summarize-pmc", nargs=2, default=None)
    ap.add_argument("--summarize-mfma", default=None)
    ap.add_argument("--pmc-kind", default="gemv", choices=sorted(GATE_UP_KERNELS))
    ap.add_argument("--pmc-copy-bytes", type=int, default=512 << 20)
    ap.add_argument("--pmc-bytes-per-launch", type=float, default=0.0)
    ap.add_argument("--command", nargs="*", default=[])
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    if a.summarize_kernels:
        summarize_kernels(a.summarize_kernels, a.out, " ".join(a.command))
        return 0
    if a.summarize_mfma:
        summarize_mfma(a.summarize_mfma, a.out, " ".join(a.command))
        return 0
    if a.summarize_pmc:
        # the two commands as two arguments, or in one joined by " ;; "
        cmds = list(a.command) if len(a.command) == 2 else " ".join(a.command).split(" ;; ")
        summarize_pmc(a.summarize_pmc[0], a.summarize_pmc[1], a.out, cmds[0], cmds[-1], a.pmc_kind,
                      a.pmc_copy_bytes, a.pmc_bytes_per_launch)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}, "
              f"WORLD_SIZE {world}). Run with --gpus 1.", file=sys.stderr)
        return 2
    rec = run(a)
    if a.prefill and a.config == "decode_bf16" and a.T is None and a.E is None and not (
            a.tiers or a.lru or a.plan_slots or a.graph_layers):
        # the metric's prefill leg: the 4096-token chunk (FP8 weights, Zipf routing) on the matrix
        # cores, mode A (bf16 MFMA) and mode B (block-scaled FP8 MFMA), in the same process
        import gc
        import torch
        gc.collect()
        torch.cuda.empty_cache()
        legs = {}
        for mode in ("A", "B"):
            pa = argparse.Namespace(**vars(a))
            pa.config, pa.mode, pa.path = "prefill_fp8_zipf", mode, "auto"
            pa.steps, pa.warmup = a.prefill_steps, max(2, min(a.warmup, 5))
            pa.cpu_baseline = a.cpu_baseline and mode == "A"
            pa.copy_probe_mib = 0
            legs[mode] = prefill_leg(run(pa))
            gc.collect()
            torch.cuda.empty_cache()
        rec["prefill"] = dict(legs["A"], mode_b=legs["B"])
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

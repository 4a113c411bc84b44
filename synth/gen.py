"""Seeded generators for the five MoE-layer workloads and their shrunken variants.

Every tensor draws from its own numpy stream,
``default_rng(SeedSequence(entropy=seed, spawn_key=(tensor_id, ...)))``, so a
tensor (or one expert's weights) can be regenerated alone, in any order, on
any host.  Expert weights are drawn in fp32 and then encoded into the storage
format (bf16 by round-to-nearest-even, FP8 e4m3fn with one fp32 scale per
128x128 block, MXFP4 e2m1 with one e8m0 scale per 32 K-elements).  Encoding
is part of producing the inputs; decoding them is the layer's job and lives
elsewhere.

Workloads (the pages' MoE shape: 384 routed experts per layer, a resident
subset of 110 expert slots, 4096-token prefill chunks, FP4 checkpoint bytes --
vLLM-Moet README, MoET hybrid tables):

* ``tiny``              T=16, H=256, E=8, I=128, top-2 softmax, fp32
* ``decode_bf16``       T=4, H=4096, E=384, I=1024, top-8 sigmoid, bf16
* ``decode_fp8``        T=32, FP8 block-scaled weights, uniform logits
* ``prefill_fp8_zipf``  T=4096, FP8, Zipf(1.1)-biased logits
* ``compact_mxfp4``     T=1 or 4096, MXFP4, 110 resident slots, Zipf logits
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# tensor ids for the per-tensor streams
_X, _WR, _LOGITS, _ZIPF_RANK, _SLOTS, _EXPERT = 0, 1, 2, 3, 4, 10


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    E: int
    I: int
    k: int
    score: str          # "softmax" | "sigmoid"
    wdtype: str         # "f32" | "bf16" | "fp8" | "mxfp4"
    xdtype: str         # "f32" | "bf16"
    router: str         # "weights" | "uniform" | "zipf"
    seed: int
    x_sd: float = 1.0
    w_sd: float = 0.02
    wr_sd: float = 0.05
    zipf_s: float = 1.1
    resident: Optional[int] = None   # number of resident slots (compact), None = all
    renorm: bool = True
    out_dtype: str = "bf16"          # "f32" | "bf16"

    @property
    def S(self) -> int:
        return self.E if self.resident is None else self.resident

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", T=16, H=256, E=8, I=128, k=2, score="softmax", wdtype="f32",
                   xdtype="f32", router="weights", seed=0, x_sd=0.02, w_sd=0.02, wr_sd=0.1,
                   out_dtype="f32"),
    "decode_bf16": Config("decode_bf16", T=4, H=4096, E=384, I=1024, k=8, score="sigmoid",
                          wdtype="bf16", xdtype="bf16", router="weights", seed=1, wr_sd=0.05),
    "decode_fp8": Config("decode_fp8", T=32, H=4096, E=384, I=1024, k=8, score="sigmoid",
                         wdtype="fp8", xdtype="bf16", router="uniform", seed=2),
    "prefill_fp8_zipf": Config("prefill_fp8_zipf", T=4096, H=4096, E=384, I=1024, k=8,
                               score="sigmoid", wdtype="fp8", xdtype="bf16", router="zipf",
                               seed=3),
    "compact_mxfp4": Config("compact_mxfp4", T=4096, H=4096, E=384, I=1024, k=8,
                            score="sigmoid", wdtype="mxfp4", xdtype="bf16", router="zipf",
                            seed=4, resident=110),
}


def config(name: str, **overrides) -> Config:
    return CONFIGS[name].replace(**overrides) if overrides else CONFIGS[name]


def _rng(cfg: Config, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=cfg.seed, spawn_key=tuple(key)))


# ----------------------------------------------------------------------------------------------
# storage encoders (input production only)
# ----------------------------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _encode_e4m3fn(v: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes, saturating to +-448, round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_fp8_block128(w: np.ndarray):
    """[N,K] fp32 -> (codes uint8 [N,K], scales fp32 [ceil(N/128), ceil(K/128)]).

    scale = amax(block)/448 (1 for an all-zero block); code = e4m3fn(w/scale)."""
    N, K = w.shape
    nb, kb = -(-N // 128), -(-K // 128)
    pad = np.zeros((nb * 128, kb * 128), np.float32)
    pad[:N, :K] = w
    amax = np.abs(pad.reshape(nb, 128, kb, 128)).max(axis=(1, 3))
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = pad.reshape(nb, 128, kb, 128) / scale[:, None, :, None]
    codes = _encode_e4m3fn(q.reshape(nb * 128, kb * 128))[:N, :K]
    return np.ascontiguousarray(codes), scale


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)


def _encode_e2m1(m: np.ndarray) -> np.ndarray:
    """fp64 -> e2m1 4-bit codes (sign in bit 3), saturating at +-6, ties to even code."""
    mag = np.minimum(np.abs(m), 6.0)
    lo = np.clip(np.searchsorted(_E2M1_GRID, mag, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = mag - _E2M1_GRID[lo]
    d_hi = _E2M1_GRID[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    sign = ((m < 0) & (code != 0)).astype(np.uint8) << 3
    return code | sign


def quantize_mxfp4(w: np.ndarray):
    """[N,K] fp32 (K % 32 == 0) -> (packed uint8 [N, K/2], e8m0 uint8 [N, K/32]).

    OCP MX v1.0 rule: shared exponent X = floor(log2 amax) - 2 (e2m1's emax), element =
    e2m1(w / 2^X).  Byte j of a row holds K index 2j in its low nibble, 2j+1 in its high one."""
    N, K = w.shape
    assert K % 32 == 0
    blk = w.astype(np.float64).reshape(N, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(amax)                    # amax = m * 2^ex, m in [0.5, 1)
    X = np.where(amax > 0, ex - 1 - 2, -127)
    X = np.clip(X, -127, 127)
    scaled = np.ldexp(blk, -X[:, :, None])
    codes = _encode_e2m1(scaled).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), (X + 127).astype(np.uint8)


def _store(cfg: Config, w: np.ndarray):
    if cfg.wdtype == "f32":
        return np.ascontiguousarray(w, np.float32), None
    if cfg.wdtype == "bf16":
        return f32_to_bf16_bits(w), None
    if cfg.wdtype == "fp8":
        return quantize_fp8_block128(w)
    if cfg.wdtype == "mxfp4":
        return quantize_mxfp4(w)
    raise ValueError(cfg.wdtype)


def expert_weights(cfg: Config, e: int):
    """Storage bytes of expert e: (w_gu [2I,H], s_gu, w_d [H,I], s_d).

    w_gu rows [0,I) are the gate projection, rows [I,2I) the up projection."""
    r = _rng(cfg, _EXPERT, e, 0)
    gu = r.standard_normal((2 * cfg.I, cfg.H), dtype=np.float32)
    gu *= np.float32(cfg.w_sd)
    w_gu, s_gu = _store(cfg, gu)
    del gu
    r = _rng(cfg, _EXPERT, e, 1)
    d = r.standard_normal((cfg.H, cfg.I), dtype=np.float32)
    d *= np.float32(cfg.w_sd)
    w_d, s_d = _store(cfg, d)
    return w_gu, s_gu, w_d, s_d


def stack_weights(cfg: Config, experts, threads: Optional[int] = None):
    """Weights of the listed experts stacked slot-major: dict(w_gu, s_gu, w_d, s_d)."""
    experts = [int(e) for e in experts]
    if threads is None:
        import os
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda e: expert_weights(cfg, e), experts))
    out = {}
    for i, key in enumerate(("w_gu", "s_gu", "w_d", "s_d")):
        if parts and parts[0][i] is not None:
            out[key] = np.stack([p[i] for p in parts])
        else:
            out[key] = None
    return out


# ----------------------------------------------------------------------------------------------
# activations, router, slot map
# ----------------------------------------------------------------------------------------------

def make_x(cfg: Config) -> np.ndarray:
    """[T,H] activations: float32, or bf16 bit patterns (uint16)."""
    x = _rng(cfg, _X).standard_normal((cfg.T, cfg.H), dtype=np.float32) * np.float32(cfg.x_sd)
    return x.astype(np.float32) if cfg.xdtype == "f32" else f32_to_bf16_bits(x)


def make_router_weights(cfg: Config) -> np.ndarray:
    w = _rng(cfg, _WR).standard_normal((cfg.E, cfg.H), dtype=np.float32) * np.float32(cfg.wr_sd)
    return w.astype(np.float32)


def zipf_probabilities(cfg: Config) -> np.ndarray:
    """p_r proportional to r^-s, r = 1..E, assigned to experts through a seeded permutation."""
    r = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = r ** (-cfg.zipf_s)
    p /= p.sum()
    rank = _rng(cfg, _ZIPF_RANK).permutation(cfg.E)     # rank[e] = popularity rank of expert e
    return p[rank]


def make_logits(cfg: Config, batch: int = 0) -> np.ndarray:
    """[T,E] fp32 router logits for the configs that hand logits in directly.

    uniform: U[0,1).  zipf: ln p_e + Gumbel(0,1) noise, so that the top-1 pick of a token is
    expert e with probability p_e (Gumbel-max) and top-k picks are Gumbel-top-k samples.
    ``batch`` selects the noise of another batch of the same workload: the experts' popularity
    (the Zipf rank permutation) belongs to the config and is shared by every batch."""
    g = _rng(cfg, _LOGITS) if batch == 0 else _rng(cfg, _LOGITS, batch)
    if cfg.router == "uniform":
        return g.random((cfg.T, cfg.E), dtype=np.float32)
    if cfg.router == "zipf":
        lp = np.log(zipf_probabilities(cfg))
        return (lp[None, :] + g.gumbel(size=(cfg.T, cfg.E))).astype(np.float32)
    raise ValueError(cfg.router)


def make_slot_map(cfg: Config):
    """(slot_map [E] int32 or None, slot_expert [S] int32).

    Compact configs keep ``resident`` experts chosen by a seeded permutation pi:
    slot_map[pi[i]] = i for i < resident, -1 for every other expert."""
    if cfg.resident is None:
        return None, np.arange(cfg.E, dtype=np.int32)
    pi = _rng(cfg, _SLOTS).permutation(cfg.E).astype(np.int32)
    sm = np.full(cfg.E, -1, np.int32)
    sm[pi[: cfg.resident]] = np.arange(cfg.resident, dtype=np.int32)
    return sm, pi[: cfg.resident].copy()


def make_pool_map(cfg: Config):
    """(pool_map [E] int32, pool_expert [P] int32): the second weight pool of a compact config,
    holding exactly the experts without a resident slot (in the order of the same seeded
    permutation), pool_map[e] = its pool slot, -1 for the resident experts."""
    if cfg.resident is None:
        raise ValueError("a pool map needs a compact config")
    pi = _rng(cfg, _SLOTS).permutation(cfg.E).astype(np.int32)
    absent = pi[cfg.resident:]
    pm = np.full(cfg.E, -1, np.int32)
    pm[absent] = np.arange(absent.size, dtype=np.int32)
    return pm, absent.copy()


@dataclasses.dataclass
class LayerInputs:
    cfg: Config
    x: np.ndarray
    w_router: Optional[np.ndarray]
    logits: Optional[np.ndarray]
    bias: Optional[np.ndarray]
    slot_map: Optional[np.ndarray]
    slot_expert: np.ndarray
    weights: Optional[dict]

    def expert(self, e: int):
        """Storage bytes of any expert (resident or not)."""
        return expert_weights(self.cfg, e)


def make_inputs(cfg: Config, with_weights: bool = True, bias: bool = False) -> LayerInputs:
    x = make_x(cfg)
    w_router = make_router_weights(cfg) if cfg.router == "weights" else None
    logits = None if cfg.router == "weights" else make_logits(cfg)
    b = None
    if bias:
        b = (_rng(cfg, _WR, 1).standard_normal(cfg.E, dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    slot_map, slot_expert = make_slot_map(cfg)
    weights = stack_weights(cfg, slot_expert) if with_weights else None
    return LayerInputs(cfg, x, w_router, logits, b, slot_map, slot_expert, weights)


def harmonic(n: int, s: float) -> float:
    return math.fsum(r ** (-s) for r in range(1, n + 1))

"""Device-buffer marshalling for the C ABI: numpy arrays in, torch device tensors out.

PyTorch serves only as the device allocator here; every computation happens in libmoe_hip.so.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import (MOE_BF16, MOE_F32, MOE_PATH_AUTO, MOE_MODE_A, DTYPES, moe_layer, moe_layer_workspace_size,
               routing, weights)


def to_device(a: Optional[np.ndarray], device="cuda"):
    """numpy -> contiguous torch tensor on the device, byte-for-byte (uint16 is carried as int16,
    uint8 as uint8)."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def empty(shape, dtype, device="cuda"):
    import torch
    return torch.empty(shape, dtype=dtype, device=device)


def workspace(nbytes: int, device="cuda"):
    """A byte workspace whose address is 256-byte aligned (torch's allocator aligns to >= 512)."""
    import torch
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


@dataclasses.dataclass
class DeviceWeights:
    wdtype: str
    S: int
    H: int
    I: int
    w_gu: object
    s_gu: object
    w_d: object
    s_d: object

    @property
    def desc(self):
        return weights(self.wdtype, self.S, self.H, self.I, self.w_gu, self.s_gu, self.w_d, self.s_d)

    @property
    def nbytes_per_slot(self) -> int:
        n = 0
        for t in (self.w_gu, self.s_gu, self.w_d, self.s_d):
            if t is not None:
                n += t.numel() * t.element_size() // self.S
        return n


def upload_weights(wdtype: str, H: int, I: int, w: dict, device="cuda") -> DeviceWeights:
    S = w["w_gu"].shape[0]
    return DeviceWeights(wdtype, S, H, I, to_device(w["w_gu"], device), to_device(w.get("s_gu"), device),
                         to_device(w["w_d"], device), to_device(w.get("s_d"), device))


class Layer:
    """One MoE layer's device state plus its preallocated buffers; ``__call__`` runs moe_layer."""

    def __init__(self, *, T, H, I, E, k, score, renorm, xdtype, out_dtype, weights: DeviceWeights,
                 w_router=None, slot_map=None, bias=None, path=MOE_PATH_AUTO, mode=MOE_MODE_A,
                 device="cuda"):
        import torch
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.cfg = routing(E, k, score, renorm)
        self.xdt = MOE_BF16 if xdtype == "bf16" else MOE_F32
        self.odt = MOE_BF16 if out_dtype == "bf16" else MOE_F32
        self.w = weights
        self.wdesc = weights.desc
        self.w_router = w_router
        self.slot_map = slot_map
        self.bias = bias
        self.path, self.mode = path, mode
        R = T * k
        self.out = torch.empty((T, H), dtype=torch.int16 if self.odt == MOE_BF16 else torch.float32, device=device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.miss_count = torch.zeros(1, dtype=torch.int32, device=device)
        self.miss_token = torch.empty(max(R, 1), dtype=torch.int32, device=device)
        self.miss_expert = torch.empty(max(R, 1), dtype=torch.int32, device=device)
        self.miss_weight = torch.empty(max(R, 1), dtype=torch.float32, device=device)
        self.ws_bytes = moe_layer_workspace_size(T, self.cfg, self.wdesc, path, mode, w_router is not None)
        self.ws = workspace(self.ws_bytes, device)

    def __call__(self, x, logits=None, stream=None):
        compact = self.slot_map is not None
        moe_layer(x, self.xdt, self.T, self.w_router, logits, self.bias, self.cfg, self.slot_map, self.wdesc,
                  self.path, self.mode, self.out, self.odt, self.topk_idx, self.topk_w,
                  self.miss_count if compact else None, self.miss_token if compact else None,
                  self.miss_expert if compact else None, self.miss_weight if compact else None,
                  self.ws, self.ws_bytes, stream)
        return self.out


def bf16_bits_to_float(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


__all__ = ["to_device", "to_host", "empty", "workspace", "DeviceWeights", "upload_weights", "Layer",
           "bf16_bits_to_float", "DTYPES"]

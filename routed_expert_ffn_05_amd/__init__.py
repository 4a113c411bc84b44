"""Python binding of libmoe_hip.so, the C ABI of the routed MoE FFN layer on MI355X (gfx950).

Argument marshalling only: every function below forwards to the exported C function of the same
name (declared in include/moe.h).  Pointer arguments accept a torch tensor (its data pointer is
passed), an int address or None (NULL).  ``stream`` defaults to torch's current HIP stream.
A non-zero status raises :class:`MoeError` with the library's message.  There is no fallback:
if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_hip.so")

# moe_status
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_DEVICE = range(6)
# moe_dtype
MOE_F32, MOE_BF16, MOE_FP8_E4M3_B128, MOE_MXFP4 = range(4)
# moe_score / moe_path / moe_mode
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_GEMM, MOE_PATH_INVARIANT = 0, 1, 2, 3
MOE_PATH_TILES_CONTIGUOUS = 0x100  # flag, or'ed into a path value
MOE_MODE_A, MOE_MODE_B = 0, 1

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3_B128, "mxfp4": MOE_MXFP4}
SCORES = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}


class MoeError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {status_string(status)} ({status}): {msg}")
        self.status = status


class moe_weights(ctypes.Structure):
    _fields_ = [("wdtype", ctypes.c_int), ("S", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("w_gu", ctypes.c_void_p), ("s_gu", ctypes.c_void_p),
                ("w_d", ctypes.c_void_p), ("s_d", ctypes.c_void_p)]


class moe_routing(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("k", ctypes.c_int), ("score", ctypes.c_int), ("renorm", ctypes.c_int)]


_P, _I, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_W, _R = ctypes.POINTER(moe_weights), ctypes.POINTER(moe_routing)

_SIGS = {
    "moe_route_workspace_size": (_Z, [_I, _R, _I]),
    "moe_route": (_I, [_P, _I, _I, _I, _P, _P, _P, _R, _P, _P, _P, _P, _Z, _P]),
    "moe_permute_workspace_size": (_Z, [_I, _R, _I]),
    "moe_permute": (_I, [_P, _P, _I, _R, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_route_permute_workspace_size": (_Z, [_I, _R, _I, _I]),
    "moe_route_permute": (_I, [_P, _I, _I, _I, _P, _P, _P, _R, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, _Z, _P]),
    "moe_expert_ffn_workspace_size": (_Z, [_W, _I, _I, _I, _I]),
    "moe_expert_ffn_workspace_layout": (_I, [_W, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_expert_ffn": (_I, [_W, _P, _I, _I, _I, _P, _P, _I, _I, _P, _P, _Z, _P]),
    "moe_expert_gate_up": (_I, [_W, _P, _I, _I, _I, _P, _P, _I, _I, _P, _Z, _P]),
    "moe_expert_down": (_I, [_W, _I, _I, _P, _I, _I, _P, _P, _Z, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _P, _I, _P]),
    "moe_combine_tiers": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P]),
    "moe_accumulate_counts": (_I, [_P, _I, _P, _P]),
    "moe_plan_slots": (_I, [_P, _I, _I, _P, _P]),
    "moe_refill_workspace_size": (_Z, [_I]),
    "moe_refill_slots": (_I, [_P, _I, ctypes.c_longlong, _P, _P, _P, _W, _W, _P, _Z, _P]),
    "moe_layer_workspace_size": (_Z, [_I, _R, _W, _I, _I, _I]),
    "moe_layer": (_I, [_P, _I, _I, _P, _P, _P, _R, _P, _W, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P,
                       _P, _Z, _P]),
    "moe_layer_static": (_I, [_P, _I, _I, _P, _P, _P, _R, _P, _W, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P]),
    "moe_quantize_mx_e4m3": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _P]),
    "moe_check_device_error": (_I, [_P, _P]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
    "moe_resolve_path": (_I, [_W, _I, _I, _I, _I]),
    "moe_layer_decode_fused": (_I, [_I, _R, _W, _I, _I, _I]),
    "moe_decode_gate_up": (_I, [_P, _I, _I, _P, _P, _R, _P, _W, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_decode_down_combine": (_I, [_W, _I, _R, _P, _P, _P, _P, _I, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_hip.so (built in-tree by routed_expert_ffn_05_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m routed_expert_ffn_05_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


# ---------------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------------

def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is not None:
        return s if isinstance(s, int) else s.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, func: str):
    if status != MOE_OK:
        raise MoeError(status, func, lib().moe_last_error().decode())


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def version() -> str:
    return lib().moe_version().decode()


def routing(E: int, k: int, score, renorm: bool = True) -> moe_routing:
    sc = SCORES[score] if isinstance(score, str) else int(score)
    return moe_routing(E, k, sc, 1 if renorm else 0)


def weights(wdtype, S: int, H: int, I: int, w_gu, s_gu, w_d, s_d) -> moe_weights:
    dt = DTYPES[wdtype] if isinstance(wdtype, str) else int(wdtype)
    return moe_weights(dt, S, H, I, _ptr(w_gu), _ptr(s_gu), _ptr(w_d), _ptr(s_d))


def _ref(x):
    return ctypes.byref(x) if x is not None else None


# ---------------------------------------------------------------------------------------------
# the C ABI, one Python function per export
# ---------------------------------------------------------------------------------------------

def moe_route_workspace_size(T, cfg, with_router_weights) -> int:
    return lib().moe_route_workspace_size(T, _ref(cfg), int(bool(with_router_weights)))


def moe_route(x, x_dtype, T, H, w_router, logits, bias, cfg, topk_idx, topk_w, logits_out=None,
              ws=None, ws_bytes=0, stream=None):
    _check(lib().moe_route(_ptr(x), x_dtype, T, H, _ptr(w_router), _ptr(logits), _ptr(bias), _ref(cfg),
                           _ptr(topk_idx), _ptr(topk_w), _ptr(logits_out), _ptr(ws), ws_bytes,
                           _stream(stream)), "moe_route")


def moe_permute_workspace_size(T, cfg, S) -> int:
    return lib().moe_permute_workspace_size(T, _ref(cfg), S)


def moe_permute(topk_idx, topk_w, T, cfg, slot_map, S, counts, slot_offsets, perm, inv_perm,
                miss_count, miss_token, miss_expert, miss_weight, ws, ws_bytes, stream=None):
    _check(lib().moe_permute(_ptr(topk_idx), _ptr(topk_w), T, _ref(cfg), _ptr(slot_map), S, _ptr(counts),
                             _ptr(slot_offsets), _ptr(perm), _ptr(inv_perm), _ptr(miss_count),
                             _ptr(miss_token), _ptr(miss_expert), _ptr(miss_weight), _ptr(ws), ws_bytes,
                             _stream(stream)), "moe_permute")


def moe_route_permute_workspace_size(T, cfg, S, with_router_weights) -> int:
    return lib().moe_route_permute_workspace_size(T, _ref(cfg), S, int(bool(with_router_weights)))


def moe_route_permute(x, x_dtype, T, H, w_router, logits, bias, cfg, slot_map, S, topk_idx, topk_w, counts,
                      slot_offsets, perm, inv_perm, miss_count, miss_token, miss_expert, miss_weight, ws,
                      ws_bytes, stream=None):
    _check(lib().moe_route_permute(_ptr(x), x_dtype, T, H, _ptr(w_router), _ptr(logits), _ptr(bias), _ref(cfg),
                                   _ptr(slot_map), S, _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                                   _ptr(slot_offsets), _ptr(perm), _ptr(inv_perm), _ptr(miss_count),
                                   _ptr(miss_token), _ptr(miss_expert), _ptr(miss_weight), _ptr(ws), ws_bytes,
                                   _stream(stream)), "moe_route_permute")


def moe_expert_ffn_workspace_size(w, T, k, path, mode) -> int:
    return lib().moe_expert_ffn_workspace_size(_ref(w), T, k, path, mode)


def moe_expert_ffn_workspace_layout(w, T, k, path, mode):
    """[offset of a, offset of its E4M3 codes, offset of their E8M0 scales, format of a] in the
    expert-FFN workspace (offsets that do not apply are None)."""
    off = (ctypes.c_size_t * 4)()
    _check(lib().moe_expert_ffn_workspace_layout(_ref(w), T, k, path, mode, off), "moe_expert_ffn_workspace_layout")
    none = (1 << (8 * ctypes.sizeof(ctypes.c_size_t))) - 1
    return [None if v == none else int(v) for v in off[:3]] + [int(off[3])]


def moe_resolve_path(w, T, k, path, mode) -> int:
    return lib().moe_resolve_path(_ref(w), T, k, path, mode)


def moe_decode_gate_up(x, x_dtype, T, logits, bias, cfg, slot_map, w, topk_idx, topk_w, row_slot, a, miss_count,
                       miss_token, miss_expert, miss_weight, err, stream=None):
    _check(lib().moe_decode_gate_up(_ptr(x), x_dtype, T, _ptr(logits), _ptr(bias), _ref(cfg), _ptr(slot_map),
                                    _ref(w), _ptr(topk_idx), _ptr(topk_w), _ptr(row_slot), _ptr(a),
                                    _ptr(miss_count), _ptr(miss_token), _ptr(miss_expert), _ptr(miss_weight),
                                    _ptr(err), _stream(stream)), "moe_decode_gate_up")


def moe_decode_down_combine(w, T, cfg, row_slot, topk_w, a, out, out_dtype, stream=None):
    _check(lib().moe_decode_down_combine(_ref(w), T, _ref(cfg), _ptr(row_slot), _ptr(topk_w), _ptr(a), _ptr(out),
                                         out_dtype, _stream(stream)), "moe_decode_down_combine")


def moe_layer_decode_fused(T, cfg, w, path, mode, x_dtype) -> bool:
    """Whether moe_layer runs this batch as the two-launch decode layer (same results as the
    staged launches)."""
    r = lib().moe_layer_decode_fused(T, _ref(cfg), _ref(w), path, mode, x_dtype)
    if r < 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "moe_layer_decode_fused", lib().moe_last_error().decode())
    return bool(r)


def moe_expert_ffn(w, x, x_dtype, T, k, perm, slot_offsets, path, mode, y_perm, ws, ws_bytes,
                   stream=None):
    _check(lib().moe_expert_ffn(_ref(w), _ptr(x), x_dtype, T, k, _ptr(perm), _ptr(slot_offsets), path,
                                mode, _ptr(y_perm), _ptr(ws), ws_bytes, _stream(stream)), "moe_expert_ffn")


def moe_expert_gate_up(w, x, x_dtype, T, k, perm, slot_offsets, path, mode, ws, ws_bytes, stream=None):
    _check(lib().moe_expert_gate_up(_ref(w), _ptr(x), x_dtype, T, k, _ptr(perm), _ptr(slot_offsets), path,
                                    mode, _ptr(ws), ws_bytes, _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(w, T, k, slot_offsets, path, mode, y_perm, ws, ws_bytes, stream=None):
    _check(lib().moe_expert_down(_ref(w), T, k, _ptr(slot_offsets), path, mode, _ptr(y_perm), _ptr(ws),
                                 ws_bytes, _stream(stream)), "moe_expert_down")


def moe_quantize_mx_e4m3(x, x_dtype, rows, K, codes=None, scales=None, deq=None, deq_dtype=MOE_F32, stream=None):
    _check(lib().moe_quantize_mx_e4m3(_ptr(x), x_dtype, rows, K, _ptr(codes), _ptr(scales), _ptr(deq), deq_dtype,
                                      _stream(stream)), "moe_quantize_mx_e4m3")


def moe_combine(y_perm, inv_perm, topk_w, T, k, H, out, out_dtype, stream=None):
    _check(lib().moe_combine(_ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), T, k, H, _ptr(out), out_dtype,
                             _stream(stream)), "moe_combine")


def moe_combine_tiers(y_a, inv_a, y_b, inv_b, topk_w, T, k, H, out, out_dtype, stream=None):
    _check(lib().moe_combine_tiers(_ptr(y_a), _ptr(inv_a), _ptr(y_b), _ptr(inv_b), _ptr(topk_w), T, k, H,
                                   _ptr(out), out_dtype, _stream(stream)), "moe_combine_tiers")


def moe_accumulate_counts(counts, E, hist, stream=None):
    _check(lib().moe_accumulate_counts(_ptr(counts), E, _ptr(hist), _stream(stream)), "moe_accumulate_counts")


def moe_plan_slots(hist, E, S, slot_map, stream=None):
    _check(lib().moe_plan_slots(_ptr(hist), E, S, _ptr(slot_map), _stream(stream)), "moe_plan_slots")


def moe_refill_workspace_size(S) -> int:
    return lib().moe_refill_workspace_size(S)


def moe_refill_slots(counts, E, step, slot_map, slot_expert, last_use, store, slots, ws, ws_bytes, stream=None):
    _check(lib().moe_refill_slots(_ptr(counts), E, step, _ptr(slot_map), _ptr(slot_expert), _ptr(last_use),
                                  _ref(store), _ref(slots), _ptr(ws), ws_bytes, _stream(stream)), "moe_refill_slots")


def moe_layer_workspace_size(T, cfg, w, path, mode, with_router_weights) -> int:
    return lib().moe_layer_workspace_size(T, _ref(cfg), _ref(w), path, mode, int(bool(with_router_weights)))


def moe_layer(x, x_dtype, T, w_router, logits, bias, cfg, slot_map, w, path, mode, out, out_dtype,
              topk_idx, topk_w, miss_count, miss_token, miss_expert, miss_weight, ws, ws_bytes,
              stream=None):
    _check(lib().moe_layer(_ptr(x), x_dtype, T, _ptr(w_router), _ptr(logits), _ptr(bias), _ref(cfg),
                           _ptr(slot_map), _ref(w), path, mode, _ptr(out), out_dtype, _ptr(topk_idx),
                           _ptr(topk_w), _ptr(miss_count), _ptr(miss_token), _ptr(miss_expert),
                           _ptr(miss_weight), _ptr(ws), ws_bytes, _stream(stream)), "moe_layer")


MOE_STATIC_WORKSPACE_BYTES = 32 << 20


def moe_layer_static(x, x_dtype, T, w_router, logits, bias, cfg, slot_map, w, path, mode, out, out_dtype,
                     topk_idx, topk_w, miss_count, miss_token, miss_expert, miss_weight, stream=None):
    _check(lib().moe_layer_static(_ptr(x), x_dtype, T, _ptr(w_router), _ptr(logits), _ptr(bias), _ref(cfg),
                                  _ptr(slot_map), _ref(w), path, mode, _ptr(out), out_dtype, _ptr(topk_idx),
                                  _ptr(topk_w), _ptr(miss_count), _ptr(miss_token), _ptr(miss_expert),
                                  _ptr(miss_weight), _stream(stream)), "moe_layer_static")


def moe_check_device_error(ws, stream=None):
    _check(lib().moe_check_device_error(_ptr(ws), _stream(stream)), "moe_check_device_error")

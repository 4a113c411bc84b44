"""The C-ABI library without a GPU: it loads, exports every function include/moe.h declares, and
rejects malformed arguments on the host (validation precedes every HIP call, so none of these
calls touches a device)."""
import os
import re
import subprocess

import pytest

import routed_expert_ffn_05_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libmoe_hip.so is not built (run python -m routed_expert_ffn_05_amd.build)")
    return moe.lib()


def test_every_declared_function_is_exported(L):
    names = _declared()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(moe.exported_symbols()) == names       # the binding covers exactly the header


def test_version_and_status_strings(L):
    assert "gfx950" in moe.version()
    assert moe.status_string(moe.MOE_ERR_WORKSPACE) == "workspace too small"
    assert moe.status_string(12345) == "unknown status"


def _expect(status, fn, *args, **kw):
    with pytest.raises(moe.MoeError) as ei:
        fn(*args, **kw)
    assert ei.value.status == status, str(ei.value)
    return str(ei.value)


FAKE = 1 << 20          # a non-NULL, 256-byte aligned address never dereferenced by validation


def test_route_validation(L):
    cfg = moe.routing(8, 2, "softmax")
    # both / neither of w_router and logits
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, FAKE, moe.MOE_F32, 4, 64, FAKE, FAKE, None, cfg, FAKE, FAKE,
            None, FAKE, 1 << 20, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, FAKE, moe.MOE_F32, 4, 64, None, None, None, cfg, FAKE, FAKE,
            None, FAKE, 1 << 20, 0)
    # k > E, k = 0, E too large, bad score
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, None, 0, 4, 64, None, FAKE, None, moe.routing(8, 9, 0),
            FAKE, FAKE, None, None, 0, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, None, 0, 4, 64, None, FAKE, None, moe.routing(8, 0, 0),
            FAKE, FAKE, None, None, 0, 0)
    _expect(moe.MOE_ERR_UNSUPPORTED, moe.moe_route, None, 0, 4, 64, None, FAKE, None, moe.routing(4096, 8, 0),
            FAKE, FAKE, None, None, 0, 0)
    _expect(moe.MOE_ERR_UNSUPPORTED, moe.moe_route, None, 0, 4, 64, None, FAKE, None, moe.routing(128, 65, 0),
            FAKE, FAKE, None, None, 0, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, None, 0, 4, 64, None, FAKE, None, moe.routing(8, 2, 7),
            FAKE, FAKE, None, None, 0, 0)
    # negative T; missing outputs; misaligned x; short workspace
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, None, 0, -1, 64, None, FAKE, None, cfg, FAKE, FAKE, None,
            None, 0, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, None, 0, 4, 64, None, FAKE, None, cfg, None, FAKE, None,
            None, 0, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_route, FAKE + 4, moe.MOE_F32, 4, 64, FAKE, None, None, cfg, FAKE,
            FAKE, None, FAKE, 1 << 20, 0)
    # the router GEMV covers H up to 8192 (8 chunks of 4 per thread, 256 threads)
    _expect(moe.MOE_ERR_UNSUPPORTED, moe.moe_route, FAKE, moe.MOE_F32, 4, 8196, FAKE, None, None, cfg, FAKE,
            FAKE, None, FAKE, 1 << 20, 0)
    _expect(moe.MOE_ERR_UNSUPPORTED, moe.moe_route_permute, FAKE, moe.MOE_F32, 4, 8196, FAKE, None, None, cfg,
            None, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, FAKE, 1 << 20, 0)
    msg = _expect(moe.MOE_ERR_WORKSPACE, moe.moe_route, FAKE, moe.MOE_F32, 4, 64, FAKE, None, None, cfg, FAKE,
                  FAKE, None, FAKE, 16, 0)
    assert "need" in msg
    assert moe.moe_route_workspace_size(4, cfg, 1) >= 4 * 8 * 4


def test_permute_validation(L):
    cfg = moe.routing(16, 2, "sigmoid")
    args = dict(topk_idx=FAKE, topk_w=FAKE, T=4, cfg=cfg, slot_map=None, S=16, counts=FAKE, slot_offsets=FAKE,
                perm=FAKE, inv_perm=FAKE, miss_count=None, miss_token=None, miss_expert=None, miss_weight=None,
                ws=FAKE, ws_bytes=256, stream=0)
    def call(**kw):
        a = dict(args)
        a.update(kw)
        return moe.moe_permute(*a.values())
    _expect(moe.MOE_ERR_INVALID_ARG, call, S=8)                              # S != E without a map
    _expect(moe.MOE_ERR_INVALID_ARG, call, slot_map=FAKE, S=8)                # map without miss buffers
    _expect(moe.MOE_ERR_INVALID_ARG, call, S=17)
    _expect(moe.MOE_ERR_INVALID_ARG, call, ws=FAKE + 64)                      # misaligned workspace
    _expect(moe.MOE_ERR_WORKSPACE, call, ws_bytes=8)
    _expect(moe.MOE_ERR_INVALID_ARG, call, perm=None)


def test_expert_ffn_validation(L):
    def w(dt, S=8, H=256, I=128, sc=True):
        return moe.weights(dt, S, H, I, FAKE, FAKE if sc else None, FAKE, FAKE if sc else None)
    big = 1 << 30
    ok = dict(w=w("bf16"), x=FAKE, x_dtype=moe.MOE_BF16, T=4, k=2, perm=FAKE, slot_offsets=FAKE,
              path=moe.MOE_PATH_GEMV, mode=moe.MOE_MODE_A, y_perm=FAKE, ws=FAKE, ws_bytes=big, stream=0)
    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return moe.moe_expert_ffn(*a.values())
    _expect(moe.MOE_ERR_INVALID_ARG, call, w=w(9))                            # unknown dtype
    _expect(moe.MOE_ERR_INVALID_ARG, call, w=w("fp8", sc=False))              # scaled dtype without scales
    _expect(moe.MOE_ERR_UNSUPPORTED, call, w=w("mxfp4", H=272))               # K % 32 for MXFP4
    _expect(moe.MOE_ERR_UNSUPPORTED, call, w=w("fp8", I=136))                 # K % 16 for FP8
    _expect(moe.MOE_ERR_UNSUPPORTED, call, w=w("bf16", H=16384))
    _expect(moe.MOE_ERR_INVALID_ARG, call, x_dtype=moe.MOE_FP8_E4M3_B128)
    _expect(moe.MOE_ERR_INVALID_ARG, call, path=7)
    _expect(moe.MOE_ERR_INVALID_ARG, call, mode=5)
    _expect(moe.MOE_ERR_INVALID_ARG, call, x=FAKE + 8)
    _expect(moe.MOE_ERR_WORKSPACE, call, ws_bytes=1024)
    _expect(moe.MOE_ERR_INVALID_ARG, call, slot_offsets=None)
    n = moe.moe_expert_ffn_workspace_size(w("bf16"), 4, 2, moe.MOE_PATH_GEMV, moe.MOE_MODE_A)
    assert n >= 4 * 2 * 128 * 4
    # mode B: the matrix-core path only for FP8 / MXFP4 weights; one scale per 32 elements
    _expect(moe.MOE_ERR_UNSUPPORTED, call, path=moe.MOE_PATH_GEMM, mode=moe.MOE_MODE_B)
    _expect(moe.MOE_ERR_UNSUPPORTED, call, w=w("bf16", H=264), mode=moe.MOE_MODE_B)
    _expect(moe.MOE_ERR_UNSUPPORTED, call, w=w("fp8", H=8192), path=moe.MOE_PATH_GEMM, mode=moe.MOE_MODE_B)
    nb = moe.moe_expert_ffn_workspace_size(w("fp8"), 4, 2, moe.MOE_PATH_GEMM, moe.MOE_MODE_B)
    na = moe.moe_expert_ffn_workspace_size(w("fp8"), 4, 2, moe.MOE_PATH_GEMM, moe.MOE_MODE_A)
    assert nb >= na + 4 * 256 + 4 * 2 * 128  # quantised x and a with their scales


def test_quantize_validation(L):
    q = moe.moe_quantize_mx_e4m3
    _expect(moe.MOE_ERR_INVALID_ARG, q, FAKE, moe.MOE_F32, 4, 48, FAKE, FAKE, None, moe.MOE_F32, 0)   # K % 32
    _expect(moe.MOE_ERR_INVALID_ARG, q, FAKE, 7, 4, 64, FAKE, FAKE, None, moe.MOE_F32, 0)             # dtype
    _expect(moe.MOE_ERR_INVALID_ARG, q, FAKE, moe.MOE_BF16, 4, 64, None, None, FAKE, moe.MOE_BF16, 0)  # in place, bf16
    _expect(moe.MOE_ERR_INVALID_ARG, q, FAKE, moe.MOE_F32, 4, 64, None, None, None, moe.MOE_F32, 0)    # no output
    _expect(moe.MOE_ERR_INVALID_ARG, q, FAKE + 4, moe.MOE_F32, 4, 64, FAKE, None, None, moe.MOE_F32, 0)  # alignment


def test_combine_and_layer_validation(L):
    _expect(moe.MOE_ERR_UNSUPPORTED, moe.moe_combine, FAKE, FAKE, FAKE, 4, 2, 30, FAKE, moe.MOE_F32, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_combine, FAKE, FAKE, FAKE, 4, 2, 64, FAKE, 3, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_combine, FAKE, None, FAKE, 4, 2, 64, FAKE, moe.MOE_F32, 0)
    # two tiers: y_b and inv_b together, y_b 16-byte aligned
    ct = moe.moe_combine_tiers
    _expect(moe.MOE_ERR_INVALID_ARG, ct, FAKE, FAKE, FAKE, None, FAKE, 4, 2, 64, FAKE, moe.MOE_F32, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, ct, FAKE, FAKE, None, FAKE, FAKE, 4, 2, 64, FAKE, moe.MOE_F32, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, ct, FAKE, FAKE, FAKE + 4, FAKE, FAKE, 4, 2, 64, FAKE, moe.MOE_F32, 0)
    _expect(moe.MOE_ERR_UNSUPPORTED, ct, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 30, FAKE, moe.MOE_F32, 0)
    cfg = moe.routing(16, 2, "sigmoid")
    w = moe.weights("bf16", 16, 256, 128, FAKE, None, FAKE, None)
    big = moe.moe_layer_workspace_size(4, cfg, w, moe.MOE_PATH_AUTO, moe.MOE_MODE_A, 0)
    assert big > 4 * 2 * 256 * 4
    base = [FAKE, moe.MOE_BF16, 4, None, FAKE, None, cfg, None, w, moe.MOE_PATH_AUTO, moe.MOE_MODE_A, FAKE,
            moe.MOE_BF16, None, None, None, None, None, None, FAKE, big, 0]
    bad = list(base)
    bad[7] = FAKE                                                          # slot map without miss buffers
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_layer, *bad)
    bad = list(base)
    bad[-2] = 100
    _expect(moe.MOE_ERR_WORKSPACE, moe.moe_layer, *bad)
    bad = list(base)
    bad[13] = FAKE                                                         # topk_idx without topk_w
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_layer, *bad)
    bad = list(base)
    bad[8] = moe.weights("bf16", 8, 256, 128, FAKE, None, FAKE, None)      # S != E without a map
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_layer, *bad)


def test_plan_validation(L):
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_accumulate_counts, FAKE, 0, FAKE, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_accumulate_counts, FAKE, 1025, FAKE, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_accumulate_counts, FAKE, 8, FAKE + 4, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_accumulate_counts, None, 8, FAKE, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_plan_slots, FAKE, 8, 9, FAKE, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_plan_slots, FAKE, 8, 0, FAKE, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_plan_slots, FAKE, 2048, 8, FAKE, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_plan_slots, FAKE + 4, 8, 4, FAKE, 0)
    _expect(moe.MOE_ERR_INVALID_ARG, moe.moe_plan_slots, FAKE, 8, 4, None, 0)


def test_last_error_is_per_call(L):
    _expect(moe.MOE_ERR_UNSUPPORTED, moe.moe_combine, FAKE, FAKE, FAKE, 4, 2, 30, FAKE, moe.MOE_F32, 0)
    assert "H = 30" in moe.lib().moe_last_error().decode()


def test_auto_path_crossovers(L):
    """AUTO's choice between the GEMV and the matrix cores (host logic, no device work): GEMM once
    T*k exceeds c*S with c = 2.75 (bf16), 2 (FP8), 0.5 (MXFP4), where the measured crossovers lie;
    an explicit path passes through; invalid arguments give -1."""
    def w(dt, S, H=4096, I=1024):
        return moe.weights(dt, S, H, I, FAKE, FAKE, FAKE, FAKE)
    A, GEMV, GEMM = moe.MOE_PATH_AUTO, moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM
    rp = lambda wd, T, k=8, path=A, mode=moe.MOE_MODE_A: moe.moe_resolve_path(wd, T, k, path, mode)
    bf, f8, f4 = w("bf16", 384), w("fp8", 384), w("mxfp4", 110)
    # the stated workloads keep their paths: decode on the GEMV, prefill on the matrix cores
    assert rp(bf, 4) == GEMV and rp(f8, 32) == GEMV and rp(f4, 1) == GEMV
    assert rp(f8, 4096) == GEMM and rp(f4, 4096) == GEMM
    # thresholds: bf16 T*k > 1056, FP8 > 768, MXFP4 (S = 110) > 55
    assert rp(bf, 132) == GEMV and rp(bf, 133) == GEMM
    assert rp(f8, 96) == GEMV and rp(f8, 97) == GEMM
    assert rp(f4, 6) == GEMV and rp(f4, 7) == GEMM
    # an explicit path is returned as is; fp32 weights never take the matrix cores
    assert rp(f8, 4096, path=GEMV) == GEMV and rp(bf, 1, path=GEMM) == GEMM
    assert rp(w("f32", 8, 256, 128), 4096) == GEMV
    # mode B needs FP8 / MXFP4 weights on the matrix-core path: bf16 stays on the GEMV
    assert rp(bf, 4096, mode=moe.MOE_MODE_B) == GEMV and rp(f8, 4096, mode=moe.MOE_MODE_B) == GEMM
    assert rp(w("fp8", 384, H=4100), 4) == -1 and rp(f8, 4, path=9) == -1 and rp(f8, 4, k=0) == -1


def test_invariant_path_and_tile_order_flag(L):
    """INVARIANT resolves by the weights and mode alone -- the matrix cores wherever they take the
    shape, else the GEMV -- so its choice never depends on T; the tile-order flag is accepted on
    every path and leaves the choice alone; other flag bits are rejected."""
    def w(dt, S, H=4096, I=1024):
        return moe.weights(dt, S, H, I, FAKE, FAKE, FAKE, FAKE)
    INV, GEMV, GEMM = moe.MOE_PATH_INVARIANT, moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM
    C = moe.MOE_PATH_TILES_CONTIGUOUS
    rp = lambda wd, T, path, mode=moe.MOE_MODE_A: moe.moe_resolve_path(wd, T, 8, path, mode)
    for wd in (w("bf16", 384), w("fp8", 384), w("mxfp4", 110)):
        assert {rp(wd, T, INV) for T in (1, 4, 32, 4096)} == {GEMM}
        assert rp(wd, 1, GEMV | C) == GEMV and rp(wd, 1, GEMM | C) == GEMM and rp(wd, 4096, moe.MOE_PATH_AUTO | C) == GEMM
    # shapes the matrix cores do not take stay on the GEMV for every T
    for wd in (w("f32", 8, 256, 128), w("fp8", 384, H=4096, I=1056), w("bf16", 384, H=4096, I=1000)):
        assert {rp(wd, T, INV) for T in (1, 4096)} == {GEMV}
    assert rp(w("bf16", 384), 4096, INV, mode=moe.MOE_MODE_B) == GEMV
    assert rp(w("fp8", 384), 1, INV, mode=moe.MOE_MODE_B) == GEMM
    assert rp(w("fp8", 384), 4, 0x200 | GEMM) == -1 and rp(w("fp8", 384), 4, C | 7) == -1


def test_ffn_workspace_layout(L):
    """Where the intermediate a lives in the expert-FFN workspace (host logic only): its format by
    path and mode, 256-byte aligned offsets whose regions fit in the workspace size."""
    def w(dt, S, H=4096, I=1024):
        return moe.weights(dt, S, H, I, FAKE, FAKE, FAKE, FAKE)
    A, B = moe.MOE_MODE_A, moe.MOE_MODE_B
    T, k = 4096, 8
    R = T * k
    for wd, path, mode, fmt in ((w("fp8", 384), moe.MOE_PATH_GEMM, A, 1), (w("fp8", 384), moe.MOE_PATH_GEMM, B, 3),
                                (w("fp8", 384), moe.MOE_PATH_GEMV, A, 0), (w("fp8", 384), moe.MOE_PATH_GEMV, B, 0),
                                (w("bf16", 8, 8192, 8192), moe.MOE_PATH_GEMM, A, 2),
                                (w("fp8", 8, 8192, 4096), moe.MOE_PATH_GEMM, A, 2),
                                (w("fp8", 8, 4096, 8192), moe.MOE_PATH_GEMM, A, 2),
                                (w("fp8", 8, 8192, 2048), moe.MOE_PATH_GEMM, A, 1),
                                (w("mxfp4", 110), moe.MOE_PATH_AUTO, B, 3)):
        off_a, off_q, off_s, f = moe.moe_expert_ffn_workspace_layout(wd, T, k, path, mode)
        size = moe.moe_expert_ffn_workspace_size(wd, T, k, path, mode)
        I = wd.I
        assert f == fmt, (wd.wdtype, path, mode, f)
        if f == 3:
            assert off_a is None and off_q % 256 == 0 and off_s % 256 == 0
            assert off_q + R * I <= off_s and off_s + R * I // 32 <= size
        else:
            assert off_q is None and off_s is None and off_a % 256 == 0
            assert off_a + R * I * (4 if f in (0, 2) else 2) <= size
    with pytest.raises(moe.MoeError):
        moe.moe_expert_ffn_workspace_layout(w("fp8", 384), T, k, 9, A)


def test_static_layer_rejects_oversize_calls(L):
    """moe_layer_static checks the call's workspace need against its static workspace on the host,
    before any HIP call: a 4096-token batch is refused with a message naming both sizes."""
    w = moe.weights("fp8", 384, 4096, 1024, FAKE, FAKE, FAKE, FAKE)
    cfg = moe.routing(384, 8, "sigmoid", True)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_static(FAKE, moe.MOE_BF16, 4096, None, FAKE, None, cfg, None, w, moe.MOE_PATH_AUTO,
                             moe.MOE_MODE_A, FAKE, moe.MOE_BF16, FAKE, FAKE, None, None, None, None, 0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED and "static" in str(ei.value)
    need = moe.moe_layer_workspace_size(192, cfg, w, moe.MOE_PATH_AUTO, moe.MOE_MODE_A, 0)
    assert need <= moe.MOE_STATIC_WORKSPACE_BYTES < moe.moe_layer_workspace_size(200, cfg, w, moe.MOE_PATH_AUTO,
                                                                                 moe.MOE_MODE_A, 0)


def test_layer_decode_fused_rule(L):
    """Which batches moe_layer runs as the two-launch decode layer."""
    bf = moe.MOE_BF16
    cfg = moe.routing(384, 8, "sigmoid")

    def fused(T, k=8, I=1024, wd=moe.MOE_BF16, path=moe.MOE_PATH_GEMV, mode=moe.MOE_MODE_A, xdt=bf, E=384):
        c = moe.routing(E, k, "sigmoid")
        w = moe.weights(wd, E, 4096, I, FAKE, FAKE, FAKE, FAKE)
        return moe.moe_layer_decode_fused(T, c, w, path, mode, xdt)
    mx = moe.MOE_MXFP4
    assert fused(1) and fused(2, k=4) and not fused(2)  # bf16: up to 8 rows
    assert fused(2, wd=mx) and fused(4, wd=mx)          # MXFP4: up to 32 rows
    assert not fused(4, k=16, wd=mx)                    # 64 rows: the staged launches
    assert not fused(5, k=2)                            # a fifth token
    assert not fused(1, k=64, I=512, wd=mx)             # 64 rows
    assert fused(1, k=16, I=512, wd=mx)
    assert not fused(2, I=8192, wd=mx)                  # the rows of a beyond the LDS budget
    assert not fused(0)
    assert not fused(1, wd=moe.MOE_FP8_E4M3_B128, mode=moe.MOE_MODE_B)      # mode B stays staged
    assert not fused(1, wd=moe.MOE_FP8_E4M3_B128, path=moe.MOE_PATH_GEMM)   # the matrix-core path
    assert fused(1, wd=moe.MOE_FP8_E4M3_B128, path=moe.MOE_PATH_AUTO)        # AUTO picks the GEMV here
    assert fused(1, xdt=moe.MOE_F32)
    _expect(moe.MOE_ERR_INVALID_ARG, fused, 1, xdt=7)


def test_decode_calls_validation(L):
    """The two decode launches reject shapes outside the two-launch layer and missing buffers
    before any HIP call."""
    bf, inv, uns = moe.MOE_BF16, moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED
    cfg = moe.routing(384, 8, "sigmoid")
    w = moe.weights(moe.MOE_BF16, 384, 4096, 1024, FAKE, FAKE, FAKE, FAKE)
    wc = moe.weights(moe.MOE_MXFP4, 110, 4096, 1024, FAKE, FAKE, FAKE, FAKE)

    def gu(T=1, x=FAKE, logits=FAKE, slot_map=None, w=w, miss=FAKE, err=FAKE, a=FAKE):
        moe.moe_decode_gate_up(x, bf, T, logits, None, cfg, slot_map, w, FAKE, FAKE, FAKE, a, FAKE, miss, miss, miss,
                               err, 0)
    _expect(uns, gu, T=3)                       # 24 rows
    _expect(inv, gu, logits=None)
    _expect(inv, gu, err=None)
    _expect(inv, gu, a=FAKE + 4)                # a must be 16-byte aligned
    _expect(inv, gu, w=wc)                      # S < E without a slot map
    _expect(inv, gu, w=wc, slot_map=FAKE, miss=None)
    _expect(uns, moe.moe_decode_down_combine, w, 3, cfg, FAKE, FAKE, FAKE, FAKE, bf, 0)
    _expect(inv, moe.moe_decode_down_combine, w, 1, cfg, None, FAKE, FAKE, FAKE, bf, 0)
    _expect(inv, moe.moe_decode_down_combine, w, 1, cfg, FAKE, FAKE, FAKE, FAKE, 9, 0)
    # moe_route computes logits alone only with router weights and logits_out
    _expect(inv, moe.moe_route, FAKE, bf, 1, 4096, FAKE, None, None, cfg, None, None, None, FAKE, 1 << 20, 0)
    _expect(inv, moe.moe_route, None, bf, 1, 4096, None, FAKE, None, cfg, None, None, FAKE, None, 0, 0)

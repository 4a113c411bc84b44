"""Pins for the oracle's number-format decoding and its mode-B activation quantiser.

Each check compares against something other than the oracle itself: torch's own CPU
conversions of the same codes (library routines), spot values printed in the OCP format
specifications (tests/golden), or hand-built byte layouts with a known answer."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    num = ~np.isnan(a)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[num], b[num]) and \
        np.array_equal(np.signbit(a[num]), np.signbit(b[num]))


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(O.e4m3fn_to_f64(codes), ref)


def test_e4m3fn_spec_spot_values():
    for c, v in _read_golden("e4m3fn_ocp_spot.txt"):
        got = float(O.e4m3fn_to_f64(np.uint8(c)))
        if math.isnan(v):
            assert math.isnan(got), hex(c)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), hex(c)


def test_e8m0_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert _same(O.e8m0_to_f64(codes), ref)


def test_e2m1_matches_spec_table():
    for c, v in _read_golden("e2m1_ocp.txt"):
        got = float(O.e2m1_to_f64(np.uint8(c)))
        assert got == v and math.copysign(1, got) == math.copysign(1, v), hex(c)


def test_e2m1_is_e4m3_with_rebased_exponent():
    # e2m1 code s.EE.M has the value of the e4m3fn code s.(EE+6).M00 for EE>0, and of
    # s.0110.000 times M for EE=0 (0.5 = 2^-1); torch decodes the e4m3 side.
    for c in range(16):
        s, ee, m = c >> 3, (c >> 1) & 3, c & 1
        if ee == 0:
            e4 = (s << 7) | (6 << 3)
            ref = torch.tensor([e4], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item() * m
        else:
            e4 = (s << 7) | ((ee + 6) << 3) | (m << 2)
            ref = torch.tensor([e4], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        assert float(O.e2m1_to_f64(np.uint8(c))) == ref, c


def test_bf16_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, 4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(O.bf16_to_f64(bits), ref)


def test_fp8_block_scale_indexing():
    # every code is 1.0 (0x38); the block at (nb, kb) has scale 2^(3*nb + kb): a transposed or
    # mis-strided scale lookup changes the result.
    N, K = 256, 384
    w = np.full((N, K), 0x38, np.uint8)
    s = np.array([[2.0 ** (3 * nb + kb) for kb in range(3)] for nb in range(2)], np.float32)
    d = O.dequant("fp8", w, s, N, K)
    for n in (0, 127, 128, 255):
        for k in (0, 127, 128, 255, 256, 383):
            assert d[n, k] == 2.0 ** (3 * (n // 128) + k // 128)


def test_mxfp4_nibble_order_and_scales():
    # one row, 64 elements: byte j = (hi << 4) | lo with lo -> k = 2j, hi -> k = 2j + 1.
    K = 64
    codes = np.array([(j % 8) for j in range(K)], np.uint8)       # 0,1,..,7,0,1,..
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[127 + 1, 127 - 2]], np.uint8)               # x2 for k<32, x1/4 for k>=32
    d = O.dequant("mxfp4", packed, scales, 1, K)[0]
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for k in range(K):
        assert d[k] == grid[k % 8] * (2.0 if k < 32 else 0.25), k


def test_e4m3fn_round_matches_torch_cast():
    # torch's float -> float8_e4m3fn conversion rounds to nearest even; it does not saturate,
    # so compare inside +-448 and check saturation separately.
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(20000) * 40,
        rng.standard_normal(5000) * 0.01,                    # subnormal range
        np.arange(-448, 449, 0.5),                           # many exact ties
        np.ldexp(np.arange(1, 64) + 0.5, -12),               # subnormal ties
    ])
    v32 = v.astype(np.float32).astype(np.float64)
    v32 = v32[np.abs(v32) <= 448]
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.e4m3fn_round(v32), ref)
    assert O.e4m3fn_round(np.array([500.0, -1e6]))[0] == 448.0
    assert O.e4m3fn_round(np.array([-1e6]))[0] == -448.0


def test_act_quant_block_rule():
    # block amax 1.0 -> X = -8: 1.0 -> 256 (exact), 1/1024 -> 0.25 (exact), 3/1000 rounds.
    a = np.zeros((1, 64))
    a[0, 0] = 1.0
    a[0, 1] = 1.0 / 1024
    a[0, 2] = 0.003
    a[0, 32] = 500.0                                   # second block: amax 500 -> X = 0
    a[0, 33] = 449.0
    q = O.act_quant_mx_e4m3(a)
    assert q[0, 0] == 1.0 and q[0, 1] == 1.0 / 1024
    ref = torch.tensor([0.003 * 256], dtype=torch.float32).to(torch.float8_e4m3fn).double().item() / 256
    assert q[0, 2] == ref
    assert q[0, 32] == 448.0 and q[0, 33] == 448.0     # saturated, not NaN
    assert np.all(q[0, 3:32] == 0) and np.all(q[0, 34:] == 0)


def test_act_quant_e8m0_lower_clamp():
    # OCP MX v1.0: the E8M0 scale encodes 2^-127 .. 2^127, so X never drops below -127.  A block
    # with amax = 2^-121 would want X = -129; clamped it takes X = -127 (scale byte 0), and its
    # elements are coded against 2^-127: 2^-121 -> 2^6, 3 * 2^-126 -> 6, 5 * 2^-136 -> 5 * 2^-9
    # (an exact e4m3 subnormal), and 2^-140 -> 2^-13, below half the smallest e4m3 subnormal
    # (2^-9), so 0.  A block with amax = 2^-118 needs no clamp (X = -126).
    a = np.zeros((1, 96))
    a[0, 0] = 2.0 ** -121
    a[0, 1] = 3.0 * 2.0 ** -126
    a[0, 2] = 2.0 ** -140
    a[0, 3] = 5.0 * 2.0 ** -136
    a[0, 32] = 2.0 ** -118                              # X = -126: inside the range
    a[0, 64] = 1.5 * 2.0 ** -119                        # X = floor(-118.4) - 8 = -127 exactly
    X, q = O.act_quant_mx_e4m3_parts(a)
    assert X.tolist() == [[-127, -126, -127]]
    assert q[0, 0] == 64.0 and q[0, 1] == 6.0 and q[0, 2] == 0.0 and q[0, 3] == 5.0 * 2.0 ** -9
    assert q[0, 32] == 256.0 and q[0, 64] == 384.0
    deq = O.act_quant_mx_e4m3(a)
    assert deq[0, 0] == a[0, 0] and deq[0, 1] == a[0, 1] and deq[0, 2] == 0.0 and deq[0, 3] == a[0, 3]
    # a subnormal-range element that the clamp does change: 2^-138 -> 2^-11 against 2^-127 (rounds
    # to 0); against 2^-129 it would be 2^-9, the smallest e4m3 subnormal
    b = np.zeros((1, 32))
    b[0, 0] = 2.0 ** -121
    b[0, 1] = 2.0 ** -138
    assert O.act_quant_mx_e4m3(b)[0, 1] == 0.0


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp4"])
def test_generator_encoders_roundtrip(wdtype):
    # the generator's encoders (input production) decoded by the oracle stay close to the
    # fp32 draws: relative RMS error within each format's resolution.
    from synth import gen
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    cfg = gen.config("tiny", wdtype=wdtype)
    stored, scale = gen._store(cfg, w)
    d = O.dequant(wdtype, stored, scale, 256, 256)
    rel = np.sqrt(np.mean((d - w) ** 2) / np.mean(w.astype(np.float64) ** 2))
    assert rel < {"bf16": 3e-3, "fp8": 4e-2, "mxfp4": 0.2}[wdtype]

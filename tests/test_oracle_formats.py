"""Pins of the oracle's number formats (FP8 E4M3FN, BF16, FP4 E2M1, MXFP4) against
library routines and the formats' bit-field definitions, plus the pages' "FP4 to FP8 is
lossless" property ("DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 3.4)."""
import math

import numpy as np
import pytest
import torch


def minifloat_value(code: int, ebits: int, mbits: int, bias: int) -> float:
    """Generic sign/exponent/mantissa decoder (subnormal when the exponent field is 0)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    f = code & ((1 << mbits) - 1)
    if e == 0:
        v = f / (1 << mbits) * 2.0 ** (1 - bias)
    else:
        v = (1 + f / (1 << mbits)) * 2.0 ** (e - bias)
    return -v if s else v


def test_generic_decoder_matches_torch_e4m3():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        if c & 0x7F == 0x7F:
            assert math.isnan(ref[c])
            continue
        assert minifloat_value(c, 4, 3, 7) == ref[c]


def test_e4m3_decode_all_codes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = orc.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == ref[c], c


def _finite_e4m3_values():
    vals = sorted({minifloat_value(c, 4, 3, 7) for c in range(128) if c != 0x7F})
    return np.array(vals, np.float64)


def test_e4m3_encode_roundtrip_and_midpoints(orc):
    vals = _finite_e4m3_values()
    # every code round-trips
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        v = orc.e4m3_decode(c)
        got = orc.e4m3_encode(v)
        assert orc.e4m3_decode(got) == v
    # midpoints between neighbours round to the even code, checked against torch (RNE)
    mids = (vals[:-1] + vals[1:]) / 2
    xs = np.concatenate([mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)]).astype(np.float32)
    xs = xs[np.abs(xs) < 448]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in xs], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_random_vs_torch(orc):
    g = np.random.default_rng(1)
    xs = (g.standard_normal(20000) * np.exp2(g.integers(-14, 9, 20000))).astype(np.float32)
    xs = xs[np.abs(xs) < 448]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in xs], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_saturates(orc):
    for x in (448.0, 449.0, 463.9, 464.0, 1e6, 3.0e38):
        assert orc.e4m3_encode(x) == 0x7E
        assert orc.e4m3_encode(-x) == 0xFE


def test_bf16_encode_vs_torch(orc):
    g = np.random.default_rng(2)
    xs = (g.standard_normal(5000) * np.exp2(g.integers(-30, 30, 5000))).astype(np.float32)
    # exact midpoints between bf16 neighbours
    b = xs.view(np.uint32) & np.uint32(0xFFFF0000)
    mids = (b | np.uint32(0x8000)).view(np.float32)
    xs = np.concatenate([xs, mids])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_encode(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, ref)


def test_e2m1_decode_from_bitfields(orc):
    for c in range(16):
        assert orc.e2m1_decode(c) == minifloat_value(c, 2, 1, 1)


def test_e2m1_encode_nearest_even(orc):
    mags = [minifloat_value(c, 2, 1, 1) for c in range(8)]
    for c in range(16):
        assert orc.e2m1_encode(orc.e2m1_decode(c)) == c
    for c in range(7):
        mid = (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert orc.e2m1_encode(mid) == even
        assert orc.e2m1_encode(-mid) == 8 | even
        assert orc.e2m1_encode(np.nextafter(mid, 0)) == c
        assert orc.e2m1_encode(np.nextafter(mid, 10)) == c + 1
    for x in (6.0, 6.5, 7.0, 100.0):
        assert orc.e2m1_encode(x) == 7
        assert orc.e2m1_encode(-x) == 15


def test_mxfp4_scale_rule(orc):
    # X = floor(log2(amax)) - 2, clamped; amax = 0 -> X = -127 with zero codes
    cases = {6.0: 0, 1.0: -2, 7.9: 0, 8.0: 1, 0.75: -3, 1e-3: -12, 0.0: -127}
    for amax, X in cases.items():
        x = np.zeros((1, 32), np.float32)
        x[0, 5] = amax
        x[0, 6] = -amax / 3
        codes, scales = orc.quant_mxfp4(x)
        assert int(scales[0, 0]) - 127 == X, amax
        if amax == 0.0:
            assert not codes.any()
    # 7.9 saturates to 6 at X = 0
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 7.9
    codes, scales = orc.quant_mxfp4(x)
    assert codes[0, 0] & 15 == 7


def test_mxfp4_roundtrip_and_nibble_order(orc):
    g = np.random.default_rng(3)
    X = g.integers(-20, 20, size=(64, 4))
    c = g.integers(0, 16, size=(64, 128))
    vals = np.vectorize(lambda v: minifloat_value(int(v), 2, 1, 1))(c)
    x = (vals * np.exp2(np.repeat(X, 32, axis=1))).astype(np.float32)
    # force each block's amax to sit in [4, 8) * 2^X so the scale is exactly X
    x[:, ::32] = (6.0 * np.exp2(X)).astype(np.float32)
    codes, scales = orc.quant_mxfp4(x)
    assert np.array_equal(scales.astype(int) - 127, X)
    back = orc.dequant_mxfp4(codes, scales)
    assert np.array_equal(back, x.astype(np.float64))
    # element 2j sits in the low nibble of byte j
    lo = codes & 15
    hi = codes >> 4
    v_lo = np.vectorize(lambda v: minifloat_value(int(v), 2, 1, 1))(lo) * np.exp2(np.repeat(X, 16, axis=1))
    v_hi = np.vectorize(lambda v: minifloat_value(int(v), 2, 1, 1))(hi) * np.exp2(np.repeat(X, 16, axis=1))
    assert np.array_equal(v_lo, x[:, 0::2]) and np.array_equal(v_hi, x[:, 1::2])


def test_quant_kv_record(orc):
    g = np.random.default_rng(4)
    x = g.standard_normal((50, 128)).astype(np.float32)
    x[3, :96] = 0.0
    nope, rope, scale = orc.quant_kv(x, 32)
    assert nope.shape == (50, 96) and rope.shape == (50, 32) and scale.shape == (50,)
    amax = np.abs(x[:, :96]).max(1)
    nz = amax > 0
    assert np.array_equal(scale[nz], (amax[nz] / np.float32(448.0)).astype(np.float32))
    assert scale[3] == 1.0 and not nope[3].any()
    inv = (np.float32(448.0) / amax[nz]).astype(np.float32)
    prod = (x[nz, :96] * inv[:, None]).astype(np.float32)
    ref = torch.from_numpy(np.ascontiguousarray(prod)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nope[nz], ref)
    # the row's largest element maps to +-448 exactly
    assert set(np.unique(np.abs(orc.dequant_kv(nope, rope, scale)[nz, :96]).max(1) /
                         scale[nz].astype(np.float64)).tolist()) == {448.0}
    ref_rope = torch.from_numpy(x[:, 96:].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rope, ref_rope)


def test_dequant_kv_layout(orc):
    """dequant_kv puts dims 0..D-R-1 back as FP8 code x scale and dims D-R..D-1 as the BF16
    values of x, each in its own position (the record layout: non-RoPE dims first, RoPE dims
    last).  Both halves are checked against torch's own conversions, so a swapped or shifted
    half fails."""
    g = np.random.default_rng(5)
    for D, R in ((128, 32), (512, 64)):
        x = g.standard_normal((40, D)).astype(np.float32)
        x[7, :D - R] = 0.0
        nope, rope, scale = orc.quant_kv(x, R)
        back = orc.dequant_kv(nope, rope, scale)
        assert back.shape == (40, D)
        bf = torch.from_numpy(np.ascontiguousarray(x[:, D - R:])).to(torch.bfloat16).double().numpy()
        assert np.array_equal(back[:, D - R:], bf)
        fp8 = torch.from_numpy(np.ascontiguousarray(nope)).view(torch.float8_e4m3fn).double().numpy()
        assert np.array_equal(back[:, :D - R], fp8 * scale.astype(np.float64)[:, None])
        # the non-RoPE half approximates x (FP8 keeps 3 mantissa bits), the RoPE half is not x's
        # non-RoPE part: a swap would break one of these
        assert np.abs(back[:, :D - R] - x[:, :D - R]).max() <= np.abs(x[:, :D - R]).max() * 2.0 ** -3
        assert not back[7, :D - R].any() and scale[7] == 1.0


def test_fp4_to_fp8_lossless(orc):
    """Every E2M1 value times 2^k that lies in E4M3's normal range survives an E4M3 round
    trip: E4M3 has two more exponent bits and two more mantissa bits than E2M1, so only the
    scale range limits the claim."""
    checked = 0
    for c in range(16):
        v = orc.e2m1_decode(c)
        for k in range(-20, 20):
            x = v * 2.0 ** k
            if x != 0 and not (2.0 ** -6 <= abs(x) <= 448.0):
                continue
            assert orc.e4m3_decode(orc.e4m3_encode(x)) == x
            checked += 1
    assert checked > 100
    # below the normal range the claim needs the scale condition: 1.5 * 2^-9 falls between
    # two points of E4M3's subnormal grid (step 2^-9)
    assert orc.e4m3_decode(orc.e4m3_encode(1.5 * 2.0 ** -9)) != 1.5 * 2.0 ** -9

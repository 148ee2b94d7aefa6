"""Pins of the oracle's number formats against library routines and round trips (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from synth import gen as G



def generic_minifloat(code: int, ebits: int, mbits: int, bias: int, ieee_specials: bool,
                      fn_nan: bool) -> float:
    """Test-side generic minifloat decoder, checked below against library tables."""
    s = -1.0 if (code >> (ebits + mbits)) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    mant = code & ((1 << mbits) - 1)
    emax = (1 << ebits) - 1
    if ieee_specials and e == emax:
        return s * math.inf if mant == 0 else math.nan
    if fn_nan and e == emax and mant == (1 << mbits) - 1:
        return math.nan
    if e == 0:
        return s * (mant / (1 << mbits)) * 2.0 ** (1 - bias)
    return s * (1.0 + mant / (1 << mbits)) * 2.0 ** (e - bias)


def _same(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


def test_generic_decoder_matches_library_tables():
    codes8 = torch.arange(256, dtype=torch.uint8)
    e4m3 = codes8.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    e5m2 = codes8.view(torch.float8_e5m2).to(torch.float64).numpy()
    assert _same([generic_minifloat(c, 4, 3, 7, False, True) for c in range(256)], e4m3)
    assert _same([generic_minifloat(c, 5, 2, 15, True, False) for c in range(256)], e5m2)
    codes16 = np.arange(65536, dtype=np.uint16)
    f16 = codes16.view(np.float16).astype(np.float64)
    assert _same([generic_minifloat(int(c), 5, 10, 15, True, False) for c in codes16[::97]], f16[::97])


def test_e4m3_table_is_the_library_table():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(F.E4M3_TABLE, lib)
    assert F.E4M3_TABLE[0x7E] == 448.0 and np.isnan(F.E4M3_TABLE[0x7F])


def test_e2m1_table_is_the_generic_minifloat():
    ref = [generic_minifloat(c, 2, 1, 1, False, False) for c in range(16)]
    assert _same(F.E2M1_TABLE, ref)
    assert sorted(set(np.abs(F.E2M1_TABLE))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(F.decode_bf16(bits), lib)


def test_ue8m0_decode():
    assert F.decode_ue8m0(127) == 1.0
    assert F.decode_ue8m0(130) == 8.0
    assert F.decode_ue8m0(0) == 2.0 ** -127
    assert np.isnan(F.decode_ue8m0(255))


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(5000).astype(np.float32)])
    x32 = x.astype(np.float32)
    # exact ties: bf16 value plus half an ulp
    b = torch.from_numpy(x32[:2000]).to(torch.bfloat16).to(torch.float32).numpy()
    half = np.abs(b) * 2.0 ** -8
    ties = (b + half).astype(np.float32)
    x32 = np.concatenate([x32, ties, -ties])
    lib = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.round_bf16(x32.astype(np.float64)), lib)


def test_round_e4m3_matches_torch_cast():
    rng = np.random.default_rng(2)
    x = rng.uniform(-448, 448, 20000)
    x = np.concatenate([x, rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000)])
    x = np.clip(x, -448, 448).astype(np.float32)
    # exact midpoints between neighbouring codes, incl. subnormals
    vals = F.E4M3_TABLE[:0x7E]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.round_e4m3(x.astype(np.float64))
    # +0 and -0 both decode to 0
    assert np.array_equal(F.decode_e4m3(ours), F.decode_e4m3(lib))
    assert np.array_equal(ours[x != 0], lib[x != 0])


def test_ue8m0_exponent_is_smallest_fitting_power():
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(5000)) * 2.0 ** rng.integers(-40, 40, 5000)
    amax = np.concatenate([amax, 448.0 * 2.0 ** np.arange(-20, 20.0)])
    for qmax in (448.0, 6.0):
        e = F.ue8m0_exponent(amax, qmax)
        assert np.all(amax <= qmax * np.ldexp(1.0, e))
        assert np.all(amax > qmax * np.ldexp(1.0, e - 1))
    assert F.ue8m0_exponent(0.0, 448.0) == 0


def _e4m3_half_ulp(scaled):
    """Half the e4m3 spacing at |v| (spacing 2**(floor(log2|v|) - 3), never below 2**-9)."""
    _, e = np.frexp(np.maximum(scaled, 2.0 ** -6))
    return np.ldexp(1.0, e - 1 - 3 - 1)


def test_quantize_fp8ds_round_trip_half_ulp():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 512)) / math.sqrt(512)).astype(np.float32)
    x[3, :64] = 0.0
    codes, rope, scales = F.quantize_fp8ds(x)
    y = F.decode_fp8ds(codes, rope, scales)
    lat, ylat = x[:, :448].astype(np.float64), y[:, :448]
    sc = F.decode_ue8m0(scales)
    # e4m3 spacing at |v| is 2**(floor(log2|v|) - 3) (>= 2**-9 in scaled units)
    scaled = np.abs(lat).reshape(64, 7, 64) / sc[..., None]
    half_ulp = _e4m3_half_ulp(scaled) * sc[..., None]
    assert np.all(np.abs(ylat - lat).reshape(64, 7, 64) <= half_ulp)
    assert np.array_equal(rope, torch.from_numpy(x[:, 448:]).to(torch.bfloat16).view(torch.int16).numpy()
                          .view(np.uint16))
    assert np.all(scales[3, 0] == 127)


def test_generator_fp8ds_records_decode_within_half_ulp():
    x = torch.randn(200, 512) / math.sqrt(512)
    rec = G.make_fp8ds(x)
    y = F.decode_fp8ds(rec.codes.numpy(), rec.rope.view(torch.int16).numpy().view(np.uint16),
                       rec.scales.numpy())
    lat = x[:, :448].double().numpy().reshape(200, 7, 64)
    sc = F.decode_ue8m0(rec.scales.numpy())
    assert np.all(np.abs(lat).max(-1) <= 448 * sc)
    half_ulp = _e4m3_half_ulp(np.abs(lat) / sc[..., None]) * sc[..., None]
    assert np.all(np.abs(y[:, :448].reshape(200, 7, 64) - lat) <= half_ulp)


def test_generator_mxfp4_rows_decode_to_nearest():
    x = torch.randn(300, 128)
    rec = G.make_mxfp4(x)
    y = F.decode_mxfp4(rec.codes.numpy(), rec.scales.numpy())
    sc = F.decode_ue8m0(rec.scales.numpy())                     # [300, 4]
    xs = x.double().numpy().reshape(300, 4, 32) / sc[..., None]
    ys = y.reshape(300, 4, 32) / sc[..., None]
    assert np.all(np.abs(xs) <= 6.0)
    grid = np.array(sorted(set(F.E2M1_TABLE)))
    nearest_err = np.abs(xs[..., None] - grid).min(-1)
    assert np.allclose(np.abs(ys - xs), nearest_err)
    # element order inside a byte: element 2j in the low nibble
    assert F.decode_mxfp4(np.array([[0x21] + [0] * 15]), np.array([127]))[0, :2].tolist() == [0.5, 1.0]


def test_e2m1_rounding_round_trips_and_ties_to_even():
    # every magnitude code decodes and rounds back to itself, with either sign
    for c in range(16):
        v = F.decode_e2m1(np.array([c]))[0]
        if c == 8:
            continue                                     # -0 decodes to 0, which rounds to +0
        assert F.round_e2m1(np.array([v]))[0] == c
    # halfway points between neighbouring magnitudes go to the even code (OCP MX: RNE)
    halfway = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in halfway.items():
        assert F.round_e2m1(np.array([v]))[0] == c
        assert F.round_e2m1(np.array([-v]))[0] == c | 8
    # just off a halfway point: the nearer neighbour
    mags = F.E2M1_TABLE[:8]
    for k in range(7):
        mid = (mags[k] + mags[k + 1]) / 2
        assert F.round_e2m1(np.array([mid - 1e-9]))[0] == k
        assert F.round_e2m1(np.array([mid + 1e-9]))[0] == k + 1


def test_mxfp4_quantizer_scale_rule_and_error_bound():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-6, 6, (40, 1)))).astype(np.float32)
    x[3, :32] = 0.0                                      # an all-zero block: scale byte 127
    packed, sc = F.quantize_mxfp4(x)
    assert packed.shape == (40, 64) and sc.shape == (40, 4)
    assert np.all(sc[3, 0] == 127)
    blk = np.abs(x.astype(np.float64)).reshape(40, 4, 32).max(axis=-1)
    e = sc.astype(np.int64) - 127
    # brute force: the smallest power of two with amax <= 6 * 2**e
    for i in range(40):
        for j in range(4):
            if blk[i, j] == 0:
                continue
            best = min(k for k in range(-140, 140) if blk[i, j] <= 6.0 * 2.0 ** k)
            assert e[i, j] == best
    dec = F.decode_mxfp4(packed, sc)
    # within half the e2m1 spacing at the value's place (spacing 0.5 below 2, 1 up to 4, 2 above)
    y = np.abs(x.astype(np.float64)) / np.repeat(np.ldexp(1.0, e), 32, axis=1)
    half_step = np.where(y < 2.0, 0.25, np.where(y < 4.0, 0.5, 1.0)) * np.repeat(np.ldexp(1.0, e), 32, axis=1)
    assert np.all(np.abs(dec - x) <= half_step * (1 + 1e-12))
    # element 2j is the low nibble of byte j
    one = np.zeros((1, 32), dtype=np.float32)
    one[0, 0], one[0, 1] = 6.0, 1.0
    p1, s1 = F.quantize_mxfp4(one)
    assert p1[0, 0] == (0x7 | (0x2 << 4)) and s1[0, 0] == 127


def test_fp8ix_quantizer_round_trip():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((30, 128)) * np.exp(rng.uniform(-8, 8, (30, 1)))).astype(np.float32)
    codes, scale = F.quantize_fp8ix(x)
    assert codes.shape == (30, 128) and scale.shape == (30,) and scale.dtype == np.float32
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    # the scale is the smallest power of two with amax <= 448 * scale
    assert np.all(amax <= 448.0 * scale) and np.all(amax > 224.0 * scale)
    dec = F.decode_fp8ix(codes, scale)
    rel = np.abs(dec - x) / np.maximum(np.abs(x), 2.0 ** -6 * scale[:, None])
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-12)          # e4m3 keeps 4 significant bits
    # exactly representable rows come back unchanged
    reps = F.decode_e4m3(rng.integers(0, 126, (4, 128))) * 2.0 ** 5
    c2, s2 = F.quantize_fp8ix(reps.astype(np.float32))
    assert np.array_equal(F.decode_fp8ix(c2, s2), reps)


def test_mxfp8_record_round_trip_and_scale_rule():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((20, 512)) * np.exp(rng.uniform(-5, 5, (20, 16))).repeat(32, axis=1)).astype(np.float32)
    codes, sc = F.quantize_mxfp8(x)
    assert codes.shape == (20, 512) and sc.shape == (20, 16)
    blk = np.abs(x.astype(np.float64)).reshape(20, 16, 32).max(axis=-1)
    s = np.ldexp(1.0, sc.astype(np.int64) - 127)
    assert np.all(blk <= 448.0 * s) and np.all(blk > 224.0 * s)      # smallest power of two
    dec = F.decode_mxfp8(codes, sc)
    tiny = np.repeat(s, 32, axis=1) * 2.0 ** -9                      # e4m3 subnormal step
    assert np.all(np.abs(dec - x) <= np.abs(x) * 2.0 ** -4 + tiny / 2)
    # a row of representable values comes back exactly; the block of dim c is c // 32
    reps = F.decode_e4m3(rng.integers(1, 126, (2, 512))) * 2.0 ** -3
    c2, s2 = F.quantize_mxfp8(reps.astype(np.float32))
    assert np.array_equal(F.decode_mxfp8(c2, s2), reps)
    one = np.zeros((1, 512), dtype=np.float32)
    one[0, 40] = 448.0 * 4                                           # block 1 only
    c3, s3 = F.quantize_mxfp8(one)
    assert s3[0, 1] == 129 and s3[0, 0] == 127 and c3[0, 40] == 0x7E


def test_nvfp4_record_scale_and_codes():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((30, 512)) * np.exp(rng.uniform(-4, 4, (30, 32))).repeat(16, axis=1)).astype(np.float32)
    packed, sc = F.quantize_nvfp4(x)
    assert packed.shape == (30, 256) and sc.shape == (30, 32)
    amax = np.abs(x.astype(np.float64)).reshape(30, 32, 16).max(axis=-1)
    sv = F.decode_e4m3(sc)
    # the scale is the e4m3 value nearest amax / 6 (brute force over the positive codes)
    pos = F.decode_e4m3(np.arange(0, 127))
    for i in range(30):
        for j in range(32):
            d = np.abs(pos - amax[i, j] / 6.0)
            assert abs(sv[i, j] - amax[i, j] / 6.0) <= d.min() * (1 + 1e-6) + 1e-30
    dec = F.decode_nvfp4(packed, sc)
    # each value within half an e2m1 step of x / s (in units of s), or saturated at 6 s
    y = x.astype(np.float64) / np.repeat(sv, 16, axis=1)
    half = np.where(np.abs(y) < 2, 0.25, np.where(np.abs(y) < 4, 0.5, 1.0)) * np.repeat(sv, 16, axis=1)
    sat = np.abs(y) > 6
    assert np.all((np.abs(dec - x) <= half * (1 + 1e-6)) | sat)
    assert np.all(np.abs(dec[sat]) == 6 * np.repeat(sv, 16, axis=1)[sat])
    # low nibble first, scale per 16 values
    one = np.zeros((1, 512), dtype=np.float32)
    one[0, 16], one[0, 17] = 6.0, 3.0                                # block 1: amax 6 -> scale 1
    p1, s1 = F.quantize_nvfp4(one)
    assert s1[0, 1] == 0x38 and p1[0, 8] == (0x7 | (0x5 << 4)) and s1[0, 0] == 0

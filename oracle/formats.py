"""Number formats of the stored caches, decoded exactly to float64.

The caches of the DeepSeek-V4 path hold bf16 rows, "fp8_ds_mla" records
(e4m3 latent dims with one power-of-two UE8M0 scale per 64 dims, bf16 rotary
dims; "DeepSeek V4 Attention: Code Reading Map", compression steps 6-7 and the
"What This Repo Is For" list) and MXFP4 indexer keys (e2m1 with one UE8M0 scale
per 32 values; "DeepSeek V4.1 attention" API page, indexer K cache row width).
The bit-level meaning of e4m3, e2m1 and UE8M0 is the OCP 8-bit floating point
and OCP Microscaling v1.0 definitions, which the pages name but do not print.

Parity pins (tests/test_oracle_formats.py): the minifloat decoders agree with
torch's float8_e4m3fn / float8_e5m2 / bfloat16 and NumPy's float16 tables through
one generic decoder; the rounding encoders agree with torch's round-to-nearest-
even casts; record decoders round-trip independently made records.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------- decoders


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the value is the float32 with these as its top 16 bits."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    mant = code & 0x7
    if e == 0xF and mant == 0x7:
        return float("nan")          # e4m3fn has no infinities; S.1111.111 is NaN
    if e == 0:
        return s * (mant / 8.0) * 2.0 ** (1 - 7)      # subnormal
    return s * (1.0 + mant / 8.0) * 2.0 ** (e - 7)


def _e2m1_value(code: int) -> float:
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    mant = code & 0x1
    if e == 0:
        return s * (mant / 2.0)                         # subnormal: 0 or 0.5
    return s * (1.0 + mant / 2.0) * 2.0 ** (e - 1)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def decode_e4m3(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e2m1(nibbles) -> np.ndarray:
    return E2M1_TABLE[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def decode_ue8m0(b) -> np.ndarray:
    """UE8M0 scale byte -> 2**(b-127); 255 is NaN."""
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


FP8DS_LATENT, FP8DS_ROPE, FP8DS_BLOCK = 448, 64, 64


def decode_fp8ds(codes, rope_bits, scales) -> np.ndarray:
    """fp8_ds record -> float64 [..., 512]: latent c = e4m3(code c) * 2**(scale[c // 64] - 127),
    rotary dims are bf16 as stored."""
    codes = np.asarray(codes, dtype=np.uint8)
    lead = codes.shape[:-1]
    lat = decode_e4m3(codes).reshape(*lead, FP8DS_LATENT // FP8DS_BLOCK, FP8DS_BLOCK)
    lat = lat * decode_ue8m0(scales)[..., None]
    return np.concatenate([lat.reshape(*lead, FP8DS_LATENT), decode_bf16(rope_bits)], axis=-1)


MX_BLOCK = 32


def decode_mxfp4(packed, scales) -> np.ndarray:
    """MXFP4 row -> float64 [..., D]: element 2j is the low nibble of byte j, 2j+1 the high one;
    element c is scaled by 2**(scale[c // 32] - 127)."""
    packed = np.asarray(packed, dtype=np.uint8)
    lead, half = packed.shape[:-1], packed.shape[-1]
    nib = np.empty(lead + (2 * half,), dtype=np.uint8)
    nib[..., 0::2] = packed & 0xF
    nib[..., 1::2] = packed >> 4
    v = decode_e2m1(nib).reshape(*lead, 2 * half // MX_BLOCK, MX_BLOCK)
    return (v * decode_ue8m0(scales)[..., None]).reshape(*lead, 2 * half)


FP8IX_DIM = 128


def decode_fp8ix(codes, scale) -> np.ndarray:
    """FP8 indexer key row (128 e4m3 codes + one float32 scale; the 132-byte row of the "DeepSeek
    V4.1 attention" page's indexer cache, one scale per 128 dims) -> float64 [..., 128]."""
    return decode_e4m3(codes) * np.asarray(scale, dtype=np.float64)[..., None]


MXFP8_DIM, MXFP8_BLOCK = 512, 32
NVFP4_DIM, NVFP4_BLOCK = 512, 16


def decode_mxfp8(codes, scales) -> np.ndarray:
    """MXFP8 row (the "DeepSeek V4.1 attention" page's 528-byte KV record: 512 e4m3 codes and one
    UE8M0 scale per 32 values) -> float64 [..., 512]: value c = e4m3(code c) * 2**(scale[c // 32] - 127)."""
    codes = np.asarray(codes, dtype=np.uint8)
    lead = codes.shape[:-1]
    v = decode_e4m3(codes).reshape(*lead, MXFP8_DIM // MXFP8_BLOCK, MXFP8_BLOCK)
    return (v * decode_ue8m0(scales)[..., None]).reshape(*lead, MXFP8_DIM)


def decode_nvfp4(packed, scales) -> np.ndarray:
    """NVFP4 row (the same page's 288-byte compressed record: 256 bytes of e2m1 pairs, element 2j
    in the low nibble of byte j, and one e4m3 scale per 16 values) -> float64 [..., 512]:
    value c = e2m1(code c) * e4m3(scale[c // 16])."""
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    nib = np.empty(lead + (2 * packed.shape[-1],), dtype=np.uint8)
    nib[..., 0::2] = packed & 0xF
    nib[..., 1::2] = packed >> 4
    v = decode_e2m1(nib).reshape(*lead, NVFP4_DIM // NVFP4_BLOCK, NVFP4_BLOCK)
    return (v * decode_e4m3(scales)[..., None]).reshape(*lead, NVFP4_DIM)


# ----------------------------------------------------------------- rounding (reference rules)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); returns uint16 bit patterns.
    bf16 keeps 8 significant bits; normal exponents down to -126."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| = f * 2**e, f in [0.5, 1)
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x / quantum) * quantum       # np.rint rounds half to even
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_e4m3(y) -> np.ndarray:
    """Round float64 values with |y| <= 448 to the nearest e4m3fn code (ties to even mantissa).
    4 significant bits for |y| >= 2**-6, a fixed 2**-9 step below."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) > 448.0):
        raise ValueError("e4m3 rounding needs |y| <= 448 (the block scale guarantees it)")
    a = np.abs(y)
    _, e = np.frexp(a)
    quantum = np.where(a >= 2.0 ** -6, np.ldexp(1.0, e - 4), 2.0 ** -9)
    r = np.rint(a / quantum) * quantum
    # encode r: exponent field E (bias 7), 3 mantissa bits
    _, er = np.frexp(np.where(r > 0, r, 1.0))
    normal = r >= 2.0 ** -6
    E = np.where(normal, er - 1 + 7, 0)
    mant = np.where(normal, np.rint((r / np.ldexp(1.0, er - 1) - 1.0) * 8.0), np.rint(r / 2.0 ** -9))
    code = (E.astype(np.int64) << 3) | mant.astype(np.int64)
    code = code | np.where(y < 0, 0x80, 0)
    return code.astype(np.uint8)


def ue8m0_exponent(amax, qmax: float) -> np.ndarray:
    """Smallest integer e with amax <= qmax * 2**e (0 where amax == 0), clamped to [-127, 127].
    This is the power-of-two block-scale rule (scale = 2**ceil(log2(amax / qmax)))."""
    amax = np.asarray(amax, dtype=np.float64)
    qf, qe = np.frexp(qmax)                  # qmax = qf * 2**qe
    f, E = np.frexp(np.where(amax > 0, amax, 1.0))
    e = E - qe + (f > qf)
    e = np.where(amax > 0, e, 0)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_fp8ds(x32):
    """fp8_ds record of float32 values [..., 512]: per 64-dim latent block the power-of-two scale
    2**e with e the smallest integer such that amax <= 448 * 2**e, codes = RNE_e4m3(x / 2**e);
    the 64 rotary dims are rounded to bf16. Returns (codes uint8, rope bits uint16, scales uint8)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    lead = x.shape[:-1]
    lat = x[..., :FP8DS_LATENT].reshape(*lead, FP8DS_LATENT // FP8DS_BLOCK, FP8DS_BLOCK)
    e = ue8m0_exponent(np.abs(lat).max(axis=-1), 448.0)
    codes = round_e4m3(lat / np.ldexp(1.0, e)[..., None]).reshape(*lead, FP8DS_LATENT)
    return codes, round_bf16(x[..., FP8DS_LATENT:]), (e + 127).astype(np.uint8)


def round_e2m1(y) -> np.ndarray:
    """Nearest e2m1 code (nibble, sign in bit 3) of values with |y| <= 6; a value halfway
    between two neighbours takes the one whose code is even (mantissa bit 0), as the OCP MX
    round-to-nearest-even conversion does."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) > 6.0):
        raise ValueError("e2m1 rounding needs |y| <= 6 (the block scale guarantees it)")
    a = np.abs(y)
    mags = E2M1_TABLE[:8]                     # 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7
    dist = np.abs(a[..., None] - mags)
    best = dist.min(axis=-1, keepdims=True)
    # among the nearest (one, or two at a tie) prefer the even code
    cand = np.where(dist == best, np.arange(8) + 16 * (np.arange(8) & 1), 99)
    code = (cand.min(axis=-1) % 16).astype(np.int64)
    code = code | np.where(y < 0, 0x8, 0)     # the sign is kept, also when the value rounds to 0
    return code.astype(np.uint8)


def quantize_mxfp4(x32):
    """MXFP4 row of float32 values [..., D]: per 32 values the power-of-two scale 2**e with e the
    smallest integer such that amax <= 6 * 2**e, codes = nearest-even e2m1 of x / 2**e, element
    2j in the low nibble of byte j. Returns (packed uint8 [..., D/2], scales uint8 [..., D/32])."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.reshape(*lead, D // MX_BLOCK, MX_BLOCK)
    e = ue8m0_exponent(np.abs(blk).max(axis=-1), 6.0)
    nib = round_e2m1(blk / np.ldexp(1.0, e)[..., None]).reshape(*lead, D)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def quantize_fp8ix(x32):
    """FP8 indexer key row of float32 values [..., 128]: one power-of-two scale 2**e for the row
    (e the smallest integer with amax <= 448 * 2**e), codes = RNE_e4m3(x / 2**e). Returns
    (codes uint8 [..., 128], scale float32 [...])."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    e = ue8m0_exponent(np.abs(x).max(axis=-1), 448.0)
    codes = round_e4m3(x / np.ldexp(1.0, e)[..., None])
    return codes, np.ldexp(1.0, e).astype(np.float32)


def quantize_mxfp8(x32):
    """MXFP8 row of float32 values [..., 512]: per 32 values the power-of-two scale 2**e with e the
    smallest integer such that amax <= 448 * 2**e, codes = RNE_e4m3(x / 2**e).
    Returns (codes uint8 [..., 512], scales uint8 [..., 16])."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    lead = x.shape[:-1]
    blk = x.reshape(*lead, MXFP8_DIM // MXFP8_BLOCK, MXFP8_BLOCK)
    e = ue8m0_exponent(np.abs(blk).max(axis=-1), 448.0)
    codes = round_e4m3(blk / np.ldexp(1.0, e)[..., None]).reshape(*lead, MXFP8_DIM)
    return codes, (e + 127).astype(np.uint8)


def quantize_nvfp4(x32):
    """NVFP4 row of float32 values [..., 512]: per 16 values the scale s = RNE_e4m3(amax / 6)
    (the quotient taken in float32), codes = nearest-even e2m1 of x / s in float32, saturated to
    +-6 (a scale rounded down can leave amax / s slightly above 6); a block whose scale rounds to
    0 stores zero codes. Returns (packed uint8 [..., 256], scales uint8 [..., 32])."""
    x = np.asarray(x32, dtype=np.float32)
    lead = x.shape[:-1]
    blk = x.reshape(*lead, NVFP4_DIM // NVFP4_BLOCK, NVFP4_BLOCK)
    amax = np.abs(blk).max(axis=-1)
    sq = (amax / np.float32(6.0)).astype(np.float32)
    sc = round_e4m3(np.minimum(sq.astype(np.float64), 448.0))
    sv = decode_e4m3(sc).astype(np.float32)
    safe = np.where(sv > 0, sv, np.float32(1.0)).astype(np.float32)
    y = (blk / safe[..., None]).astype(np.float32).astype(np.float64)
    y = np.where(sv[..., None] > 0, np.clip(y, -6.0, 6.0), 0.0)
    nib = round_e2m1(y).reshape(*lead, NVFP4_DIM)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, sc

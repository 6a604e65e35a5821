"""Exact value decoders for the KV-cache storage formats (oracle, test-only).

The cache stores keys and values as 16-bit floats (bf16 / fp16), as 32-bit
floats, or as 8-bit codes (INT8 or FP8).  "KV Cache Engineering for LLM
Serving", section "The cache formula", fixes two bytes per value for BF16 and
one for FP8; section 8 "Quantization" describes storing a small code plus a
scale.  The FP8 flavours here are OCP E4M3 (the "fn" variant: no infinities,
one NaN pattern per sign) and OCP E5M2 (IEEE-like: infinities and NaNs in
the top exponent), the two FP8 formats the gfx950 converts in hardware; "Chapter 18 -
KV-Cache Optimization Strategies", section "vLLM with PagedAttention + KV
Quantization", stores the cache as ``fp8_e5m2``.

Nothing here rounds except the two FP8 encoders; every decoder is exact.
"""

import numpy as np

# ---------------------------------------------------------------------------
# bf16 / fp16 / fp32
# ---------------------------------------------------------------------------


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> exact float32 values.

    A bf16 number is the upper half of an IEEE binary32 number, so placing the
    16 bits in the high half of a 32-bit word gives the same value exactly.
    """
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits_to_f32(bits):
    """IEEE binary16 bit patterns (uint16) -> exact float32 values."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP "fn" flavour)
# ---------------------------------------------------------------------------

E4M3_BIAS = 7
E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of one FP8-E4M3 code, from the format definition.

    Bit layout S.EEEE.MMM, exponent bias 7.  Exponent field 0 encodes
    subnormals m * 2^-9; fields 1..15 encode (1 + m/8) * 2^(e-7), except
    S.1111.111 which is NaN.  There is no infinity, so the largest finite
    magnitude is 1.75 * 2^8 = 448.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** (1 - E4M3_BIAS - 3)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)
    return sign * mag


# All 256 code values; every finite one is exactly representable in fp32.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite magnitudes, indexed by code 0x00..0x7E (increasing).
_E4M3_MAGS = E4M3_TABLE[:0x7F].copy()


def e4m3_to_f32(codes):
    """FP8-E4M3 codes (uint8) -> exact float32 values (table lookup)."""
    c = np.asarray(codes).astype(np.uint8)
    return E4M3_TABLE[c].astype(np.float32)


def _fp8_encode(x, mags, largest, name):
    """float32 values -> FP8 codes of the format whose non-negative finite
    magnitudes, by code 0 .. len(mags) - 1, are ``mags`` (increasing); round
    to nearest, ties to even.

    Brute force: for each |x| the distance to every finite non-negative
    magnitude is computed and the nearest is taken; on an exact tie the
    candidate whose code integer is even wins (codes are monotonic in
    magnitude, so a tie is always between neighbours c, c+1 and exactly one
    is even).  Magnitudes above the largest finite one saturate to it.  The
    sign bit of x is kept, so a negative value that rounds to zero gives
    0x80.  Distances are taken in float64, which is exact wherever a tie can
    occur (x and both neighbours lie within a few binades of each other).
    """
    xf = np.asarray(x, dtype=np.float32)
    flat = xf.reshape(-1)
    if np.isnan(flat).any():
        raise ValueError(f"{name}: NaN input is outside the quantiser's domain")
    mag = np.abs(flat.astype(np.float64))
    n = len(mags)
    out = np.empty(flat.shape, dtype=np.uint8)
    chunk = 1 << 16
    for lo in range(0, flat.size, chunk):
        m = mag[lo:lo + chunk]
        d = np.abs(m[:, None] - mags[None, :])                 # [n_x, n]
        best = d.min(axis=1, keepdims=True)
        is_best = d == best
        # among the (one or two) nearest codes, prefer the even code integer
        even = (np.arange(n) % 2 == 0)[None, :]
        pick_even = is_best & even
        has_even = pick_even.any(axis=1)
        first_best = is_best.argmax(axis=1)
        first_even = pick_even.argmax(axis=1)
        code = np.where(has_even, first_even, first_best).astype(np.uint8)
        code[m > largest] = n - 1
        out[lo:lo + chunk] = code
    sign = np.signbit(flat)
    out = out | np.where(sign, np.uint8(0x80), np.uint8(0))
    return out.reshape(xf.shape)


def e4m3_encode(x):
    """float32 values -> FP8-E4M3 codes, round to nearest, ties to even;
    magnitudes above 448 saturate to 448 (code 0x7E)."""
    return _fp8_encode(x, _E4M3_MAGS, E4M3_MAX, "e4m3_encode")


# ---------------------------------------------------------------------------
# FP8 E5M2 (OCP)
# ---------------------------------------------------------------------------

E5M2_BIAS = 15
E5M2_MAX = 57344.0


def e5m2_value(code):
    """Value of one FP8-E5M2 code, from the format definition.

    Bit layout S.EEEEE.MM, exponent bias 15.  Exponent field 0 encodes
    subnormals m * 2^-16; fields 1..30 encode (1 + m/4) * 2^(e-15); field 31
    is infinity (m = 0) or NaN.  The largest finite magnitude is
    1.75 * 2^15 = 57344.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        mag = m * 2.0 ** (1 - E5M2_BIAS - 2)
    else:
        mag = (1.0 + m / 4.0) * 2.0 ** (e - E5M2_BIAS)
    return sign * mag


E5M2_TABLE = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite magnitudes, indexed by code 0x00..0x7B (increasing).
_E5M2_MAGS = E5M2_TABLE[:0x7C].copy()


def e5m2_to_f32(codes):
    """FP8-E5M2 codes (uint8) -> exact float32 values (table lookup)."""
    c = np.asarray(codes).astype(np.uint8)
    return E5M2_TABLE[c].astype(np.float32)


def e5m2_encode(x):
    """float32 values -> FP8-E5M2 codes, round to nearest, ties to even;
    magnitudes above 57344 saturate to 57344 (code 0x7B), so the quantiser
    never stores an infinity."""
    return _fp8_encode(x, _E5M2_MAGS, E5M2_MAX, "e5m2_encode")


# ---------------------------------------------------------------------------
# INT4: two signed 4-bit codes per byte
# ---------------------------------------------------------------------------
# "KV Cache Engineering", section 8 "Quantization": a 4-bit format keeps a
# quarter of the BF16 payload; its codes are -7..7.  Storage here: element
# 2i in the low nibble of byte i, element 2i + 1 in the high nibble, each a
# two's-complement 4-bit number.


def i4_pack(codes):
    """Signed codes in [-8, 7], last dimension even -> packed uint8 bytes
    (last dimension halved)."""
    c = np.asarray(codes).astype(np.int64)
    if c.shape[-1] % 2:
        raise ValueError("i4_pack: last dimension must be even")
    if (c < -8).any() or (c > 7).any():
        raise ValueError("i4_pack: code outside [-8, 7]")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def i4_unpack(raw):
    """Packed uint8 bytes -> signed codes (int8), last dimension doubled."""
    b = np.asarray(raw).astype(np.uint8).astype(np.int64)
    lo = b & 0xF
    hi = b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------------------
# dispatch by storage dtype name
# ---------------------------------------------------------------------------

def decode(raw, dtype):
    """Raw stored data -> exact float32 values, for dtype in
    {"f32", "bf16", "f16", "i8", "i4", "fp8e4m3", "fp8e5m2"}.

    ``raw`` holds the storage words: float32 for "f32", uint16 bit patterns
    for "bf16"/"f16", int8 codes for "i8", packed uint8 nibbles for "i4"
    (the last dimension holds half the elements), uint8 codes for
    "fp8e4m3".
    Integer and FP8 codes decode to the code's own value (the scale is
    applied separately, see ``quant.dequantize``).
    """
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(raw)
    if dtype == "f16":
        return f16_bits_to_f32(raw)
    if dtype == "i8":
        return np.asarray(raw).astype(np.int8).astype(np.float32)
    if dtype == "i4":
        return i4_unpack(raw).astype(np.float32)
    if dtype == "fp8e4m3":
        return e4m3_to_f32(raw)
    if dtype == "fp8e5m2":
        return e5m2_to_f32(raw)
    raise ValueError(f"unknown dtype {dtype!r}")

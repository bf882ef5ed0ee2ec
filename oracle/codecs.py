"""Bit-level codecs for the cache storage formats (oracle; test infrastructure only).

The pages say only that the KV cache can be compressed "down to 8-bit or 4-bit"
("KV Cache Management", "Watch Out For" and "What to Read Next"); they fix no format.
The reading taken here: 8-bit means OCP FP8 E4M3FN (1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, no infinities, the all-ones pattern of each sign is NaN, largest
finite magnitude 448), with one float32 scale per (layer, KV head):

    stored code   c = round_to_nearest_even_saturating(float32(x / scale))
    decoded value     e4m3(c) * scale

bfloat16 is the top 16 bits of an IEEE binary32.  Decoding is exact in float64.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- bfloat16

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even.  NaN stays NaN.

    Written from the definition: among the two bfloat16 neighbours of x (truncation and
    truncation + 1 ulp) take the nearer; on a tie take the one whose last kept bit is 0.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lo = u >> np.uint64(16)                  # truncated pattern
    rem = u & np.uint64(0xFFFF)              # dropped bits
    half = np.uint64(0x8000)
    up = (rem > half) | ((rem == half) & ((lo & np.uint64(1)) == np.uint64(1)))
    out = (lo + up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(x)
    out[nan] = (lo[nan].astype(np.uint16) | np.uint16(0x0040))  # keep sign, force quiet NaN
    return out


# ----------------------------------------------------------------------------- fp8 e4m3fn

E4M3_MAX = 448.0


def _e4m3_value(code: int) -> float:
    """Value of one E4M3FN code, from the format definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)      # subnormal: 0.m * 2^(1-bias)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)     # normal: 1.m * 2^(e-bias)


E4M3_DECODE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
"""float64 value of each of the 256 codes (index = code)."""

# finite non-negative codes 0x00..0x7E in increasing value order (values strictly increase)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = E4M3_DECODE[:0x7F]


def e4m3_bits_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of E4M3FN codes (uint8) as float64."""
    return E4M3_DECODE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN code: nearest representable value, ties to the even code,
    magnitudes beyond 448 saturate to 448, NaN -> 0x7F with the sign of x.

    Nearest-value search over the 127 finite non-negative codes (the plain definition);
    the sign is carried separately, so -0.0 encodes to 0x80.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    sign = (np.signbit(x)).astype(np.uint8) << np.uint8(7)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # index of the first value >= a; candidates are that code and the one below it
    hi = np.searchsorted(_POS_VALS, a, side="left")
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_POS_VALS[hi] - a)
    d_lo = np.abs(a - _POS_VALS[lo])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


def e4m3_quantize(x_f64: np.ndarray, scale) -> np.ndarray:
    """Codes for values x (float64, exactly the stored input values) under float32 scale(s)
    (broadcast against x).

    The quotient is formed in float64 and rounded once to float32: for a division of two
    float32 values that equals the correctly rounded float32 quotient (double rounding is
    innocuous for division when the wide format has at least 2p+2 bits; Figueroa,
    "When is double rounding innocuous?", SIGNUM Newsletter 1995).
    """
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    q = (np.asarray(x_f64, dtype=np.float64) / s).astype(np.float32)
    return e4m3_encode(q)


# ----------------------------------------------------------------------------- 4-bit: OCP MXFP4
#
# The pages allow a cache "down to 8-bit or 4-bit" and fix no 4-bit format.  The reading taken
# here: OCP Microscaling MXFP4 (OCP "Microscaling Formats (MX) Specification" v1.0), the 4-bit
# format gfx950 converts in hardware.  Each 32 consecutive head dims of one token's K (or V)
# row form a block sharing one E8M0 scale 2^E; each element is an E2M1 code (1 sign bit, 2
# exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
#   E      = floor(log2(max |x| over the block)) - 2   (2 = the largest E2M1 exponent),
#            clamped to the E8M0 range [-127, 127]; a block of zeros takes E = -127
#   code_i = round_to_nearest_even_saturating(x_i / 2^E)   (saturating at 6)
#   value  = e2m1(code_i) * 2^E
# A block holding NaN or an infinity stores the NaN scale (0xFF) and zero codes; it decodes to
# NaN.  The sign of an element is kept also when it rounds to zero (code 8 is -0).

MX_BLOCK = 32
E2M1_MAX = 6.0
E8M0_NAN = 0xFF


def _e2m1_value(code: int) -> float:
    """Value of one E2M1 code, from the format definition."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * (m / 2.0)                           # subnormal: 0.m * 2^(1-bias)
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)        # normal: 1.m * 2^(e-bias)


E2M1_DECODE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_E2M1_POS = E2M1_DECODE[:8]


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float64 values -> E2M1 codes: nearest representable magnitude, ties to the even code
    (mantissa bit 0), magnitudes beyond 6 saturate to 6; the sign is carried separately."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    hi = np.clip(np.searchsorted(_E2M1_POS, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    d_hi = np.abs(_E2M1_POS[hi] - a)
    d_lo = np.abs(a - _E2M1_POS[lo])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << np.uint8(3))


def mx_block_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent E of blocks with the given max |x| (finite, >= 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                                 # amax = f * 2^e, f in [0.5, 1)
    E = np.where(amax > 0, e - 1 - 2, -127)
    return np.clip(E, -127, 127).astype(np.int64)


def mxfp4_quantize(x: np.ndarray):
    """Rows x [..., D] (float64, D a multiple of 32) -> (codes uint8 [..., D] in 0..15,
    E8M0 scale codes uint8 [..., D // 32])."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(*x.shape[:-1], x.shape[-1] // MX_BLOCK, MX_BLOCK)
    finite = np.all(np.isfinite(blocks), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0.0)), axis=-1)
    E = mx_block_exponent(amax)
    codes = e2m1_encode(blocks / np.ldexp(1.0, E)[..., None])
    codes = np.where(finite[..., None], codes, np.uint8(0)).astype(np.uint8)
    scales = np.where(finite, E + 127, E8M0_NAN).astype(np.uint8)
    return codes.reshape(x.shape), scales


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of codes [..., D] under their blocks' E8M0 scales [..., D // 32]."""
    codes = np.asarray(codes, dtype=np.int64)
    scales = np.asarray(scales, dtype=np.int64)
    blocks = E2M1_DECODE[codes].reshape(*codes.shape[:-1], codes.shape[-1] // MX_BLOCK, MX_BLOCK)
    f = np.where(scales == E8M0_NAN, np.nan, np.ldexp(1.0, scales - 127))
    return (blocks * f[..., None]).reshape(codes.shape)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """4-bit codes [..., D] -> bytes [..., D // 2]: element 2i in the low nibble of byte i."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out


# ----------------------------------------------------------------------------- storage views

def storage_to_f64(arr: np.ndarray, fmt: str) -> np.ndarray:
    """Exact float64 value of a stored array.  fmt in {'f32', 'bf16', 'fp8'}; fp8 values are
    returned unscaled (the caller multiplies by the per-head scale)."""
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(arr)
    if fmt == "fp8":
        return e4m3_bits_to_f64(arr)
    raise ValueError(f"unknown storage format {fmt!r}")

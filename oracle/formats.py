"""Exact number-format codecs for the oracle (float64, numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the formats but not their bit layouts: FP8 operands with fp32
scale factors on SM90 (usage guide, "五、使用方法"), FP4 weights with UE8M0
scale factors packed four to an int32 (news page on the Mega-MoE update,
"FP4 精度支持").  The plainest reading is the OCP definitions, written out here:

* e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
  subnormal; S.1111.111 is NaN; no infinities; largest finite 448.
* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no NaN/inf.
* UE8M0: unsigned 8-bit exponent, value 2**(e-127); 255 is NaN.
* bf16: the upper 16 bits of an IEEE binary32.
"""

import numpy as np


def _e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9          # subnormal: m/8 * 2**(1-7)
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def _e2m1_value(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5                # subnormal: m/2 * 2**(1-1)
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_MAX = 448.0
E2M1_MAX = 6.0


def decode_e4m3(codes) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e2m1_nibbles(nibbles) -> np.ndarray:
    """4-bit E2M1 codes (values 0..15) -> float64 values (exact)."""
    return E2M1_TABLE[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def unpack_e2m1(packed) -> np.ndarray:
    """Packed FP4 bytes [..., K/2] -> float64 [..., K].

    Two elements per byte; element 2i is the low nibble of byte i, element 2i+1
    the high nibble (the pages say only "FP4"; this order is a stated reading).
    """
    p = np.asarray(packed, dtype=np.uint8)
    lo = decode_e2m1_nibbles(p & 0xF)
    hi = decode_e2m1_nibbles(p >> 4)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def decode_ue8m0(exps) -> np.ndarray:
    """UE8M0 bytes -> float64 powers of two (255 -> NaN)."""
    e = np.asarray(exps, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def unpack_ue8m0_int32(packed) -> np.ndarray:
    """int32 words holding four UE8M0 bytes [..., W] -> float64 scales [..., 4W].

    Scale j of a row sits in word j // 4, byte j % 4 counted from the least
    significant byte (the pages say only "4 UE8M0 per int32"; little-endian
    byte order is the stated reading).
    """
    w = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
    b = np.stack([(w >> (8 * i)) & 0xFF for i in range(4)], axis=-1)
    return decode_ue8m0(b.reshape(w.shape[:-1] + (4 * w.shape[-1],)))


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return u.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); returns float64.

    Done directly from the float64 value (one rounding), by scaling the
    significand to 8 bits and using numpy's half-to-even rounding.  Values
    beyond the bf16 range become +-inf; bf16 subnormals are not needed by any
    workload here and are rounded on the subnormal grid for completeness.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                      # below 2**-126 use the subnormal grid
    # 8 significant bits: the grid step is 2**(e-8); np.round is half-to-even
    q = np.round(np.ldexp(x[fin], 8 - e))
    r = np.ldexp(q, e - 8)
    big = np.abs(r) > float.fromhex("0x1.fep127")
    r = np.where(big, np.sign(r) * np.inf, r)
    out[fin] = r
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 to bf16 (ties to even) and return the uint16 bit patterns."""
    r = round_to_bf16(x).astype(np.float32)      # exact: r already has 8 significant bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# Encoder used inside the FFN pipeline (requantisation of the SwiGLU output).
# ----------------------------------------------------------------------------

_E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)         # 0x00..0x7E: all finite non-negative
_E4M3_POS_VALUES = E4M3_TABLE[_E4M3_POS_CODES]                # strictly increasing


def encode_e4m3_rne(x) -> np.ndarray:
    """Float values -> e4m3fn codes, round to nearest (ties to even code), saturating at +-448.

    Written as a nearest-neighbour search over the 127 finite non-negative
    codes: the two neighbours of |x| are found with a sorted search, the nearer
    one wins and an exact tie goes to the code with an even mantissa (even code
    number).  The sign bit is set for negative inputs (so -0.0 keeps its sign).
    NaN inputs are not expected and raise.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("encode_e4m3_rne: NaN input")
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS_VALUES, mag, side="left")  # first value >= mag
    hi = np.minimum(hi, len(_E4M3_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    v_hi = _E4M3_POS_VALUES[hi]
    v_lo = _E4M3_POS_VALUES[lo]
    d_hi = v_hi - mag
    d_lo = mag - v_lo
    exact = v_hi == mag
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(x)
    return np.where(sign, code | 0x80, code).astype(np.uint8)


def pow2_scale_exponent(amax, qmax: float) -> np.ndarray:
    """Smallest integer e with 2**e * qmax >= amax (amax > 0); 0 where amax == 0.

    This is the power-of-two scale rule 2**ceil(log2(amax/qmax)) evaluated with
    exact comparisons instead of a floating-point log, so no rounding of
    amax/qmax or of log2 can move the result.
    """
    a = np.asarray(amax, dtype=np.float64)
    out = np.zeros(a.shape, dtype=np.int64)
    pos = a > 0
    _, ex = np.frexp(a[pos] / qmax)              # starting guess
    e = ex.astype(np.int64)
    # adjust to the exact smallest e with 2**e * qmax >= a
    for _ in range(3):
        up = np.ldexp(qmax, e) < a[pos]
        e = np.where(up, e + 1, e)
        down = np.ldexp(qmax, e - 1) >= a[pos]
        e = np.where(down, e - 1, e)
    out[pos] = e
    return out

"""Number-format codecs of the CPU oracle (bf16, OCP e4m3fn), written from the
format definitions.

TEST INFRASTRUCTURE ONLY: nothing on the product path may import this module.
Only tests/, the smoke check and the CPU-baseline leg of the benchmark use it.

Storage of fp8 pools as raw bytes follows the SGLang memory-pool article
(pinghaoyang.com.cn, "SGLang 源码完全拆解(十五)", section 二重映射: KV 存储池):
fp8 K/V live in byte buffers and are re-interpreted on read.  Which fp8 variant
and which rounding is a reading of ours (the article lists e4m3fn, e4m3fnuz and
e5m2 side by side): OCP e4m3fn, round to nearest with ties to the even code,
finite inputs beyond the largest finite value saturate to it, NaN encodes as
0x7F.

Everything here works on numpy arrays and in float64, where bf16 and e4m3 values
are exact.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits — the
# upper half of an IEEE binary32 word.
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16 / int16 array) as float64."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen unchanged
        return b.view(np.float32).astype(np.float64)


def _round_to_format(x: np.ndarray, sig_bits: int, min_normal_exp: int) -> np.ndarray:
    """Round float64 values to a binary format with `sig_bits` significant bits
    (hidden bit included) and smallest normal 2**min_normal_exp, ties to even.

    Written as the definition: the representable neighbours of |x| are the
    multiples of the quantum 2**(e - sig_bits + 1) where 2**e <= |x| < 2**(e+1)
    (e clamped at min_normal_exp for the subnormal range); np.round rounds the
    quotient half to even, which is ties-to-even on the last significant bit.
    No overflow handling here: callers saturate or compare against the range.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # floor(log2) can be off by one right at powers of two in floating point;
    # correct it exactly with ldexp comparisons.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, min_normal_exp)
    quantum = np.ldexp(1.0, (e - (sig_bits - 1)).astype(np.int64))
    return np.where(ax > 0, np.round(x / quantum) * quantum, x)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round to nearest bf16 (ties to even); returns uint16 bit patterns.

    bf16 has 8 significant bits and smallest normal 2**-126.  NaN maps to the
    quiet pattern 0x7FC0; overflow past the largest finite bf16 gives +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_format(x, 8, -126)
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)  # exact: r is a bf16 value (or overflows to inf)
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


# ---------------------------------------------------------------------------
# OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
#   exponent field 0      -> subnormal  m * 2**-9
#   exponent field 1..15  -> (1 + m/8) * 2**(E - 7)
#   S.1111.111            -> NaN (no infinities); largest finite 448 (0x7E)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    """Value of every one of the 256 codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = s * man * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of e4m3fn byte codes as float64 (NaN for the NaN codes)."""
    return E4M3_VALUES[np.asarray(codes).astype(np.uint8)]


def f64_to_e4m3(x) -> np.ndarray:
    """Encode to e4m3fn bytes: nearest finite code, ties to the even code,
    |x| > 448 (and +-inf) saturates to +-448, NaN -> 0x7F.

    Implemented as a search over the table of the 127 non-negative finite codes
    (their values increase with the code), independent of any bit trick.
    """
    x = np.asarray(x, dtype=np.float64)
    pos_vals = E4M3_VALUES[:0x7F]  # codes 0x00..0x7E, increasing
    ax = np.minimum(np.abs(np.nan_to_num(x, nan=0.0, posinf=E4M3_MAX, neginf=-E4M3_MAX)), E4M3_MAX)
    hi = np.searchsorted(pos_vals, ax, side="left")  # first code with value >= ax
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = pos_vals[hi] - ax
    d_lo = ax - pos_vals[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(pos_vals[hi] == ax, hi, code)
    code = code.astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code


def decode_store(bits, dtype: str) -> np.ndarray:
    """Exact float64 values of pool / tensor storage in `dtype`
    ('f32' float32 array, 'bf16' uint16 bits, 'e4m3' uint8 codes)."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "e4m3":
        return e4m3_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def encode_store(x, dtype: str) -> np.ndarray:
    """Round float64 values into storage `dtype` (see decode_store)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    if dtype == "e4m3":
        return f64_to_e4m3(x)
    raise ValueError(f"unknown dtype {dtype!r}")

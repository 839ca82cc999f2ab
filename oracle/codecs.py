"""Number formats of the pool: fp32 and bf16 bit patterns, and fp8 e4m3.

[ch7] 「vLLM 关键参数速记」 names `--kv-cache-dtype fp8_e4m3`, which halves the KV bytes of bf16
(7.1 「KV cache 显存估算」: bf16 = 2 bytes, fp8 = 1 byte).  The pages do not define the format;
the reading taken is the OCP 8-bit E4M3 ("FN") format native to gfx950: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448.

Quantisation of a stored value x with a per-tensor fp32 scale s (the reading taken where the pages
are silent): inv = fp32(1 / s) rounded once; y = fp32(x * inv) rounded to nearest-even; y is
clamped to [-448, 448]; y is rounded to the nearest e4m3 value, ties to the even code.
Dequantisation: decode(code) * s.
"""
import numpy as np

E4M3_MAX = 448.0


def f32_bits_to_f64(bits) -> np.ndarray:
    """fp32 bit patterns (uint32) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """e4m3 codes (uint8) -> float64 from the format's definition.

    exponent field e, mantissa field m:
      e == 0           : (-1)^s * 2^-6 * (m / 8)          (subnormal)
      e in 1..15       : (-1)^s * 2^(e - 7) * (1 + m / 8)  (normal)
      e == 15, m == 7  : NaN
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


# Positive finite e4m3 values, ascending: code i has value _E4M3_POS[i] for i in 0..126.
_E4M3_POS = e4m3_decode(np.arange(0, 127, dtype=np.uint8))


def e4m3_encode(y) -> np.ndarray:
    """Nearest e4m3 code to each fp32 value, ties to the even code, saturating at +-448.

    The value is first clamped to [-448, 448]; the nearest of the 127 non-negative finite values is
    then found by search; the sign bit is copied from the input (so -0.0 -> 0x80).  NaN -> 0x7F.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")       # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_POS[hi], hi, code).astype(np.uint8)   # exact hits
    code = code | (np.signbit(y).astype(np.uint8) << np.uint8(7))
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def e4m3_quantise(x_f32, scale: float) -> np.ndarray:
    """Stored code of value x under per-tensor scale `scale` (see module docstring)."""
    inv = np.float32(1.0) / np.float32(scale)          # one fp32 division, rounded to nearest
    y = np.asarray(x_f32, dtype=np.float32) * inv       # fp32 product, rounded to nearest-even
    return e4m3_encode(y)


def decode_pool(pool_codes: np.ndarray, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """Stored codes -> float64 values (fp8 codes are multiplied by the fp32 scale, exactly in fp64)."""
    if kv_dtype == "f32":
        return f32_bits_to_f64(pool_codes)
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(pool_codes)
    if kv_dtype == "fp8":
        return e4m3_decode(pool_codes) * float(np.float32(scale))
    raise ValueError(kv_dtype)

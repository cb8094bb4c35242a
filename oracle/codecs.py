"""Exact decoding of the stored element formats (oracle; test infrastructure).

* bf16: the upper 16 bits of an IEEE-754 binary32 word. Decoding is the
  definition: shift the 16 bits into the high half of a 32-bit word.
* fp8: OCP 8-bit e4m3fn ("FN": finite, no infinities). Sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits. Exponent field 0 is subnormal
  (m/8 * 2^-6); the all-ones pattern S.1111.111 is NaN; the largest finite
  magnitude is 1.75 * 2^8 = 448. The pages only say "fp8" for the KV cache and
  the a8w8 kernel (ATOM pull request 2760, "Problem"; vLLM pull request 53001,
  "Test Plan" uses --kv-cache-dtype fp8); gfx950's matrix cores take the OCP
  formats, so the reading is OCP e4m3fn.

Values come back as float64, which holds every bf16 and e4m3fn value exactly.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def decode(codes: np.ndarray, dtype: str, scale=None) -> np.ndarray:
    """Real value = stored value * per-tensor scale (scale None means 1)."""
    if dtype == "bf16":
        v = bf16_to_f64(codes)
    elif dtype == "fp8":
        v = e4m3fn_to_f64(codes)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    if scale is not None:
        v = v * np.float64(np.float32(scale))
    return v

"""Latent cache write, by its definition (oracle; test infrastructure).

The decode step writes each new token's latent row into the paged cache: the
512 compressed dims kv_c and the 64 RoPE dims k_pe go, concatenated, into the
token's slot (vLLM pull request 57942, "Details": the KV-cache write goes
through concat_and_cache_mla). The same page's review thread traces corrupted
RoPE columns to an fp32 k_pe tensor read as if it were bf16; here every
source value is taken at its own dtype and converted.

Conversion to the cache format (this library's reading; the pages give no
rounding rule):
* bf16 cache: the source value rounded to the nearest bf16, ties to even;
  NaN stays NaN.
* fp8 cache (OCP e4m3fn, per-tensor scale s): v = x / s computed in float32
  (one correctly rounded division; the quantised code is decided in the
  kernel's precision), saturated to [-448, 448], rounded to the nearest e4m3fn
  value with ties to the even code; NaN becomes code 0x7F. The sign bit is
  kept for values that round to zero.
Tokens whose slot is negative (padding) or not below num_slots are skipped.
"""
import numpy as np

from .codecs import e4m3fn_to_f64

# Finite non-negative e4m3fn values in code order 0x00..0x7E (increasing).
_E4M3_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_E4M3_POS_VALS = e4m3fn_to_f64(_E4M3_POS_CODES)


def encode_bf16(x) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    quiet = ((u >> 16) | 0x40).astype(np.uint16)
    return np.where(nan, quiet, rounded).astype(np.uint16)


def encode_e4m3fn(v) -> np.ndarray:
    """float32 values (already divided by the scale) -> e4m3fn codes."""
    f = np.asarray(v, dtype=np.float32).astype(np.float64)
    sign = np.signbit(f)
    mag = np.minimum(np.abs(f), 448.0)
    # nearest representable magnitude: candidates below and above
    hi = np.clip(np.searchsorted(_E4M3_POS_VALS, mag, side="left"), 0, len(_E4M3_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_E4M3_POS_VALS) - 1)
    d_lo = np.abs(mag - _E4M3_POS_VALS[lo])
    d_hi = np.abs(_E4M3_POS_VALS[hi] - mag)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_E4M3_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _E4M3_POS_CODES[hi], _E4M3_POS_CODES[lo]).astype(np.uint8)
    code = np.where(sign, code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(f), np.uint8(0x7F), code).astype(np.uint8)


def cache_write(pool_codes: np.ndarray, kv_c, k_pe, slot_mapping, kv_dtype: str, kv_scale=None):
    """Return a copy of pool_codes ([num_slots, 576] uint16 bf16 bits or uint8
    e4m3fn codes) with each token's row written. kv_c [T, 512] and k_pe
    [T, 64] are the source values as float32 (every bf16, fp16 and fp32 value
    is one)."""
    out = np.array(pool_codes, copy=True)
    kv_c = np.asarray(kv_c, dtype=np.float32)
    k_pe = np.asarray(k_pe, dtype=np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    n = out.shape[0]
    for t, slot in enumerate(slots):
        if slot < 0 or slot >= n:
            continue
        row = np.concatenate([kv_c[t], k_pe[t]]).astype(np.float32)
        if kv_dtype == "bf16":
            out[slot] = encode_bf16(row)
        elif kv_dtype == "fp8":
            s = np.float32(1.0 if kv_scale is None else kv_scale)
            out[slot] = encode_e4m3fn(row / s)          # float32 division
        else:
            raise ValueError(f"unknown kv dtype {kv_dtype!r}")
    return out

"""Pins for the oracle's cache-write encoders (CPU only): torch's own casts
(round to nearest even) on values inside the format's range, exact round
trips over every code, and the saturation / NaN / sign rules."""
import numpy as np
import torch

from oracle.cache_write import cache_write, encode_bf16, encode_e4m3fn
from oracle.codecs import bf16_to_f64, e4m3fn_to_f64


def _halfway_points():
    """float32 values exactly halfway between adjacent finite e4m3fn values."""
    vals = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    return np.concatenate([mids, -mids]).astype(np.float32)


def test_e4m3_encoder_matches_torch_inside_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 60, 20000), rng.uniform(-448, 448, 20000),
        rng.normal(0, 2.0 ** -7, 20000), _halfway_points(), [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = encode_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all(), np.flatnonzero(ours != ref)[:10]


def test_e4m3_encoder_round_trips_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = encode_e4m3fn(e4m3fn_to_f64(codes).astype(np.float32))
    assert (back == codes).all()


def test_e4m3_encoder_saturates_and_maps_nan():
    got = encode_e4m3fn(np.array([449.0, 1e30, -1e30, np.inf, -np.inf, np.nan, -1e-30], np.float32))
    assert list(got) == [0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0x80]
    # halfway between 448 and the next (absent) step still saturates to 448
    assert encode_e4m3fn(np.array([464.0], np.float32))[0] == 0x7E


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e30, 1000),
                        rng.normal(0, 1e-38, 1000)]).astype(np.float32)
    # exact ties: bf16 values plus half an ulp
    base = torch.from_numpy(rng.normal(0, 1, 1000).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, [0.0, -0.0, np.inf, -np.inf]]).astype(np.float32)
    ours = encode_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    assert np.isnan(bf16_to_f64(encode_bf16(np.array([np.nan], np.float32)))).all()


def test_cache_write_rows_and_skips():
    rng = np.random.default_rng(13)
    pool = rng.integers(0, 256, (10, 576), dtype=np.uint8)
    kv_c = rng.normal(0, 3, (4, 512)).astype(np.float32)
    k_pe = rng.normal(0, 3, (4, 64)).astype(np.float32)
    out = cache_write(pool, kv_c, k_pe, [7, -1, 2, 10], "fp8", kv_scale=0.5)
    assert (out[7] == encode_e4m3fn(np.concatenate([kv_c[0], k_pe[0]]) / np.float32(0.5))).all()
    assert (out[2, 512:] == encode_e4m3fn(k_pe[2] / np.float32(0.5))).all()
    untouched = [i for i in range(10) if i not in (7, 2)]
    assert (out[untouched] == pool[untouched]).all()
    # decoding what was written gives the source back within half an fp8 step
    dec = e4m3fn_to_f64(out[7]) * 0.5
    src = np.concatenate([kv_c[0], k_pe[0]]).astype(np.float64)
    assert (np.abs(dec - src) <= np.abs(src) * 2.0 ** -4 + 2.0 ** -10).all()

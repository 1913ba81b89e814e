"""Pins of the 8-bit cache oracle (R22-R24) against the E4M3 field definition, torch's own
float8_e4m3fn conversion (a library routine), rounding and error bounds, and the 16-bit
compaction and decode oracles."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8

ALL = np.arange(256)


def test_known_codes():
    """Values the E4M3 definition fixes: 1.0, the extremes of each range, NaN and -0."""
    cases = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0x0F: 1.875 * 2.0 ** -6, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5}
    for c, v in cases.items():
        assert fp8.e4m3_decode(c) == v, hex(c)
    assert math.isnan(fp8.e4m3_decode(0x7F)) and math.isnan(fp8.e4m3_decode(0xFF))
    z = fp8.e4m3_decode(0x80)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    finite = fp8.e4m3_decode(ALL)
    assert np.sum(np.isnan(finite)) == 2 and np.nanmax(finite) == 448.0


def test_decode_matches_torch_float8():
    t = torch.tensor(ALL, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    d = fp8.e4m3_decode(ALL)
    assert np.array_equal(np.isnan(t), np.isnan(d))
    ok = ~np.isnan(d)
    assert np.array_equal(t[ok], d[ok]) and np.array_equal(np.signbit(t[ok]), np.signbit(d[ok]))


def test_encode_matches_torch_float8():
    """torch's round-to-nearest-even cast, on magnitudes from the subnormals to 448."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200_000) * np.exp2(rng.uniform(-14, 9, 200_000))
    x = np.clip(x, -448, 448).astype(np.float32)
    mids = (fp8._POS[:-1] + fp8._POS[1:]) / 2                 # exact ties, both signs
    x = np.concatenate([x, mids.astype(np.float32), -mids.astype(np.float32), np.float32([0.0, -0.0, 1e-30, -1e-30])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x), ref)


def test_round_trip_every_code():
    ok = ~np.isnan(fp8.e4m3_decode(ALL))
    codes = ALL[ok]
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_ties_go_to_the_even_code():
    for c in range(0x7E):
        mid = (fp8.e4m3_decode(c) + fp8.e4m3_decode(c + 1)) / 2
        want = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(mid) == want
        assert fp8.e4m3_encode(-mid) == want | 0x80


def test_saturation_and_monotonicity():
    assert fp8.e4m3_encode(1e6) == 0x7E and fp8.e4m3_encode(-464.0) == 0xFE and fp8.e4m3_encode(449) == 0x7E
    grid = np.linspace(0, 500, 200_001)
    v = fp8.e4m3_decode(fp8.e4m3_encode(grid))
    assert np.all(np.diff(v) >= 0)


def test_rounding_error_bound():
    """Half a unit in the last place: 2^-4 relative for normals, 2^-10 absolute below 2^-6."""
    rng = np.random.default_rng(3)
    x = rng.uniform(-448, 448, 100_000) * np.exp2(-rng.integers(0, 16, 100_000))
    err = np.abs(fp8.e4m3_decode(fp8.e4m3_encode(x)) - x)
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4)
    assert np.all(err[~normal] <= 2.0 ** -10)


def test_quantize_rows():
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((64, 8, 128)) * 3).to(torch.bfloat16).float().numpy()
    x[5, 2] = 0.0                                   # a zero row
    x[6, 1] = np.float32(2.0 ** -113) * np.sign(x[6, 1])   # below the smallest live row
    x[7, 3] *= np.float32(2.0 ** -108)              # small but live
    codes, scale = fp8.quantize_rows(x)
    assert codes.shape == x.shape and scale.shape == x.shape[:2] and scale.dtype == np.float32
    for z in ((5, 2), (6, 1)):
        assert scale[z] == 0 and not codes[z].any()
    amax = np.abs(x).max(-1)
    live = amax >= 2.0 ** -112
    assert live.sum() == 64 * 8 - 2
    assert np.array_equal(scale[live], (amax[live] / np.float32(448)).astype(np.float32))
    # the largest element of each row lands on +-448 (rounding moves it by far less than an ulp)
    top = np.take_along_axis(codes, np.abs(x).argmax(-1)[..., None], -1)[..., 0]
    assert np.all((top[live] & 0x7F) == 0x7E)
    y = fp8.dequantize_rows(codes, scale)
    tiny = np.abs(x) < scale[..., None].astype(np.float64) * 2.0 ** -6
    bound = np.where(tiny, scale[..., None] * 2.0 ** -10, np.abs(x) * 2.0 ** -4) * (1 + 1e-6)
    assert np.all(np.abs(y - x)[live] <= bound[live])
    # the code is the E4M3 rounding of the float32 product x * fp32(448 / amax)
    r = (np.float32(448) / amax[live]).astype(np.float32)
    assert np.array_equal(codes[live], fp8.e4m3_encode((x[live] * r[:, None]).astype(np.float32)))


def test_exact_values_survive_quantization():
    """Rows that are E4M3 values times a power of two, with 448 at the top, come back exactly."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7E, (40, 4, 64))
    codes[:, :, 0] = 0x7E
    signs = np.where(rng.random(codes.shape) < 0.5, 0x80, 0)
    x = fp8.e4m3_decode(codes | signs) * 2.0 ** -5
    c, s = fp8.quantize_rows(x)
    assert np.all(s == np.float32(448 * 2.0 ** -5 / 448)) and np.array_equal(fp8.dequantize_rows(c, s), x)


def test_compaction_is_quantized_plain_compaction():
    """The 8-bit compaction reads back as the quantized rows of the 16-bit compaction."""
    rng = np.random.default_rng(2)
    n, hkv, d, keep_n = 70, 2, 32, 37
    k = torch.from_numpy(rng.standard_normal((n, hkv, d))).to(torch.bfloat16).float().numpy()
    v = torch.from_numpy(rng.standard_normal((n, hkv, d))).to(torch.bfloat16).float().numpy()
    keep = np.stack([np.sort(rng.choice(n, keep_n, replace=False)) for _ in range(hkv)])
    table = [9, 3, 0, 6]
    pk = np.zeros((10, hkv, 16, d)); pv = np.zeros_like(pk)
    oracle.compact_into_pool(k, v, keep, table, pk, pv, off=5)
    qk = np.zeros((10, hkv, 16, d), np.uint8); qv = np.zeros_like(qk)
    sk = np.zeros((10, hkv, 16), np.float32); sv = np.zeros_like(sk)
    fp8.compact_into_pool_fp8(k, v, keep, table, qk, qv, sk, sv, off=5)
    L = 5 + keep_n
    plain_k = oracle.gather_rows(pk, table, L)[5:]
    plain_v = oracle.gather_rows(pv, table, L)[5:]
    assert np.array_equal(fp8.gather_rows_fp8(qk, sk, table, L)[5:], fp8.dequantize_rows(*fp8.quantize_rows(plain_k)))
    assert np.array_equal(fp8.gather_rows_fp8(qv, sv, table, L)[5:], fp8.dequantize_rows(*fp8.quantize_rows(plain_v)))


def test_decode_on_exact_rows_equals_plain_decode():
    """When every cached row is exact at 8 bits, the 8-bit cache decodes like the 16-bit one."""
    rng = np.random.default_rng(4)
    L, hkv, G, d = 45, 2, 4, 64
    def exact_rows(m):
        c = rng.integers(0, 0x7E, (m, hkv, d)); c[..., 3] = 0x7E
        return fp8.e4m3_decode(c | np.where(rng.random(c.shape) < 0.5, 0x80, 0)) * 2.0 ** -8
    k, v = exact_rows(L), exact_rows(L)
    q = rng.standard_normal((hkv * G, d))
    table = [4, 1, 7]
    qk = np.zeros((8, hkv, 16, d), np.uint8); qv = np.zeros_like(qk)
    sk = np.zeros((8, hkv, 16), np.float32); sv = np.zeros_like(sk)
    fp8.compact_into_pool_fp8(k[:-1], v[:-1], None, table, qk, qv, sk, sv)
    fp8.append_row_fp8(qk, qv, sk, sv, table, L - 1, k[-1], v[-1])
    o8, l8 = oracle.decode_attention(q, fp8.gather_rows_fp8(qk, sk, table, L), fp8.gather_rows_fp8(qv, sv, table, L))
    o, l = oracle.decode_attention(q, k, v)
    assert np.array_equal(o8, o) and np.array_equal(l8, l)

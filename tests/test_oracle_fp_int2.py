"""Pins for the oracle's storage rounding and INT2 quantiser (CPU only).

Each check compares the oracle with something it does not use itself: torch's bf16 conversion, an exhaustive
table of every finite fp16 value, exact rational arithmetic, hand-worked bit patterns, and closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import fp, int2

ALL_F16 = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
FINITE_F16 = np.unique(ALL_F16[np.isfinite(ALL_F16)].astype(np.float64))  # sorted, -0 merged into 0


def brute_round_down(x):
    i = np.searchsorted(FINITE_F16, x, side="right") - 1
    return FINITE_F16[i]


def brute_round_up(x):
    i = np.searchsorted(FINITE_F16, x, side="left")
    return FINITE_F16[i]


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(fp.storage_to_f32(bits, "bf16"))]
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(fp.storage_to_f32(bits, "bf16"), ref)


def test_bf16_rne_matches_torch_including_ties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50000).astype(np.float32) * np.float32(10.0)
    # exact halfway cases: bf16 value plus half an ulp, both parities of the kept lsb
    base = (rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | 0x8000
    ties = base.view(np.float32)
    ties = ties[np.isfinite(ties)]
    for arr in (x, ties):
        ref = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(fp.f32_to_bf16_rne(arr), ref)


def test_f16_directed_rounding_against_exhaustive_table():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000) * 4, rng.standard_normal(2000) * 1e-5,
                        rng.uniform(-60000, 60000, 2000), FINITE_F16[::97][1:-1]]).astype(np.float32)
    x = x[np.abs(x) < 65504]
    down = fp.f16_round_down(x).astype(np.float64)
    up = fp.f16_round_up(x).astype(np.float64)
    np.testing.assert_array_equal(down, brute_round_down(x.astype(np.float64)))
    np.testing.assert_array_equal(up, brute_round_up(x.astype(np.float64)))


def test_pack_bit_positions_hand_worked():
    codes = np.array([[1, 2, 3, 0, 3, 3, 3, 3]], np.uint8)
    # byte 0 = 1 | 2<<2 | 3<<4 | 0<<6 = 0x39 ; byte 1 = 0xFF
    np.testing.assert_array_equal(int2.pack_codes(codes), np.array([[0x39, 0xFF]], np.uint8))
    np.testing.assert_array_equal(int2.unpack_codes(int2.pack_codes(codes)), codes)
    s = np.array([1.5], np.float16)
    z = np.array([-2.0], np.float16)
    # fp16 1.5 = 0x3E00, -2.0 = 0xC000 -> word 0xC0003E00
    assert int(int2.pack_meta(s, z)[0]) == 0xC0003E00
    s2, z2 = int2.unpack_meta(int2.pack_meta(s, z))
    assert s2[0] == s[0] and z2[0] == z[0]


def _exact_check(bits, dtype):
    codes, s16, z16 = int2.quantize(bits, dtype)
    x = fp.storage_to_f32(bits, dtype).astype(np.float64)
    G = x.shape[-1] // 32
    xg = x.reshape(x.shape[:-1] + (G, 32))
    cg = codes.reshape(xg.shape).astype(np.float64)
    s = s16.astype(np.float64)[..., None]
    z = z16.astype(np.float64)[..., None]
    lo, hi = xg.min(-1), xg.max(-1)
    # z: largest fp16 <= lo; s: smallest fp16 >= fl32(fl32(hi - z)/3) (0 iff hi == z)
    np.testing.assert_array_equal(z[..., 0], brute_round_down(lo))
    t = ((hi.astype(np.float32) - z[..., 0].astype(np.float32)).astype(np.float32) / np.float32(3)).astype(
        np.float64)
    flat = hi == z[..., 0]
    np.testing.assert_array_equal(s[..., 0][~flat], brute_round_up(t[~flat]))
    assert np.all(s[..., 0][flat] == 0)
    # codes = nearest level to d = fl32(x - z), ties upward (written as an argmin over the four levels)
    d = (xg.astype(np.float32) - z.astype(np.float32)).astype(np.float64)
    levels = np.arange(4, dtype=np.float64)
    dist = np.abs(d[..., None] - levels * s[..., None])
    best = 3 - np.argmin(dist[..., ::-1], axis=-1)  # argmin with ties resolved to the larger level
    best = np.where(s == 0, 0, best)
    np.testing.assert_array_equal(cg, best)
    # error bound |x - (c s + z)| <= s/2 + |fl32(x - z) - (x - z)| (exact in fp64)
    err = np.abs(xg - (cg * s + z))
    slack = np.abs(d - (xg - z))
    assert np.all(err <= s / 2 + slack)
    # dequantisation: c*s + z is exact in fp64 (checked with rationals), so one cast to fp32 is the fma
    xr = int2.dequantize(codes, s16, z16).reshape(xg.shape)
    flat_c, flat_s, flat_z = cg.reshape(-1)[:64], np.broadcast_to(s, cg.shape).reshape(-1)[:64], \
        np.broadcast_to(z, cg.shape).reshape(-1)[:64]
    for c_, s_, z_ in zip(flat_c, flat_s, flat_z):
        assert Fraction(c_) * Fraction(s_) + Fraction(z_) == Fraction(float(c_ * s_ + z_))
    np.testing.assert_array_equal(xr, (cg * s + z).astype(np.float32))
    return codes, s16, z16


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_int2_quantiser_normal_rows(dtype):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    from oracle.fp import f32_to_storage_rne
    _exact_check(f32_to_storage_rne(x, dtype), dtype)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.sampled_from(["bf16", "f16"]), st.floats(1e-3, 100.0),
       st.floats(-50.0, 50.0))
def test_int2_quantiser_random_scales(seed, dtype, scale, shift):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((4, 128)) * scale + shift).astype(np.float32)
    from oracle.fp import f32_to_storage_rne
    _exact_check(f32_to_storage_rne(x, dtype), dtype)


def test_int2_exact_grid_round_trips():
    # values exactly on z + k*s with both ends present: lo = z, hi = z + 3s, t = s exactly
    rng = np.random.default_rng(4)
    z, s = np.float16(-1.5), np.float16(0.25)
    k = rng.integers(0, 4, size=(8, 4, 32))
    k[..., 0], k[..., 1] = 0, 3
    x = (np.float64(z) + k * np.float64(s)).astype(np.float16).reshape(8, 128)
    bits = x.view(np.uint16)
    codes, s16, z16 = int2.quantize(bits, "f16")
    np.testing.assert_array_equal(codes.reshape(8, 4, 32), k)
    assert np.all(s16 == s) and np.all(z16 == z)
    np.testing.assert_array_equal(int2.dequantize(codes, s16, z16), x.astype(np.float32))


def test_int2_constant_group():
    x = np.full((2, 128), 0.375, np.float16)
    codes, s16, z16 = int2.quantize(x.view(np.uint16), "f16")
    assert np.all(codes == 0) and np.all(s16 == 0) and np.all(z16 == np.float16(0.375))
    np.testing.assert_array_equal(int2.dequantize(codes, s16, z16), x.astype(np.float32))


def test_int2_two_valued_group():
    # two values a < b: z = a (fp16-representable), s = fl16up((b - a)/3), codes 0 or 3 unless 3s overshoots
    x = np.where(np.arange(128) % 2 == 0, np.float16(-0.5), np.float16(1.0)).astype(np.float16)[None]
    codes, s16, z16 = int2.quantize(x.view(np.uint16), "f16")
    assert np.all(z16 == np.float16(-0.5)) and np.all(s16 == np.float16(0.5))
    np.testing.assert_array_equal(codes[0], np.where(np.arange(128) % 2 == 0, 0, 3))

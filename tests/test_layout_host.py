"""The host-side layout conversions agree with the storage layouts include/kvc.h documents (hand-worked
positions) and round-trip."""
import numpy as np

from kv_cache_compression_gqa_amd import layout


def test_k_codes_documented_position():
    codes = np.zeros((32, 128), np.uint8)
    # head_dim 32g + 8s + 4h + e = 32*2 + 8*1 + 4*1 + 3 = 79 -> byte 8*1 + 2*2 + 1 = 13, bits 6..7
    codes[5, 79] = 3
    b = layout.k_codes_to_lib(codes)
    assert b.shape == (32, 32)
    assert b[5, 13] == 3 << 6 and b.sum() == 3 << 6
    rng = np.random.default_rng(0)
    c = rng.integers(0, 4, (3, 32, 128)).astype(np.uint8)
    np.testing.assert_array_equal(layout.k_codes_from_lib(layout.k_codes_to_lib(c)), c)


def test_v_codes_documented_position():
    codes = np.zeros((32, 128), np.uint8)
    # token 8q + e = 8*2 + 5 = 21, head_dim 16dt + r = 16*6 + 9 = 105 -> word (9, 2, 6), bits 10..11
    codes[21, 105] = 2
    wd = layout.v_codes_to_lib(codes)
    assert wd.shape == (16, 4, 8)
    assert wd[9, 2, 6] == 2 << 10 and int(wd.astype(np.int64).sum()) == 2 << 10
    rng = np.random.default_rng(1)
    c = rng.integers(0, 4, (2, 32, 128)).astype(np.uint8)
    np.testing.assert_array_equal(layout.v_codes_from_lib(layout.v_codes_to_lib(c)), c)


def test_meta_and_transposes():
    s = np.full((32, 4), np.float16(0.5))
    z = np.full((32, 4), np.float16(-1.0))
    s[19, 2] = np.float16(2.0)                 # token 19 = 8*2 + 3, group 2 -> v word (2, 2, 3)
    vm = layout.v_meta_to_lib(s, z)
    assert vm.shape == (4, 4, 8)
    assert vm[2, 2, 3] == (0x4000 | (0xBC00 << 16))
    assert layout.k_meta_to_lib(s, z)[19, 2] == (0x4000 | (0xBC00 << 16))
    v = np.arange(2 * 32 * 128, dtype=np.uint16).reshape(2, 32, 128)
    vt = layout.v_win_to_lib(v)
    assert vt[1, 7, 3] == v[1, 3, 7]
    np.testing.assert_array_equal(layout.v_win_from_lib(vt), v)
    tail = np.arange(64 * 128, dtype=np.uint16).reshape(64, 128)
    tl = layout.v_tail_to_lib(tail)
    assert tl.shape == (2, 128, 32) and tl[1, 5, 2] == tail[34, 5]
    np.testing.assert_array_equal(layout.v_tail_from_lib(tl), tail)

"""Pins for the oracle's pool layout: every index map is a bijection onto its block, and
token writes round-trip without disturbing neighbours (two V tokens share each byte)."""
import numpy as np

from oracle import layout


def _check_bijection(fn, kind, n_bytes, nibbles):
    o = np.repeat(np.arange(16), 128)
    d = np.tile(np.arange(128), 16)
    if nibbles:
        b, nib = fn(kind, o, d)
        key = b * 2 + nib
        assert key.min() == 0 and key.max() == n_bytes * 2 - 1
        assert np.unique(key).size == n_bytes * 2
    else:
        b = fn(kind, o, d)
        assert b.min() == 0 and b.max() == n_bytes - 1
        assert np.unique(b).size == n_bytes


def test_nvfp4_data_maps_are_bijections():
    for kind in ("k", "v"):
        _check_bijection(layout._idx_nvfp4_data, kind, layout.NVFP4_DATA_BYTES, True)


def test_nvfp4_scale_maps_are_bijections():
    for kind in ("k", "v"):
        o = np.repeat(np.arange(16), 8)
        j = np.tile(np.arange(8), 16)
        b = layout._idx_nvfp4_scale(kind, o, j)
        assert np.unique(b).size == 128 and b.min() == 0 and b.max() == 127


def test_fp8_maps_are_bijections():
    for kind in ("k", "v"):
        _check_bijection(layout._idx_fp8, kind, layout.FP8_BYTES, False)


def test_nvfp4_write_read_round_trip_and_neighbours_untouched():
    rng = np.random.default_rng(7)
    pages, h = 12, 3
    for kind in ("k", "v"):
        dshape, sshape = layout.nvfp4_pool_shapes(pages, h)
        data = rng.integers(0, 256, size=dshape).astype(np.uint8)
        scale = rng.integers(0, 256, size=sshape).astype(np.uint8)
        slots = rng.choice(pages * 16, size=70, replace=False)
        codes = rng.integers(0, 16, size=(70, h, 128)).astype(np.uint8)
        sb = rng.integers(0, 256, size=(70, h, 8)).astype(np.uint8)
        before_c, before_s = layout.read_nvfp4_tokens(data, scale, kind, np.arange(pages * 16))
        layout.write_nvfp4_tokens(data, scale, kind, slots, codes, sb)
        c2, s2 = layout.read_nvfp4_tokens(data, scale, kind, slots)
        assert np.array_equal(c2, codes) and np.array_equal(s2, sb)
        others = np.setdiff1d(np.arange(pages * 16), slots)
        c3, s3 = layout.read_nvfp4_tokens(data, scale, kind, others)
        assert np.array_equal(c3, before_c[others]) and np.array_equal(s3, before_s[others])


def test_fp8_write_read_round_trip():
    rng = np.random.default_rng(8)
    for kind in ("k", "v"):
        cache = rng.integers(0, 256, size=layout.fp8_pool_shape(5, 2)).astype(np.uint8)
        slots = rng.choice(80, size=33, replace=False)
        codes = rng.integers(0, 256, size=(33, 2, 128)).astype(np.uint8)
        layout.write_fp8_tokens(cache, kind, slots, codes)
        assert np.array_equal(layout.read_fp8_tokens(cache, kind, slots), codes)


def test_sequence_slots_follow_page_table():
    pt = np.array([7, 2, 9])
    s = layout.sequence_slots(pt, 35)
    assert s[0] == 7 * 16 and s[15] == 7 * 16 + 15 and s[16] == 2 * 16 and s[34] == 9 * 16 + 2

"""Pins for the oracle's E2M1 / E4M3 codecs against facts fixed outside the oracle.

* the E2M1 grid and bit layout printed for the format (tests/golden/format_facts.json);
* the hand-derived RNE threshold table (tests/golden/e2m1_rne_thresholds.txt);
* torch's float8_e4m3fn casts (a library routine with OCP E4M3 semantics:
  RNE, finite values up to 448, and saturation to 448 up to 464).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLD, "format_facts.json")) as f:
        return json.load(f)


def _thresholds():
    rows = []
    with open(os.path.join(GOLD, "e2m1_rne_thresholds.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lo, loc, hi, hic, mag, code = line.split()
            rows.append((float(lo), loc == "1", float(hi), hic == "1", float(mag), int(code)))
    return rows


def test_e2m1_decode_all_16_codes_match_grid_with_sign():
    mags = _facts()["e2m1_magnitudes"]["values"]
    for code in range(16):
        want = mags[code & 7] * (-1.0 if code & 8 else 1.0)
        got = codecs.e2m1_decode(np.array([code]))[0]
        assert got == want
        if code & 8:
            assert np.signbit(got) or want == 0
    # negative zero decodes to a zero
    assert codecs.e2m1_decode(np.array([8]))[0] == 0.0


def test_e2m1_bit_layout_one_two_one():
    f = _facts()["e2m1_bits"]
    assert (f["sign"], f["exponent"], f["mantissa"]) == (1, 2, 1)
    # the code's bit 3 is the sign: code and code|8 differ only in sign
    for c in range(8):
        assert codecs.e2m1_decode(np.array([c | 8]))[0] == -codecs.e2m1_decode(np.array([c]))[0]


def test_e2m1_encode_matches_threshold_table_on_dense_sweep():
    rng = np.random.default_rng(0)
    pts = [np.linspace(0, 8, 200001, dtype=np.float32)]
    # every boundary +- a few ulps
    for lo, _, hi, _, _, _ in _thresholds():
        for b in (lo, hi):
            if np.isfinite(b):
                v = np.float32(b)
                ups = [v]
                up = dn = v
                for _ in range(4):
                    up = np.nextafter(up, np.float32(np.inf))
                    dn = np.nextafter(dn, np.float32(0))
                    ups += [up, dn]
                pts.append(np.array(ups, dtype=np.float32))
    pts.append(rng.uniform(0, 10, 100000).astype(np.float32))
    pts.append(np.array([np.inf, 1e30, 6.0, 7.0, 1e-45], dtype=np.float32))
    y = np.abs(np.concatenate(pts))
    got = codecs.e2m1_encode_magnitude(y)
    want = np.full(y.shape, 255, dtype=np.int64)
    for lo, loc, hi, hic, _, code in _thresholds():
        above = (y >= lo) if loc else (y > lo)
        below = (y <= hi) if hic else (y < hi)
        m = above & below
        assert np.all(want[m] == 255), "threshold table rows overlap"
        want[m] = code
    assert np.all(want != 255), "threshold table leaves a gap"
    np.testing.assert_array_equal(got, want)


def test_e2m1_round_trip_of_representable_values():
    mags = np.array(_facts()["e2m1_magnitudes"]["values"], dtype=np.float32)
    assert np.array_equal(codecs.e2m1_encode_magnitude(mags), np.arange(8))


def test_e4m3_decode_matches_torch_float8_e4m3fn_all_bytes():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.e4m3_decode(np.arange(256))
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(ours[~nan], t[~nan])
    assert codecs.E4M3_MAX == _facts()["e4m3_max"]["value"] == 448.0
    assert ours[1] == 2.0 ** -9  # smallest subnormal


def _e4m3_sweep():
    rng = np.random.default_rng(1)
    vals = codecs.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = [vals, mids]
    for m in mids.astype(np.float32):
        a = b = m
        for _ in range(3):
            a = np.nextafter(a, np.float32(np.inf))
            b = np.nextafter(b, np.float32(0))
            pts.append(np.array([a, b]))
    pts.append(np.exp(rng.uniform(np.log(2.0 ** -14), np.log(464.0), 200000)))
    pts.append(np.array([0.0, 2.0 ** -10, 2.0 ** -11, 448.0, 460.0, 464.0]))
    x = np.concatenate(pts).astype(np.float32)
    x = x[(x <= 464.0)]
    return np.concatenate([x, -x])


def test_e4m3_encode_matches_torch_cast_up_to_464():
    x = _e4m3_sweep()
    ours = codecs.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_encode_saturates_beyond_448():
    x = np.array([465.0, 480.0, 1e6, np.inf, -500.0, -np.inf], dtype=np.float32)
    np.testing.assert_array_equal(codecs.e4m3_encode(x), [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])


def test_e4m3_encode_keeps_sign_of_zero():
    x = np.array([-0.0, 0.0, -(2.0 ** -12)], dtype=np.float32)
    np.testing.assert_array_equal(codecs.e4m3_encode(x), [0x80, 0x00, 0x80])


def test_codecs_reject_nan():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([np.nan], dtype=np.float32))
    with pytest.raises(ValueError):
        codecs.e2m1_encode_magnitude(np.array([np.nan], dtype=np.float32))

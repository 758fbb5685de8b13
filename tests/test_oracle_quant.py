"""Pins for the oracle's NVFP4 / FP8 quantization against facts fixed outside the oracle.

* hand-worked blocks (tests/golden/nvfp4_worked_blocks.json);
* the closed-form exact round trip of representable values;
* the scale invariants implied by g = amax / (6 * 448);
* the 9-bytes-per-16-values ledger (tests/golden/format_facts.json);
* FP8: torch's float8_e4m3fn cast of x / s and a hand-worked example.
"""
import json
import os

import numpy as np
import torch

from oracle import codecs, fp8, nvfp4

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "nvfp4_worked_blocks.json")) as f:
        return json.load(f)


def test_hand_worked_blocks():
    for b in _gold()["blocks"]:
        codes, sb = nvfp4.quantize_blocks(np.array(b["x"], dtype=np.float32), np.float32(b["g"]))
        assert codes.tolist() == b["codes"], b["name"]
        assert int(sb[0]) == b["scale_byte"], b["name"]


def test_hand_worked_fp8():
    f = _gold()["fp8"]
    got = fp8.fp8_quantize(np.array(f["x"], dtype=np.float32), np.float32(f["s"]))
    assert got.tolist() == f["bytes"]


def test_exact_round_trip_of_representable_blocks():
    """g = 2^k, codes c with max |c| = 6, any finite positive E4M3 scale s: x = c s g is
    exactly representable (<= 6 significant bits), and quantization must return s and c."""
    rng = np.random.default_rng(2)
    pos_scales = np.arange(1, 0x7F)          # every nonzero finite E4M3 scale byte
    for k in (-12, -8, -3, 0, 4):
        g = np.float32(2.0 ** k)
        n = pos_scales.size
        codes = rng.integers(0, 16, size=(n, 16)).astype(np.uint8)
        pin = rng.integers(0, 16, size=n)
        codes[np.arange(n), pin] = np.where(rng.random(n) < 0.5, 7, 15)   # a +-6 in every block
        s = codecs.e4m3_decode(pos_scales)
        x = codecs.e2m1_decode(codes) * s[:, None] * float(g)
        x32 = x.astype(np.float32)
        assert np.array_equal(x32.astype(np.float64), x)                  # exact in fp32
        # and in bf16 (the method's input type)
        xb = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(xb, x)
        got_codes, got_sb = nvfp4.quantize_blocks(x32, g)
        np.testing.assert_array_equal(got_sb[:, 0], pos_scales)
        # zero codes: the sign of a signed zero survives only if x kept it
        want = codes.copy()
        np.testing.assert_array_equal(got_codes, want)


def test_amax_block_gets_scale_448_and_all_scales_bounded():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 8, 128)) * np.exp(rng.uniform(np.log(0.1), np.log(10), (1, 8, 128)))).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    g = nvfp4.global_scale(x)
    assert g == np.float32(np.float32(np.abs(x).max()) / np.float32(2688.0))
    codes, sb = nvfp4.quantize_blocks(x, g)
    s = codecs.e4m3_decode(sb)
    assert s.max() == 448.0
    flat = np.abs(x).reshape(-1, 16).max(axis=1)
    assert s.reshape(-1)[np.argmax(flat)] == 448.0
    assert np.all(s <= 448.0)
    # every non-saturated element is within half a grid step of x / (s g)
    xh = nvfp4.dequantize_blocks(codes, sb, g)
    sg = np.repeat((s * float(g)).reshape(x.shape[:-1] + (8,)), 16, axis=-1)
    y = np.abs(x.astype(np.float64)) / sg
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(x.astype(np.float64) - xh) / sg
    assert np.all(err[y <= 6] <= step[y <= 6] / 2 * (1 + 1e-6))


def test_dequantize_is_code_times_scale_times_g():
    codes = np.arange(16, dtype=np.uint8)[None, :]
    sb = np.array([[0x71]], dtype=np.uint8)  # 144
    g = np.float32(0.25)
    want = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6]) * 144 * 0.25
    np.testing.assert_array_equal(nvfp4.dequantize_blocks(codes, sb, g)[0], want)


def test_storage_ledger_nine_bytes_per_sixteen():
    f = json.load(open(os.path.join(GOLD, "format_facts.json")))
    assert nvfp4.bytes_per_values(16) == f["bytes_per_16_values"]["total"] == 9
    n = 128 * 16  # one page of one head
    frac = nvfp4.bytes_per_values(n) / n          # FP8 takes 1 byte per value
    assert frac == f["fraction_of_fp8"]["value"]
    assert abs(1 / frac - f["capacity_ratio_vs_fp8_approx"]["value"]) < f["capacity_ratio_vs_fp8_approx"]["tolerance"]


def test_pack_nibbles_low_first_and_inverse():
    c = np.arange(16, dtype=np.uint8)
    p = nvfp4.pack_nibbles(c)
    assert p.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(nvfp4.unpack_nibbles(p), c)


def test_fp8_quantize_matches_torch_cast_of_quotient():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    s = fp8.fp8_scale(x)
    q = (x / s).astype(np.float32)
    assert np.abs(q).max() <= 448.0 * (1 + 1e-6)
    ref = torch.from_numpy(np.clip(q, -464, 464)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.fp8_quantize(x, s), ref)
    # round trip of representable values
    vals = codecs.e4m3_decode(np.arange(0x7F)) * float(s)
    np.testing.assert_array_equal(fp8.fp8_quantize(vals.astype(np.float32), s), np.arange(0x7F))


def test_workspace_transcode_exact_when_representable():
    """With g = 2^k, power-of-two block scales and s_ws = g, the workspace value
    v / s_ws = e2m1 * s_blk is an E4M3 value, so the transcode is lossless."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(50, 128)).astype(np.uint8)
    pow2_bytes = np.array([b for b in range(1, 0x7F) if (b & 7) == 0 and 2.0 ** -3 <= codecs.e4m3_decode([b])[0] <= 32])
    sb = rng.choice(pow2_bytes, size=(50, 8)).astype(np.uint8)
    g = np.float32(2.0 ** -6)
    w = fp8.nvfp4_to_fp8_workspace(codes, sb, g, g)
    want = nvfp4.dequantize_blocks(codes, sb, g) / float(g)
    got = codecs.e4m3_decode(w)
    np.testing.assert_array_equal(got, want)
    # signs follow the E2M1 code (including signed zeros)
    assert np.array_equal(w >> 7, codes >> 3)


def test_workspace_transcode_equals_fp8_quantize_of_fp32_dequant():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((40, 128)) * 2).astype(np.float32)
    g = nvfp4.global_scale(x)
    codes, sb = nvfp4.quantize_blocks(x, g)
    s_ws = np.float32(6.0) * g
    w = fp8.nvfp4_to_fp8_workspace(codes, sb, g, s_ws)
    v = nvfp4.dequantize_blocks(codes, sb, g).astype(np.float32)   # fp64 exact -> fp32 is one rounding
    ref = fp8.fp8_quantize(v, s_ws)
    nz = (codes & 7) != 0
    np.testing.assert_array_equal(w[nz], ref[nz])

"""Pins for the fp32 roundings the oracle's readings fix, against hand-worked cases.

Each case in tests/golden/nvfp4_rounding_cases.json was worked with exact rational arithmetic and
sits right next to a rounding boundary, so that the result depends on where the readings put the
fp32 roundings:

* the block scale s = E4M3(fp32(a / fp32(6 g))) -- rounding 6 g first moves a / (6 g) across an
  E4M3 midpoint (SGLang x Qwen x NVIDIA story, "The Core of the Ledger" paragraph 1);
* the element code E2M1(fp32(x / fp32(s g))) -- rounding s g first moves x / (s g) across an E2M1
  threshold (same passage; SOAR Notes 05, "02 NVFP4 KV Cache");
* the workspace byte E4M3(fp32(fp32(fp32(e2m1 s) g) / s_ws)) -- rounding the dequantized value first
  decides a tie ("Three Paths" paragraph 2);
* the per-tensor FP8 scale fp32(amax / 448), which puts the amax element on 0x7E, the OCP E4M3
  maximum (SOAR Notes 05, "03 Mixed-precision KV Cache"; 448 from the global scale amax / (6 * 448)).

The golden's stated intermediate values are re-derived here with Python fractions (exact), so a
typo in the file cannot pass; the oracle is then held to the golden's results.
"""
import json
import math
import os
from fractions import Fraction as Q

import numpy as np
import torch

from oracle import fp8, nvfp4

GOLD = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_rounding_cases.json")


def _cases():
    with open(GOLD) as f:
        return json.load(f)


def _fp32(x: Q) -> Q:
    """Exact value of the fp32 nearest to the rational x (ties to an even significand); normal range."""
    if x == 0:
        return Q(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Q(2) ** e > a:
        e -= 1
    if Q(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127
    ulp = Q(2) ** (e - 23)
    n = a / ulp
    lo = math.floor(n)
    rem = n - lo
    if rem > Q(1, 2) or (rem == Q(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * ulp


def _exact(v: float) -> Q:
    return Q(v)


def test_golden_work_is_exact_arithmetic():
    c = _cases()
    # R5: fp32(6 g) rounds down, so a / fp32(6 g) rounds above the E4M3 midpoint 29
    r5 = c["r5_block_scale"]
    g = _exact(r5["g"])
    assert g == _fp32(Q(1, 58)) == Q(9256395, 2 ** 29)
    six = _fp32(6 * g)
    assert six == _exact(0.10344827175140381) and six < 6 * g
    a = max(abs(_exact(v)) for v in r5["x"])
    assert _fp32(a / six) == _exact(29.000001907348633) > 29
    assert _fp32(a / (6 * g)) == 29
    # R6: fp32(176 g) rounds down, so 1 / fp32(176 g) lands above the E2M1 threshold 2.5
    r6 = c["r6_element_code"]
    g = _exact(r6["g"])
    assert g == _fp32(Q(1, 440))
    a = max(abs(_exact(v)) for v in r6["x"])
    u = _fp32(a / _fp32(6 * g))
    assert 168 < u < 176                      # above the 160 | 176 midpoint: s = 176
    den = _fp32(176 * g)
    assert den == _exact(0.3999999761581421) and den < 176 * g
    assert _fp32(1 / den) == _exact(2.500000238418579) > Q(5, 2)
    assert _fp32(1 / (176 * g)) == Q(5, 2)
    # R14: codes 1.5, 3, 6 under s = 128 land exactly on E4M3 midpoints only with the rounded v
    r14 = c["r14_workspace"]
    g, sws = _exact(r14["g"]), _exact(r14["s_ws"])
    assert sws == Q(15320929, 2 ** 27)
    for e, mid in ((Q(3, 2), 29), (Q(3), 58), (Q(6), 116)):
        v = _fp32(_fp32(e * 128) * g)
        assert v != e * 128 * g
        assert _fp32(v / sws) == mid
        assert _fp32(e * 128 * g / sws) > mid
    # FP8: s = fp32(5 / 448)
    f = c["fp8_per_tensor"]
    assert _exact(f["s"]) == _fp32(Q(5, 448))


def test_r5_block_scale_rounds_six_g_first():
    r5 = _cases()["r5_block_scale"]
    codes, sb = nvfp4.quantize_blocks(np.array(r5["x"], dtype=np.float32), np.float32(r5["g"]))
    assert int(sb[0]) == r5["scale_byte"] != r5["one_rounding_scale_byte"]
    assert codes.tolist() == r5["codes"]


def test_r6_element_code_rounds_s_times_g_first():
    r6 = _cases()["r6_element_code"]
    codes, sb = nvfp4.quantize_blocks(np.array(r6["x"], dtype=np.float32), np.float32(r6["g"]))
    assert int(sb[0]) == r6["scale_byte"]
    assert codes.tolist() == r6["codes"]
    assert r6["codes"] != r6["one_rounding_codes"]


def test_r14_workspace_rounds_dequantized_value_first():
    r = _cases()["r14_workspace"]
    codes = np.array([r["codes"]], dtype=np.uint8)
    w = fp8.nvfp4_to_fp8_workspace(codes, np.array([[r["scale_byte"]]], dtype=np.uint8), np.float32(r["g"]),
                                   np.float32(r["s_ws"]))
    assert w[0].tolist() == r["ws_bytes"]
    assert r["ws_bytes"] != r["one_rounding_ws_bytes"]


def test_fp8_per_tensor_scale_puts_amax_on_e4m3_max():
    f = _cases()["fp8_per_tensor"]
    # the E4M3 maximum as torch's float8_e4m3fn (the OCP variant) defines it
    assert float(torch.finfo(torch.float8_e4m3fn).max) == 448.0
    x = np.array(f["x"], dtype=np.float32)
    s = fp8.fp8_scale(x)
    assert s == np.float32(f["s"])
    got = fp8.fp8_quantize(x, s)
    assert got.tolist() == f["bytes"]
    assert got[np.argmax(np.abs(x))] == 0x7E
    assert f["divisor_240_first_bytes"][0] != 0x7E

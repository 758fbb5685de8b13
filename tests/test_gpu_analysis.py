"""GPU checks of the precision studies (studies.py, beside the bench): the per-layer sensitivity sweep
and the per-tensor scale variants, on constructed data whose answer is known."""
import numpy as np
import pytest
import torch

import workloads
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def an():
    import studies
    return studies


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _setup(seed, lens, hkv=2, hq=8):
    wl = workloads.Workload(name="study", seed=seed, batch=len(lens), h_kv=hkv, h_q=hq, seq_lens=lens, extra_pages=1)
    pt, sl = H.gpu_tables(wl, DEV)
    slots = torch.from_numpy(np.concatenate([wl.slots(b) for b in range(wl.batch)])).to(DEV)
    return wl, pt, sl, slots


def test_reference_attention_matches_oracle(an):
    """The study's fp32 torch reference agrees with the fp64 oracle on the unquantized values."""
    from oracle import attention as o_att
    wl, pt, sl, slots = _setup(41, [70, 130])
    rng = np.random.default_rng(1)
    k = _bf16(rng.standard_normal((200, 2, 128)))
    v = _bf16(rng.standard_normal((200, 2, 128)))
    q = _bf16(rng.standard_normal((2, 8, 128)))
    ref = an.attention_reference(q.to(DEV), k.to(DEV), v.to(DEV), [70, 130], 0.09).cpu().numpy()
    kn, vn = k.float().numpy(), v.float().numpy()
    want = o_att.decode_attention(q.float().numpy(), [kn[:70], kn[70:]], [vn[:70], vn[70:]], 0.09)
    np.testing.assert_allclose(ref, want, atol=2e-5, rtol=0)


def test_layer_sensitivity_finds_the_wide_range_layer(an):
    lens = [200, 333]
    wl, pt, sl, slots = _setup(42, lens)
    rng = np.random.default_rng(2)
    n = sum(lens)
    layers = []
    for i in range(4):
        k = rng.standard_normal((n, 2, 128)).astype(np.float32)
        v = rng.standard_normal((n, 2, 128)).astype(np.float32)
        if i == 2:                                  # a few huge tokens stretch this layer's per-tensor range
            k[[5, 250, 400]] *= 3000.0
            v[[7, 260, 410]] *= 3000.0
        layers.append({"q": _bf16(rng.standard_normal((2, 8, 128))).to(DEV), "k": _bf16(k).to(DEV),
                       "v": _bf16(v).to(DEV)})
    rows = an.layer_sensitivity(layers, slots, wl.num_pages, pt, sl, wl.sm_scale, 2)
    assert [r["layer"] for r in rows] == [0, 1, 2, 3]
    for r in rows:
        for key in ("nvfp4_vs_bf16", "fp8_vs_bf16", "nvfp4_vs_fp8"):
            assert np.isfinite(r[key]["rel_l2"]) and np.isfinite(r[key]["max_abs"])
    e4 = [r["nvfp4_vs_bf16"]["rel_l2"] for r in rows]
    assert int(np.argmax(e4)) == 2, e4
    for i in (0, 1, 3):       # on well-behaved layers FP8 (3 mantissa bits) is closer than NVFP4 (1 bit)
        assert rows[i]["fp8_vs_bf16"]["rel_l2"] < rows[i]["nvfp4_vs_bf16"]["rel_l2"]


def test_gscale_variants(an):
    lens = [300, 200]
    wl, pt, sl, slots = _setup(43, lens)
    rng = np.random.default_rng(3)
    n = sum(lens)
    q = _bf16(rng.standard_normal((2, 8, 128))).to(DEV)
    k = rng.standard_normal((n, 2, 128)).astype(np.float32)       # K stays N(0, 1): a mild softmax
    # (1) V of head 1 lives 1e6 x above head 0: one tensor-wide scale puts head 0's block scales
    #     below E4M3's smallest step (they round to zero); one scale per head does not
    v = rng.standard_normal((n, 2, 128)).astype(np.float32)
    v[:, 1] *= 1.0e6
    res = an.gscale_variants(q, _bf16(k).to(DEV), _bf16(v).to(DEV), slots, wl.num_pages, pt, sl, wl.sm_scale, 2,
                             calib_tokens=100)
    assert set(res) == {"tensor_amax", "calibrated_prefix", "per_head"}
    for r in res.values():
        assert np.isfinite(r["rel_l2"]) and r["decode_us"] > 0
    assert res["tensor_amax"]["rel_l2_per_kv_head"][0] > 0.9          # head 0's values quantized to zero
    assert res["per_head"]["rel_l2_per_kv_head"][0] < 0.3              # the usual NVFP4 error on random values
    # (2) V grows 30 x after the calibration prefix: the calibrated scale is smaller and the grown
    #     values saturate at 6 x 448 x g
    v2 = rng.standard_normal((n, 2, 128)).astype(np.float32)
    v2[400:] *= 30.0
    res2 = an.gscale_variants(q, _bf16(k).to(DEV), _bf16(v2).to(DEV), slots, wl.num_pages, pt, sl, wl.sm_scale, 2,
                              calib_tokens=100)
    assert res2["calibrated_prefix"]["v_gscale"] < res2["tensor_amax"]["v_gscale"]
    assert res2["calibrated_prefix"]["rel_l2"] > res2["tensor_amax"]["rel_l2"]

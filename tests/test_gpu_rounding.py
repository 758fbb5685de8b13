"""The hand-worked rounding cases (tests/golden/nvfp4_rounding_cases.json) through every writer of
the library, via the C ABI: the block scale decided by fp32(6 g), the element codes decided by
fp32(s g), the workspace bytes decided by fp32(fp32(e2m1 s) g), and the per-tensor FP8 scale that
puts the amax element on 0x7E.  The expected bytes are the golden's (worked with exact rationals),
not the oracle's."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import layout as o_layout

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLD = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_rounding_cases.json")


@pytest.fixture(scope="module")
def nv():
    import bit_paged_kv_amd as nv
    return nv


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as f:
        return json.load(f)


def _token(block, reps=8):
    """One (token, head) row of 128 channels: the 16-value block repeated; bf16-exact values."""
    x = np.tile(np.array(block, dtype=np.float32), reps)
    t = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), x)
    return t.reshape(1, 1, 128)


def _read(pool, kind, slots):
    return o_layout.read_nvfp4_tokens(pool[f"{kind}_data"].cpu().numpy(), pool[f"{kind}_scale"].cpu().numpy(), kind,
                                      slots)


def _expect(codes, sbyte, n=1):
    return np.tile(np.array(codes, dtype=np.uint8), 8)[None, None].repeat(n, 0), \
        np.full((n, 1, 8), sbyte, dtype=np.uint8)


def test_quantize_append_golden_roundings(nv, gold):
    r5, r6 = gold["r5_block_scale"], gold["r6_element_code"]
    k, v = _token(r5["x"]).to(DEV), _token(r6["x"]).to(DEV)        # K under g of R5, V under g of R6
    slots = np.array([5], dtype=np.int32)
    pool = nv.alloc_nvfp4_pool(1, 1, DEV, fill=0xA5)
    nv.nvfp4_quantize_append(k, v, torch.from_numpy(slots).to(DEV), float(r5["g"]), float(r6["g"]), pool)
    torch.cuda.synchronize()
    ck, sk = _read(pool, "k", slots)
    cv, sv = _read(pool, "v", slots)
    wk, wsk = _expect(r5["codes"], r5["scale_byte"])
    wv, wsv = _expect(r6["codes"], r6["scale_byte"])
    assert np.array_equal(sk, wsk) and np.array_equal(ck, wk)
    assert np.array_equal(sv, wsv) and np.array_equal(cv, wv)


def test_fused_append_golden_roundings(nv, gold):
    """The decode kernel's fused quantize-append of the new token (position 5 of a 6-token
    sequence) writes the same golden bytes; attention over 6 tokens still runs."""
    r5, r6 = gold["r5_block_scale"], gold["r6_element_code"]
    pool = nv.alloc_nvfp4_pool(2, 1, DEV, fill=0)
    # tokens 0..4 of the sequence: the same rows, written by the standalone writer
    k0 = _token(r5["x"]).repeat(5, 1, 1).to(DEV)
    v0 = _token(r6["x"]).repeat(5, 1, 1).to(DEV)
    pt = torch.tensor([[1]], dtype=torch.int32, device=DEV)             # the sequence lives in page 1
    nv.nvfp4_quantize_append(k0, v0, torch.arange(16, 21, dtype=torch.int32, device=DEV), float(r5["g"]),
                             float(r6["g"]), pool)
    sl = torch.tensor([6], dtype=torch.int32, device=DEV)
    q = torch.ones((1, 4, 128), dtype=torch.bfloat16, device=DEV)
    out = nv.nvfp4_decode(q, pool, float(r5["g"]), float(r6["g"]), pt, sl, 1.0 / np.sqrt(128), (2, 1), 1,
                          new_k=_token(r5["x"]).reshape(1, 1, 128).to(DEV),
                          new_v=_token(r6["x"]).reshape(1, 1, 128).to(DEV))
    torch.cuda.synchronize()
    slots = np.arange(16, 22)
    ck, sk = _read(pool, "k", slots)
    cv, sv = _read(pool, "v", slots)
    wk, wsk = _expect(r5["codes"], r5["scale_byte"], 6)
    wv, wsv = _expect(r6["codes"], r6["scale_byte"], 6)
    assert np.array_equal(sk, wsk) and np.array_equal(ck, wk)
    assert np.array_equal(sv, wsv) and np.array_equal(cv, wv)
    # every token is the same: the output is that token's dequantized V, e2m1 * 176 * g
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    codes = np.array(r6["codes"])
    vh = np.where(codes >= 8, -1.0, 1.0) * e2m1[codes & 7] * 176.0 * np.float64(np.float32(r6["g"]))
    assert np.abs(out.cpu().numpy() - np.tile(vh, 8)[None, None]).max() < 1e-5


def test_workspace_transcode_golden_roundings(nv, gold):
    r = gold["r14_workspace"]
    codes = np.tile(np.array(r["codes"], dtype=np.uint8), 8).reshape(1, 1, 128)
    sbytes = np.full((1, 1, 8), r["scale_byte"], dtype=np.uint8)
    host = {}
    dshape, sshape = o_layout.nvfp4_pool_shapes(1, 1)
    for kind in ("k", "v"):
        host[f"{kind}_data"] = np.zeros(dshape, np.uint8)
        host[f"{kind}_scale"] = np.zeros(sshape, np.uint8)
        o_layout.write_nvfp4_tokens(host[f"{kind}_data"], host[f"{kind}_scale"], kind, [3], codes, sbytes)
    pool = {k: torch.from_numpy(a).to(DEV) for k, a in host.items()}
    pt = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    prefix = torch.tensor([4], dtype=torch.int32, device=DEV)
    offs = torch.tensor([0, 4], dtype=torch.int32, device=DEV)
    kw = torch.full((4, 1, 128), 0xEE, dtype=torch.uint8, device=DEV)
    vw = kw.clone()
    g, sws = float(r["g"]), float(r["s_ws"])
    nv.dequant_to_workspace(pool, g, g, pt, prefix, offs, 4, sws, sws, 1, kw, vw)
    torch.cuda.synchronize()
    want = np.tile(np.array(r["ws_bytes"], dtype=np.uint8), 8)
    assert np.array_equal(kw.cpu().numpy()[3, 0], want)
    assert np.array_equal(vw.cpu().numpy()[3, 0], want)


def test_fp8_per_tensor_golden(nv, gold):
    f = gold["fp8_per_tensor"]
    x = np.zeros(128, dtype=np.float32)
    x[:len(f["x"])] = f["x"]
    t = torch.from_numpy(x).to(torch.bfloat16).reshape(1, 1, 128).to(DEV)
    s = nv.global_scale(t, divisor=nv.FP8_DIVISOR).item()
    assert np.float32(s) == np.float32(f["s"])
    pool = nv.alloc_fp8_pool(1, 1, DEV, fill=0x33)
    nv.fp8_quantize_append(t, t.clone(), torch.tensor([9], dtype=torch.int32, device=DEV), s, s, pool)
    torch.cuda.synchronize()
    for kind in ("k", "v"):
        got = o_layout.read_fp8_tokens(pool[kind].cpu().numpy(), kind, [9])[0, 0]
        assert got[:len(f["bytes"])].tolist() == f["bytes"]
        assert not got[len(f["bytes"]):].any()

"""GPU parity of the write side through the C ABI: bytes and scales must equal the oracle's bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import codecs as o_codecs
from oracle import fp8 as o_fp8
from oracle import layout as o_layout
from oracle import nvfp4 as o_nv
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def nv():
    import bit_paged_kv_amd as nv
    return nv


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("n", [1, 7, 16, 4093, 1 << 20])
def test_global_scale_bf16_bitexact(nv, n):
    rng = np.random.default_rng(n)
    x = _bf16(rng.standard_normal(n) * np.exp(rng.uniform(-3, 3, n)))
    if n > 4:
        x[n - 1] = -1000.0  # the maximum sits in the tail
    want = o_nv.global_scale(x.float().numpy())
    got = nv.global_scale(x.to(DEV)).item()
    assert np.float32(got) == want
    want8 = o_fp8.fp8_scale(x.float().numpy())
    got8 = nv.global_scale(x.to(DEV), divisor=448.0).item()
    assert np.float32(got8) == want8


def test_global_scale_fp8_input_bitexact(nv):
    rng = np.random.default_rng(3)
    b = rng.integers(0, 256, 10001).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x11         # no NaN patterns
    s_in = np.float32(0.37)
    x = (o_codecs.e4m3_decode(b).astype(np.float32) * s_in).astype(np.float32)
    want = o_nv.global_scale(x)
    got = nv.global_scale(torch.from_numpy(b).to(DEV), in_scale=float(s_in)).item()
    assert np.float32(got) == want


def _check_pool(got, want):
    for key in ("k_data", "k_scale", "v_data", "v_scale"):
        g = got[key].cpu().numpy()
        bad = np.argwhere(g != want[key])
        assert bad.size == 0, f"{key}: {len(bad)} bytes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("fill", [0, 0xA5])
def test_nvfp4_quantize_tiny_bitexact(nv, fill):
    wl = workloads.config(0)
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_pool(wl, ks, vs, gk, gv, fill=fill)
    pool, g_k, g_v = H.gpu_nvfp4_layer(wl, 0, DEV, fill=fill)
    assert (np.float32(g_k), np.float32(g_v)) == (gk, gv)
    _check_pool(pool, want)


def test_nvfp4_quantize_ragged_scattered_bitexact(nv):
    # several sequences, partial last pages, permuted pool with spare pages: consecutive tokens share
    # V-data bytes and are written by different threads of one launch
    wl = workloads.Workload(name="ragged-small", seed=77, batch=5, h_kv=3, h_q=6,
                            seq_lens=[1, 17, 300, 64, 95], extra_pages=7)
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_pool(wl, ks, vs, gk, gv, fill=0x5C)
    pool, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0x5C)
    _check_pool(pool, want)


@pytest.mark.parametrize("case", range(8))
def test_nvfp4_quantize_random_calls_bitexact(nv, case):
    """A cache written by many calls: every sequence is cut into random consecutive chunks (1 to 200
    tokens), the chunks are shuffled into calls of one to four chunks, and some calls list their
    tokens in a random order.  So a call meets V token quads whose other tokens are already in the
    pool, quads it completes itself, runs crossing the writer's token windows, and input orders
    unlike the slot order.  The oracle writes the same tokens at the same slots; every pool byte
    (the 0x3C fill of unused slots included) must match."""
    rng = np.random.default_rng(700 + case)
    batch = int(rng.integers(1, 9))
    h_kv = int(rng.choice([1, 2, 3, 8]))
    lens = rng.integers(1, 900, size=batch)
    wl = workloads.Workload(name=f"calls-{case}", seed=710 + case, batch=batch, h_kv=h_kv, h_q=h_kv,
                            seq_lens=lens, extra_pages=int(rng.integers(0, 4)))
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_pool(wl, ks, vs, gk, gv, fill=0x3C)
    chunks = []
    for b in range(batch):
        t = 0
        while t < lens[b]:
            n = int(min(lens[b] - t, rng.integers(1, 201)))
            chunks.append((b, t, t + n))
            t += n
    order = [int(c) for c in rng.permutation(len(chunks))]
    kb = [wl.kv("k", b) for b in range(batch)]
    vb = [wl.kv("v", b) for b in range(batch)]
    pool = nv.alloc_nvfp4_pool(wl.num_pages, h_kv, DEV, fill=0x3C)
    calls = 0
    while order:
        m = int(rng.integers(1, 5))
        sel, order = order[:m], order[m:]
        k = torch.cat([kb[chunks[c][0]][chunks[c][1]:chunks[c][2]] for c in sel])
        v = torch.cat([vb[chunks[c][0]][chunks[c][1]:chunks[c][2]] for c in sel])
        slots = np.concatenate([wl.slots(chunks[c][0], chunks[c][1], chunks[c][2]) for c in sel]).astype(np.int32)
        if rng.random() < 0.3:
            p = rng.permutation(len(slots))
            k, v, slots = k[torch.from_numpy(p)], v[torch.from_numpy(p)], slots[p]
        nv.nvfp4_quantize_append(k.contiguous().to(DEV), v.contiguous().to(DEV), torch.from_numpy(slots).to(DEV),
                                 float(gk), float(gv), pool)
        calls += 1
    torch.cuda.synchronize()
    _check_pool(pool, want)
    print(f"random calls {case}: {batch} sequences, {h_kv} kv heads, {len(chunks)} chunks in {calls} calls: "
          "every pool byte bit-exact", flush=True)


def test_nvfp4_quantize_golden_and_edge_blocks_bitexact(nv):
    """The hand-worked blocks, plus ties, saturation, subnormal and zero scales, signed zeros."""
    gold = json.load(open(os.path.join(GOLD, "nvfp4_worked_blocks.json")))["blocks"]
    rng = np.random.default_rng(5)
    g = np.float32(2.0 ** -8)
    rows = []
    for blk in gold:
        if np.float32(blk["g"]) == g:
            rows.append(np.array(blk["x"], dtype=np.float32))
    grid = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7], dtype=np.float32)
    for s in (1.0, 1.75, 448.0, 2.0 ** -9, 3 * 2.0 ** -9, 0.0):
        rows.append(np.float32(grid * s * float(g)) * np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32))
    rows.append(np.array([-0.0] * 8 + [0.0] * 8, dtype=np.float32))
    rows.append(np.float32(rng.standard_normal(16) * 1e4))            # far above 448 * 6 * g: saturates
    rows.append(np.float32(rng.standard_normal(16) * 1e-7))           # scale rounds to zero
    blocks = np.stack(rows)
    # round to bf16 (the input type) and keep those rows; 8 blocks make one token of one head
    xb = _bf16(blocks).float().numpy()
    n_tok = (xb.shape[0] + 7) // 8
    tok = np.zeros((n_tok * 8, 16), dtype=np.float32)
    tok[:xb.shape[0]] = xb
    tok = tok.reshape(n_tok, 1, 128)
    slots = np.arange(n_tok, dtype=np.int32) * 3 % (16 * 4)               # scattered in 4 pages
    dshape, sshape = o_layout.nvfp4_pool_shapes(4, 1)
    want = {k: np.zeros(s, np.uint8) for k, s in (("k_data", dshape), ("k_scale", sshape),
                                                  ("v_data", dshape), ("v_scale", sshape))}
    c, s = o_nv.quantize_blocks(tok, g)
    o_layout.write_nvfp4_tokens(want["k_data"], want["k_scale"], "k", slots, c, s)
    o_layout.write_nvfp4_tokens(want["v_data"], want["v_scale"], "v", slots, c, s)
    pool = nv.alloc_nvfp4_pool(4, 1, DEV)
    t = _bf16(tok).to(DEV)
    nv.nvfp4_quantize_append(t, t.clone(), torch.from_numpy(slots).to(DEV), float(g), float(g), pool)
    _check_pool(pool, want)
    # the hand-worked codes survive the GPU round trip too
    codes, _ = o_layout.read_nvfp4_tokens(pool["k_data"].cpu().numpy(), pool["k_scale"].cpu().numpy(), "k", slots)
    flat = codes.reshape(-1, 16)
    for i, blk in enumerate(b for b in gold if np.float32(b["g"]) == g):
        assert flat[i].tolist() == blk["codes"], blk["name"]


def test_nvfp4_quantize_near_rounding_thresholds_bitexact(nv):
    """Values whose quotient x / (s g) falls within a few ulps of an E2M1 rounding threshold (0.25,
    0.75, 1.25, 1.75, 2.5, 3.5, 5), on both sides and exactly on it, for several global scales: the
    codes must still be those of the correctly rounded fp32 quotient."""
    thresholds = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    xs = [1.0, 1.3984375, -0.6015625, 37.5]                     # bf16-exact
    cases = 0
    for t in thresholds:
        for x0 in xs:
            for k in list(range(-12, 13)) + [-40, -20, 20, 40]:
                # g such that x0 / g is k ulps away from t (one E4M3 block scale of 1.0: amax ~ 5.9 g)
                q = np.float32(t) * np.float32(1.0 + k * 2.0 ** -23)
                g = np.float32(np.float32(abs(x0)) / q)
                if not (np.isfinite(g) and g > 0):
                    continue
                a = _bf16(np.array([5.9 * float(g)])).float().numpy()[0]
                blk = np.array([a, x0, -x0, x0] + [x0 * (1 - 2.0 ** -8 * i) for i in range(12)], dtype=np.float32)
                tok = _bf16(np.tile(blk, 8)).float().numpy().reshape(1, 1, 128)
                slots = np.array([3], dtype=np.int32)
                dshape, sshape = o_layout.nvfp4_pool_shapes(1, 1)
                want = {kk: np.zeros(sh, np.uint8) for kk, sh in (("k_data", dshape), ("k_scale", sshape),
                                                                 ("v_data", dshape), ("v_scale", sshape))}
                c, sc = o_nv.quantize_blocks(tok, g)
                o_layout.write_nvfp4_tokens(want["k_data"], want["k_scale"], "k", slots, c, sc)
                o_layout.write_nvfp4_tokens(want["v_data"], want["v_scale"], "v", slots, c, sc)
                pool = nv.alloc_nvfp4_pool(1, 1, DEV)
                tt = _bf16(tok).to(DEV)
                nv.nvfp4_quantize_append(tt, tt.clone(), torch.from_numpy(slots).to(DEV), float(g), float(g), pool)
                _check_pool(pool, want)
                cases += 1
    assert cases > 800


@pytest.mark.parametrize("k", [0, 1, -1, 2, -2, 3, -3, 6, -9])
def test_nvfp4_block_scale_near_e4m3_midpoints_bitexact(nv, k):
    """Block maxima on every E4M3 value and rounding midpoint (normal and subnormal) and past the
    448 saturation, under global scales with fp32(6 g) = 1 and a few ulps off it, so that the
    scale quotients amax / fp32(6 g) sit on, or ulps beside, every E4M3 rounding decision: scale
    bytes and codes must be those of the correctly rounded quotient (one launch per scale)."""
    pos = o_codecs.E4M3_POSITIVE
    mids = (pos[:-1] + pos[1:]) / 2
    amaxes = np.concatenate([pos[1:], mids, [448.0, 464.0, 480.0, 512.0, 960.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    n_tok = -(-amaxes.size // 8)
    amaxes = np.concatenate([amaxes, np.ones(n_tok * 8 - amaxes.size)]).astype(np.float32)
    pattern = np.array([1.0, 0.5, -0.25, 0.75, -1.0, 0.375, -0.625, 0.0, 0.125, -0.875, 0.5, 0.25, -0.75, 0.875,
                        -0.5, 0.0625], np.float32)   # |max| = 1 at positions 0 and 4; <= 3 significant bits each
    tok = (amaxes[:, None] * pattern[None, :]).reshape(n_tok, 1, 128).astype(np.float32)
    assert np.array_equal(_bf16(tok).float().numpy(), tok)         # every value exact in bf16
    g = np.float32(np.float32(1.0 + k * 2.0 ** -23) / np.float32(6.0))
    six_g = np.float32(np.float32(6.0) * g)
    assert abs(float(six_g) - 1.0) <= 16 * 2.0 ** -23
    slots = np.arange(n_tok, dtype=np.int32)
    pages = -(-n_tok // 16)
    dshape, sshape = o_layout.nvfp4_pool_shapes(pages, 1)
    want = {kk: np.zeros(sh, np.uint8) for kk, sh in (("k_data", dshape), ("k_scale", sshape),
                                                     ("v_data", dshape), ("v_scale", sshape))}
    c, sc = o_nv.quantize_blocks(tok, g)
    cn, scn = o_nv.quantize_blocks(-tok, g)
    o_layout.write_nvfp4_tokens(want["k_data"], want["k_scale"], "k", slots, c, sc)
    o_layout.write_nvfp4_tokens(want["v_data"], want["v_scale"], "v", slots, cn, scn)
    pool = nv.alloc_nvfp4_pool(pages, 1, DEV)
    tt = _bf16(tok).to(DEV)
    nv.nvfp4_quantize_append(tt, -tt, torch.from_numpy(slots).to(DEV), float(g), float(g), pool)
    _check_pool(pool, want)


def test_nvfp4_quantize_fp8_input_bitexact(nv):
    rng = np.random.default_rng(9)
    n_tok, h = 40, 2
    b = rng.integers(0, 256, (n_tok, h, 128)).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x33
    sk, sv = np.float32(0.013), np.float32(3.5)
    xk = (o_codecs.e4m3_decode(b).astype(np.float32) * sk).astype(np.float32)
    xv = (o_codecs.e4m3_decode(b[::-1].copy()).astype(np.float32) * sv).astype(np.float32)
    gk, gv = o_nv.global_scale(xk), o_nv.global_scale(xv)
    slots = rng.permutation(64)[:n_tok].astype(np.int32)
    dshape, sshape = o_layout.nvfp4_pool_shapes(4, h)
    want = {k: np.zeros(s, np.uint8) for k, s in (("k_data", dshape), ("k_scale", sshape),
                                                  ("v_data", dshape), ("v_scale", sshape))}
    ck, csk = o_nv.quantize_blocks(xk, gk)
    cv, csv = o_nv.quantize_blocks(xv, gv)
    o_layout.write_nvfp4_tokens(want["k_data"], want["k_scale"], "k", slots, ck, csk)
    o_layout.write_nvfp4_tokens(want["v_data"], want["v_scale"], "v", slots, cv, csv)
    pool = nv.alloc_nvfp4_pool(4, h, DEV)
    gk_gpu = nv.global_scale(torch.from_numpy(b).to(DEV), in_scale=float(sk)).item()
    assert np.float32(gk_gpu) == gk
    nv.nvfp4_quantize_append(torch.from_numpy(b).to(DEV), torch.from_numpy(b[::-1].copy()).to(DEV),
                             torch.from_numpy(slots).to(DEV), float(gk), float(gv), pool,
                             k_in_scale=float(sk), v_in_scale=float(sv))
    _check_pool(pool, want)
    # the prepared form writes the same bytes
    pool2 = nv.alloc_nvfp4_pool(4, h, DEV)
    call = nv.prepare_nvfp4_quantize_append(torch.from_numpy(b).to(DEV), torch.from_numpy(b[::-1].copy()).to(DEV),
                                            torch.from_numpy(slots).to(DEV), float(gk), float(gv), pool2,
                                            k_in_scale=float(sk), v_in_scale=float(sv))
    call.run()
    _check_pool(pool2, want)


def test_fp8_quantize_bitexact(nv):
    wl = workloads.Workload(name="fp8-small", seed=11, batch=3, h_kv=2, h_q=8, seq_lens=[33, 5, 70], extra_pages=3)
    ks, vs = H.oracle_inputs(wl)
    sk = o_fp8.fp8_scale(np.concatenate(ks))
    sv = o_fp8.fp8_scale(np.concatenate(vs))
    want_k = np.full(o_layout.fp8_pool_shape(wl.num_pages, wl.h_kv), 0x7F, np.uint8)
    want_v = want_k.copy()
    for b in range(wl.batch):
        o_layout.write_fp8_tokens(want_k, "k", wl.slots(b), o_fp8.fp8_quantize(ks[b], sk))
        o_layout.write_fp8_tokens(want_v, "v", wl.slots(b), o_fp8.fp8_quantize(vs[b], sv))
    from bit_paged_kv_amd import paged
    k, v, slots = H.gpu_all_tokens(wl, 0, DEV)
    pool, g_sk, g_sv = paged.build_fp8_cache(k, v, slots, wl.num_pages, fill=0x7F)
    assert (np.float32(g_sk), np.float32(g_sv)) == (sk, sv)
    assert np.array_equal(pool["k"].cpu().numpy(), want_k)
    assert np.array_equal(pool["v"].cpu().numpy(), want_v)


def _fp8_edge_values():
    """Every E4M3 magnitude and every midpoint between neighbours (normal and subnormal), values at
    and past the 448 saturation (up to inf), zeros, both signs: all exact in bf16."""
    pos = o_codecs.E4M3_POSITIVE
    mids = (pos[:-1] + pos[1:]) / 2
    extra = np.array([448.0, 456.0, 464.0, 472.0, 480.0, 9984.0, np.inf, 0.0, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11])
    mags = np.concatenate([pos, mids, extra])
    vals = np.concatenate([mags, -mags]).astype(np.float32)
    bf = torch.from_numpy(vals).to(torch.bfloat16)
    assert np.array_equal(bf.float().numpy(), vals)                 # all representable in bf16
    return vals


@pytest.mark.parametrize("s", [1.0, 1.0 + 2.0 ** -23, 1.0 - 2.0 ** -24, 1.0 + 3 * 2.0 ** -23, 1.0 - 3 * 2.0 ** -24,
                               2.0 ** -3 * (1.0 + 2.0 ** -22), 0.75])
def test_fp8_encode_near_rounding_midpoints_bitexact(nv, s):
    """FP8 bytes of x / s where the quotients sit on, or a few fp32 ulps from, every E4M3 rounding
    midpoint, in the saturation range and next to zero: the FP8 cache write, the workspace append
    and the prefill copy all match the oracle byte for byte (RNE on the correctly rounded quotient)."""
    vals = _fp8_edge_values()
    s = float(np.float32(s))
    reps = -(-vals.size // 256) * 256
    x = np.resize(vals, reps).reshape(-1, 2, 128)                    # [tokens][2 heads][128]
    x[:, 1] = x[:, 1][:, ::-1]                                       # head 1: another order
    n_tok = x.shape[0]
    want = o_fp8.fp8_quantize(x, s)
    xb = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    # FP8 cache write
    pages = -(-n_tok // 16)
    slots = torch.arange(n_tok, dtype=torch.int32, device=DEV)
    pool = nv.alloc_fp8_pool(pages, 2, DEV, fill=0x7F)
    nv.fp8_quantize_append(xb, xb, slots, s, s, pool)
    want_pool = np.full(o_layout.fp8_pool_shape(pages, 2), 0x7F, np.uint8)
    o_layout.write_fp8_tokens(want_pool, "k", np.arange(n_tok), want)
    assert np.array_equal(pool["k"].cpu().numpy(), want_pool)
    # workspace append of a chunk (rows after a 3-row prefix)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    kw = torch.full((n_tok + 3, 2, 128), 0x7F, dtype=torch.uint8, device=DEV)
    vw = kw.clone()
    nv.fp8_workspace_append(xb, xb, t(np.array([0, n_tok], np.int32)), t(np.array([0], np.int32)),
                            t(np.array([3], np.int32)), n_tok, 3, s, s, 2, kw, vw)
    assert np.array_equal(kw.cpu().numpy()[3:], want)
    assert np.array_equal(vw.cpu().numpy()[3:], want)
    # prefill copy (written with the NVFP4 cache in one pass)
    pool4 = nv.alloc_nvfp4_pool(pages, 2, DEV)
    kc = torch.empty((n_tok, 2, 128), dtype=torch.uint8, device=DEV)
    vc = torch.empty_like(kc)
    nv.nvfp4_prefill_write(xb, xb, slots, 1.0, 1.0, pool4, s, s, kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), want)
    assert np.array_equal(vc.cpu().numpy(), want)


@pytest.mark.parametrize("case", ["small", "many-pages"])
def test_dequant_to_workspace_bitexact(nv, case):
    if case == "small":
        wl = workloads.Workload(name="ws-small", seed=13, batch=3, h_kv=2, h_q=4, seq_lens=[50, 16, 129])
        prefix = np.array([37, 16, 129], dtype=np.int32)
    else:
        # more (page, head) units than resident waves: each wave transcodes several pages in turn,
        # with a ragged last round and a partial last page
        wl = workloads.Workload(name="ws-many", seed=14, batch=2, h_kv=8, h_q=8, seq_lens=[13001, 9100])
        prefix = np.array([13001, 9000], dtype=np.int32)
    assert not wl.append
    ks, vs = H.oracle_inputs(wl)
    gk, gv = o_nv.global_scale(np.concatenate(ks)), o_nv.global_scale(np.concatenate(vs))
    s_wk, s_wv = np.float32(6.0) * gk, np.float32(6.0) * gv    # the layer's FP8 scale, amax / 448
    offs = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int32) + np.array([0] + [5] * wl.batch, dtype=np.int32)
    rows = int(offs[-1]) + 3
    want_k = np.full((rows, wl.h_kv, 128), 0xEE, np.uint8)
    want_v = want_k.copy()
    for b in range(wl.batch):
        n = prefix[b]
        ck, sck = o_nv.quantize_blocks(ks[b][:n], gk)
        cv, scv = o_nv.quantize_blocks(vs[b][:n], gv)
        want_k[offs[b]:offs[b] + n] = o_fp8.nvfp4_to_fp8_workspace(ck, sck, gk, s_wk)
        want_v[offs[b]:offs[b] + n] = o_fp8.nvfp4_to_fp8_workspace(cv, scv, gv, s_wv)
    pool, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV)
    kw = torch.full((rows, wl.h_kv, 128), 0xEE, dtype=torch.uint8, device=DEV)
    vw = kw.clone()
    nv.dequant_to_workspace(pool, float(gk), float(gv), torch.from_numpy(wl.page_table).to(DEV),
                            torch.from_numpy(prefix).to(DEV), torch.from_numpy(offs).to(DEV), int(prefix.max()),
                            float(s_wk), float(s_wv), wl.h_kv, kw, vw)
    assert np.array_equal(kw.cpu().numpy(), want_k)
    assert np.array_equal(vw.cpu().numpy(), want_v)
    # the prepared form, issued twice into fresh buffers, writes the same bytes
    kw2 = torch.full_like(kw, 0xEE)
    vw2 = kw2.clone()
    call = nv.prepare_dequant_to_workspace(pool, float(gk), float(gv), torch.from_numpy(wl.page_table).to(DEV),
                                           torch.from_numpy(prefix).to(DEV), torch.from_numpy(offs).to(DEV),
                                           int(prefix.max()), float(s_wk), float(s_wv), wl.h_kv, kw2, vw2)
    for _ in range(2):
        call.run()
        assert np.array_equal(kw2.cpu().numpy(), want_k)
        assert np.array_equal(vw2.cpu().numpy(), want_v)


@pytest.mark.parametrize("case", range(6))
def test_dequant_to_workspace_random_bitexact(nv, case):
    """The prefix gather on seeded random shapes: 1-6 sequences, prefixes of 0 up to the whole
    sequence, gaps between the workspace rows of consecutive sequences, 1-8 kv heads; every
    workspace byte (the untouched 0xEE rows included) against the oracle's transcode."""
    rng = np.random.default_rng(800 + case)
    batch = int(rng.integers(1, 7))
    h_kv = int(rng.choice([1, 2, 3, 8]))
    lens = rng.integers(1, 2500, size=batch)
    wl = workloads.Workload(name=f"ws-random-{case}", seed=810 + case, batch=batch, h_kv=h_kv, h_q=h_kv,
                            seq_lens=lens, extra_pages=int(rng.integers(0, 4)))
    prefix = np.array([int(rng.choice([0, int(rng.integers(0, n + 1)), n])) for n in lens], dtype=np.int32)
    gaps = rng.integers(0, 9, size=batch)
    offs = np.concatenate([[0], np.cumsum(prefix + gaps)]).astype(np.int32)
    rows = int(offs[-1]) + 2
    ks, vs = H.oracle_inputs(wl)
    gk, gv = o_nv.global_scale(np.concatenate(ks)), o_nv.global_scale(np.concatenate(vs))
    s_wk, s_wv = np.float32(6.0) * gk, np.float32(6.0) * gv
    want_k = np.full((rows, h_kv, 128), 0xEE, np.uint8)
    want_v = want_k.copy()
    for b in range(batch):
        n = int(prefix[b])
        if n == 0:
            continue
        ck, sck = o_nv.quantize_blocks(ks[b][:n], gk)
        cv, scv = o_nv.quantize_blocks(vs[b][:n], gv)
        want_k[offs[b]:offs[b] + n] = o_fp8.nvfp4_to_fp8_workspace(ck, sck, gk, s_wk)
        want_v[offs[b]:offs[b] + n] = o_fp8.nvfp4_to_fp8_workspace(cv, scv, gv, s_wv)
    pool, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV)
    kw = torch.full((rows, h_kv, 128), 0xEE, dtype=torch.uint8, device=DEV)
    vw = kw.clone()
    nv.dequant_to_workspace(pool, float(gk), float(gv), torch.from_numpy(wl.page_table).to(DEV),
                            torch.from_numpy(prefix).to(DEV), torch.from_numpy(offs).to(DEV), int(prefix.max()),
                            float(s_wk), float(s_wv), h_kv, kw, vw)
    torch.cuda.synchronize()
    assert np.array_equal(kw.cpu().numpy(), want_k), f"case {case}: K workspace differs"
    assert np.array_equal(vw.cpu().numpy(), want_v), f"case {case}: V workspace differs"


"""GPU parity of the chunked-extend path (prefix -> FP8 workspace, chunk -> FP8 workspace, causal
attention over prefix || chunk) through the C ABI, against the fp64 oracle on the same bytes."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention as o_att
from oracle import fp8 as o_fp8
from oracle import layout as o_layout
from oracle import nvfp4 as o_nv
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    import bit_paged_kv_amd as nv
    return nv


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _ws_case(seed, prefixes, chunks, hkv, hq, pad=3):
    """Random workspace bytes (E4M3 of N(0,1) with an outlier channel per head, per-tensor scales)
    and bf16 chunk queries.  Workspace rows of sequence b start at ws_off[b]; `pad` unused rows
    (0xEE bytes) separate the sequences."""
    rng = np.random.default_rng(seed)
    b = len(prefixes)
    rows = [p + c for p, c in zip(prefixes, chunks)]
    ws_off = np.zeros(b + 1, dtype=np.int32)
    for i in range(b):
        ws_off[i + 1] = ws_off[i] + rows[i] + pad
    kx = rng.standard_normal((int(ws_off[-1]), hkv, 128)).astype(np.float32)
    vx = rng.standard_normal((int(ws_off[-1]), hkv, 128)).astype(np.float32)
    kx[:, :, 7] *= 12.0
    vx[:, :, 100] *= 9.0
    sk, sv = o_fp8.fp8_scale(kx), o_fp8.fp8_scale(vx)
    k_ws, v_ws = o_fp8.fp8_quantize(kx, sk), o_fp8.fp8_quantize(vx, sv)
    for i in range(b):                                   # the padding rows hold junk (never NaN: 0xEE)
        k_ws[ws_off[i] + rows[i]:ws_off[i + 1]] = 0xEE
        v_ws[ws_off[i] + rows[i]:ws_off[i + 1]] = 0xEE
    c_off = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = _bf16(rng.standard_normal((int(c_off[-1]), hq, 128))).float().numpy()
    return q, k_ws, v_ws, sk, sv, ws_off, c_off


def _oracle(q, k_ws, v_ws, sk, sv, ws_off, c_off, prefixes, sm):
    outs = []
    for i, p in enumerate(prefixes):
        c = int(c_off[i + 1] - c_off[i])
        rows = slice(int(ws_off[i]), int(ws_off[i]) + p + c)
        outs.append(o_att.extend_attention_one(q[c_off[i]:c_off[i + 1]], o_fp8.fp8_dequantize(k_ws[rows], sk),
                                               o_fp8.fp8_dequantize(v_ws[rows], sv), p, sm))
    return np.concatenate(outs)


def _gpu(nv, q, k_ws, v_ws, sk, sv, ws_off, c_off, prefixes, sm, hkv):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    chunks = np.diff(c_off)
    out = nv.fp8_extend_attn(_bf16(q).to(DEV), t(c_off), t(k_ws), t(v_ws), t(ws_off),
                             t(np.array(prefixes, dtype=np.int32)), float(sk), float(sv), sm, hkv,
                             int(chunks.max()), int(max(prefixes)))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("prefixes,chunks,hkv,hq", [
    ([0], [1], 1, 1),                            # a single token, no prefix
    ([0], [70], 2, 8),                           # pure causal prefill, G = 4
    ([37, 300, 5], [33, 1, 129], 2, 8),          # ragged prefixes and chunks, partial tiles
    ([64], [64], 1, 16),                         # G = 16: 8 tokens per workgroup
    ([100, 0], [45, 17], 4, 4),                  # G = 1
    ([31], [96], 3, 6),                          # G = 2, tile and workgroup edges
    ([130], [200], 1, 3),                        # G = 3: 85 tokens per workgroup, one padding column
    ([9], [90], 2, 14),                          # G = 7: 36 tokens per workgroup, four padding columns
    ([250, 40], [33, 70], 2, 16),                # G = 8: 32 tokens per workgroup
])
def test_extend_attention_matches_oracle(nv, prefixes, chunks, hkv, hq):
    sm = 1.0 / np.sqrt(128.0)
    args = _ws_case(7 + sum(prefixes) + hq, prefixes, chunks, hkv, hq)
    want = _oracle(*args, prefixes, sm)
    got = _gpu(nv, *args, prefixes, sm, hkv)
    H.assert_attention_close(got, want, f"extend p={prefixes} c={chunks} G={hq // hkv}")


@pytest.mark.parametrize("case", range(12))
def test_extend_attention_random_shapes(nv, case):
    """Seeded random extend shapes: 1-4 sequences with prefixes 0-3000 and chunks 1-700 tokens
    (a prefix of 0 is a prefill), 1-8 kv heads and query groups 1-16; sequences of one call differ."""
    rng = np.random.default_rng(4000 + case)
    b = int(rng.integers(1, 5))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 11, 16]))
    prefixes = [int(rng.choice([0, int(rng.integers(1, 3001))])) for _ in range(b)]
    chunks = [int(rng.integers(1, 701)) for _ in range(b)]
    sm = 1.0 / np.sqrt(128.0)
    args = _ws_case(4100 + case, prefixes, chunks, hkv, hkv * group)
    want = _oracle(*args, prefixes, sm)
    got = _gpu(nv, *args, prefixes, sm, hkv)
    err = H.assert_attention_close(got, want, f"extend random {case}: p={prefixes} c={chunks} Hkv={hkv} G={group}")
    print(f"extend random {case}: p={prefixes} c={chunks} Hkv={hkv} G={group}: max-abs {err[0]:.2e} rel-L2 {err[1]:.2e}",
          flush=True)


@pytest.mark.parametrize("batch,hkv,group,chunk_range", [
    (128, 8, 4, (30, 91)),      # 96 tokens per workgroup: one block per sequence, 1024 workgroups
    (64, 8, 16, (30, 71)),      # 24 tokens per workgroup: two or three blocks per sequence
    (130, 8, 5, (50, 151)),     # 76 tokens per workgroup and four padding columns
    (128, 8, 3, (60, 129)),     # 128 tokens per workgroup
    (256, 4, 1, (200, 384)),    # 384 tokens per workgroup
])
def test_extend_attention_wide_tiles(nv, batch, hkv, group, chunk_range):
    """Grids long enough (at least four workgroups per compute unit on a 256-unit device) for the
    launcher to pick three 16-column score tiles per wave; ragged prefixes and chunks."""
    rng = np.random.default_rng(batch * 31 + group)
    prefixes = [int(x) for x in rng.integers(0, 200, size=batch)]
    chunks = [int(x) for x in rng.integers(chunk_range[0], chunk_range[1], size=batch)]
    tpw3 = 384 // group
    assert -(-max(chunks) // tpw3) * hkv * batch >= 4 * 256
    sm = 1.0 / np.sqrt(128.0)
    args = _ws_case(5000 + batch + group, prefixes, chunks, hkv, hkv * group, pad=1)
    want = _oracle(*args, prefixes, sm)
    got = _gpu(nv, *args, prefixes, sm, hkv)
    err = H.assert_attention_close(got, want, f"extend wide tiles B={batch} Hkv={hkv} G={group}")
    print(f"extend wide tiles B={batch} Hkv={hkv} G={group}: max-abs {err[0]:.2e} rel-L2 {err[1]:.2e}", flush=True)


def test_extend_attention_rising_maximum(nv):
    """K rows grow ~12x along the sequence, so the running maximum of every column rises again and
    again (each rise rescales the accumulated output); 100 chunk tokens at G = 4 fill both halves of
    a workgroup's columns."""
    prefixes, chunks, hkv, hq = [500], [100], 2, 8
    rng = np.random.default_rng(77)
    rows = prefixes[0] + chunks[0]
    kx = rng.standard_normal((rows, hkv, 128)).astype(np.float32) * np.linspace(1.0, 12.0, rows)[:, None, None]
    vx = rng.standard_normal((rows, hkv, 128)).astype(np.float32)
    sk, sv = o_fp8.fp8_scale(kx), o_fp8.fp8_scale(vx)
    k_ws, v_ws = o_fp8.fp8_quantize(kx, sk), o_fp8.fp8_quantize(vx, sv)
    ws_off = np.array([0, rows], dtype=np.int32)
    c_off = np.array([0, chunks[0]], dtype=np.int32)
    q = _bf16(rng.standard_normal((chunks[0], hq, 128))).float().numpy()
    sm = 1.0 / np.sqrt(128.0)
    args = (q, k_ws, v_ws, sk, sv, ws_off, c_off)
    want = _oracle(*args, prefixes, sm)
    got = _gpu(nv, *args, prefixes, sm, hkv)
    H.assert_attention_close(got, want, "extend, rising maximum")


def test_extend_attention_repeatable_and_prepared(nv):
    prefixes, chunks, hkv, hq = [200, 17], [50, 90], 2, 8
    q, k_ws, v_ws, sk, sv, ws_off, c_off = _ws_case(3, prefixes, chunks, hkv, hq)
    sm = 0.1
    first = _gpu(nv, q, k_ws, v_ws, sk, sv, ws_off, c_off, prefixes, sm, hkv)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = torch.full((q.shape[0], hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    call, out = nv.prepare_fp8_extend_attn(_bf16(q).to(DEV), t(c_off), t(k_ws), t(v_ws), t(ws_off),
                                           t(np.array(prefixes, dtype=np.int32)), float(sk), float(sv), sm, hkv,
                                           int(max(chunks)), int(max(prefixes)), out=out)
    for _ in range(2):
        call.run()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), first)


def test_fp8_workspace_append_bitexact(nv):
    rng = np.random.default_rng(5)
    prefixes, chunks, hkv = [10, 0, 333], [7, 40, 1], 3
    c_off = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    ws_off = np.array([0, 20, 70, 420], dtype=np.int32)
    k = _bf16(rng.standard_normal((int(c_off[-1]), hkv, 128)) * 3).float().numpy()
    v = _bf16(rng.standard_normal((int(c_off[-1]), hkv, 128))).float().numpy()
    k[0, 0, :4] = [0.0, -0.0, 1e-9, -5000.0]                                # zeros, underflow, saturation
    sk, sv = o_fp8.fp8_scale(k), np.float32(0.0123)
    want_k = np.full((420, hkv, 128), 0x5A, np.uint8)
    want_v = want_k.copy()
    for i, p in enumerate(prefixes):
        r0 = ws_off[i] + p
        want_k[r0:r0 + chunks[i]] = o_fp8.fp8_quantize(k[c_off[i]:c_off[i + 1]], sk)
        want_v[r0:r0 + chunks[i]] = o_fp8.fp8_quantize(v[c_off[i]:c_off[i + 1]], sv)
    kw = torch.full((420, hkv, 128), 0x5A, dtype=torch.uint8, device=DEV)
    vw = kw.clone()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    nv.fp8_workspace_append(_bf16(k).to(DEV), _bf16(v).to(DEV), t(c_off), t(ws_off),
                            t(np.array(prefixes, dtype=np.int32)), max(chunks), max(prefixes), float(sk), float(sv),
                            hkv, kw, vw)
    assert np.array_equal(kw.cpu().numpy(), want_k)
    assert np.array_equal(vw.cpu().numpy(), want_v)


def test_extend_chain_from_nvfp4_cache(nv):
    """The whole extend step on seeded workload data: NVFP4 prefix pool -> FP8 workspace (GPU),
    chunk -> FP8 workspace (GPU), attention (GPU); the oracle runs the same chain from the inputs."""
    prefixes, chunks = [150, 61], [40, 77]
    wl = workloads.Workload(name="extend-small", seed=91, batch=2, h_kv=2, h_q=8,
                            seq_lens=[p + c for p, c in zip(prefixes, chunks)], chan="outlier2")
    ks, vs = H.oracle_inputs(wl)                          # [L_b][H][128] fp32 (bf16 values)
    gk = o_nv.global_scale(np.concatenate([k[:p] for k, p in zip(ks, prefixes)]))
    gv = o_nv.global_scale(np.concatenate([v[:p] for v, p in zip(vs, prefixes)]))
    s_wk = o_fp8.fp8_scale(np.concatenate(ks))
    s_wv = o_fp8.fp8_scale(np.concatenate(vs))
    ws_off = np.array([0, 200, 400], dtype=np.int32)
    c_off = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    rng = np.random.default_rng(4)
    q = _bf16(rng.standard_normal((int(c_off[-1]), wl.h_q, 128))).float().numpy()
    # oracle chain
    want_k = np.zeros((400, wl.h_kv, 128), np.uint8)
    want_v = want_k.copy()
    for b, p in enumerate(prefixes):
        ck, sck = o_nv.quantize_blocks(ks[b][:p], gk)
        cv, scv = o_nv.quantize_blocks(vs[b][:p], gv)
        want_k[ws_off[b]:ws_off[b] + p] = o_fp8.nvfp4_to_fp8_workspace(ck, sck, gk, s_wk)
        want_v[ws_off[b]:ws_off[b] + p] = o_fp8.nvfp4_to_fp8_workspace(cv, scv, gv, s_wv)
        want_k[ws_off[b] + p:ws_off[b] + p + chunks[b]] = o_fp8.fp8_quantize(ks[b][p:], s_wk)
        want_v[ws_off[b] + p:ws_off[b] + p + chunks[b]] = o_fp8.fp8_quantize(vs[b][p:], s_wv)
    sm = wl.sm_scale
    want = _oracle(q, want_k, want_v, s_wk, s_wv, ws_off, c_off, prefixes, sm)
    # GPU chain
    from bit_paged_kv_amd import paged
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    kp = torch.cat([_bf16(ks[b][:p]) for b, p in enumerate(prefixes)]).to(DEV)
    vp = torch.cat([_bf16(vs[b][:p]) for b, p in enumerate(prefixes)]).to(DEV)
    slots = t(np.concatenate([wl.slots(b, 0, p) for b, p in enumerate(prefixes)]))
    pool, g_k, g_v = paged.build_nvfp4_cache(kp, vp, slots, wl.num_pages)
    assert (np.float32(g_k), np.float32(g_v)) == (gk, gv)
    kw = torch.zeros((400, wl.h_kv, 128), dtype=torch.uint8, device=DEV)
    vw = kw.clone()
    pre = t(np.array(prefixes, dtype=np.int32))
    nv.dequant_to_workspace(pool, float(gk), float(gv), t(wl.page_table), pre, t(ws_off), max(prefixes),
                            float(s_wk), float(s_wv), wl.h_kv, kw, vw)
    kc = torch.cat([_bf16(ks[b][p:]) for b, p in enumerate(prefixes)]).to(DEV)
    vc = torch.cat([_bf16(vs[b][p:]) for b, p in enumerate(prefixes)]).to(DEV)
    nv.fp8_workspace_append(kc, vc, t(c_off), t(ws_off), pre, max(chunks), max(prefixes), float(s_wk), float(s_wv),
                            wl.h_kv, kw, vw)
    torch.cuda.synchronize()
    assert np.array_equal(kw.cpu().numpy(), want_k)
    assert np.array_equal(vw.cpu().numpy(), want_v)
    out = nv.fp8_extend_attn(_bf16(q).to(DEV), t(c_off), kw, vw, t(ws_off), pre, float(s_wk), float(s_wv), sm,
                             wl.h_kv, max(chunks), max(prefixes))
    torch.cuda.synchronize()
    H.assert_attention_close(out.cpu().numpy(), want, "extend chain")


def test_extend_full_size_sampled(nv):
    """The bench's extend workload at full size (16384-token NVFP4 prefix + 2048-token chunk, 8 KV /
    32 query heads, one NVFP4 layer) through the same calls the bench makes.  From the same seeded
    inputs the oracle gives every byte of the NVFP4 prefix cache and of the FP8 workspace (prefix
    transcoded, chunk appended), both compared whole, and sampled chunk rows (all heads) as decode
    steps over their visible keys."""
    wl = workloads.config(4)
    layer = 1
    assert not wl.is_fp8(layer)
    prefix, chunk = wl.extend_prefix, wl.extend_chunk
    ext = workloads.Workload(name="extend", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q,
                             seq_lens=[prefix + chunk], chan=wl.chan)
    kp = ext.kv("k", 0, layer, length=prefix)
    vp = ext.kv("v", 0, layer, length=prefix)
    kc = wl.chunk("k", layer)
    vc = wl.chunk("v", layer)
    rng = np.random.default_rng(2024)
    q = _bf16(rng.standard_normal((chunk, wl.h_q, 128)))
    print("extend full size: inputs generated", flush=True)
    # GPU, as in the bench
    from bit_paged_kv_amd import paged
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    pool, gk, gv = paged.build_nvfp4_cache(kp.to(DEV), vp.to(DEV), t(ext.slots(0, 0, prefix)), ext.num_pages)
    s_wk, s_wv = 6.0 * gk, 6.0 * gv
    kw = torch.empty((prefix + chunk, wl.h_kv, 128), dtype=torch.uint8, device=DEV)
    vw = torch.empty_like(kw)
    pre = torch.tensor([prefix], dtype=torch.int32, device=DEV)
    offs = torch.tensor([0, prefix], dtype=torch.int32, device=DEV)
    c_off = torch.tensor([0, chunk], dtype=torch.int32, device=DEV)
    nv.dequant_to_workspace(pool, gk, gv, t(ext.page_table), pre, offs, prefix, s_wk, s_wv, wl.h_kv, kw, vw)
    nv.fp8_workspace_append(kc.to(DEV), vc.to(DEV), c_off, offs, pre, chunk, prefix, s_wk, s_wv, wl.h_kv, kw, vw)
    out = nv.fp8_extend_attn(q.to(DEV), c_off, kw, vw, offs, pre, s_wk, s_wv, wl.sm_scale, wl.h_kv, chunk, prefix)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    got_kw, got_vw = kw.cpu().numpy(), vw.cpu().numpy()
    got_pool = {key: a.cpu().numpy() for key, a in pool.items()}
    del pool, kw, vw
    print("extend full size: GPU done", flush=True)
    # oracle chain on the same inputs
    kpn, vpn = kp.float().numpy(), vp.float().numpy()
    g_k, g_v = o_nv.global_scale(kpn), o_nv.global_scale(vpn)
    assert (np.float32(gk), np.float32(gv)) == (g_k, g_v)
    sw_k, sw_v = np.float32(6.0) * g_k, np.float32(6.0) * g_v
    ck, sck = o_nv.quantize_blocks(kpn, g_k)
    cv, scv = o_nv.quantize_blocks(vpn, g_v)
    slots = ext.slots(0, 0, prefix)
    for name, kind, codes, scales in (("K", "k", ck, sck), ("V", "v", cv, scv)):
        gc, gs = o_layout.read_nvfp4_tokens(got_pool[kind + "_data"], got_pool[kind + "_scale"], kind, slots)
        assert np.array_equal(gc, codes), f"prefix cache {name} codes differ from the oracle's"
        assert np.array_equal(gs, scales), f"prefix cache {name} scales differ from the oracle's"
    want_kw = np.concatenate([o_fp8.nvfp4_to_fp8_workspace(ck, sck, g_k, sw_k), o_fp8.fp8_quantize(kc.float().numpy(), sw_k)])
    want_vw = np.concatenate([o_fp8.nvfp4_to_fp8_workspace(cv, scv, g_v, sw_v), o_fp8.fp8_quantize(vc.float().numpy(), sw_v)])
    assert np.array_equal(got_kw, want_kw), f"K workspace: {int((got_kw != want_kw).sum())} bytes differ"
    assert np.array_equal(got_vw, want_vw), f"V workspace: {int((got_vw != want_vw).sum())} bytes differ"
    print(f"extend full size: every prefix cache byte and all {want_kw.size + want_vw.size} workspace bytes bit-exact",
          flush=True)
    k_hat = o_fp8.fp8_dequantize(want_kw, sw_k)
    v_hat = o_fp8.fp8_dequantize(want_vw, sw_v)
    qn = q.float().numpy()
    rows = [0, 1, 31, 32, 777, 1024, 2046, 2047] + list(rng.integers(0, chunk, 8))
    want = np.stack([o_att.decode_attention_one(qn[i], k_hat[:prefix + i + 1], v_hat[:prefix + i + 1], wl.sm_scale)
                     for i in rows])
    H.assert_attention_close(got[rows], want, "extend full size, sampled rows")


@pytest.mark.parametrize("lens", [[5], [300, 1, 77, 64]])
def test_prefill_write_and_attention(nv, lens):
    """The prefill path: one pass writes the NVFP4 cache (bytes as the oracle's quantize-append) and
    the dense FP8 copy (bytes as the oracle's FP8 quantize); the causal attention over that copy
    (prefix 0) matches the fp64 oracle.  Sequences start at arbitrary token quads (misaligned runs)."""
    wl = workloads.Workload(name="prefill-small", seed=33, batch=len(lens), h_kv=2, h_q=8, seq_lens=lens,
                            chan="outlier2", extra_pages=2)
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    s_wk, s_wv = np.float32(6.0) * gk, np.float32(6.0) * gv
    want_pool = H.oracle_nvfp4_pool(wl, ks, vs, gk, gv)
    k_all, v_all = np.concatenate(ks), np.concatenate(vs)
    want_kw, want_vw = o_fp8.fp8_quantize(k_all, s_wk), o_fp8.fp8_quantize(v_all, s_wv)
    k, v, slots = H.gpu_all_tokens(wl, 0, DEV)
    pool = nv.alloc_nvfp4_pool(wl.num_pages, wl.h_kv, DEV)
    kw = torch.full(k.shape, 0x11, dtype=torch.uint8, device=DEV)
    vw = kw.clone()
    nv.nvfp4_prefill_write(k, v, slots, float(gk), float(gv), pool, float(s_wk), float(s_wv), kw, vw)
    torch.cuda.synchronize()
    for key in ("k_data", "k_scale", "v_data", "v_scale"):
        assert np.array_equal(pool[key].cpu().numpy(), want_pool[key]), key
    assert np.array_equal(kw.cpu().numpy(), want_kw)
    assert np.array_equal(vw.cpu().numpy(), want_vw)
    # prefill attention: chunk = the whole sequence, prefix 0, workspace rows = token offsets
    rng = np.random.default_rng(8)
    q = _bf16(rng.standard_normal((k_all.shape[0], wl.h_q, 128))).float().numpy()
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    prefixes = [0] * len(lens)
    want = _oracle(q, want_kw, want_vw, s_wk, s_wv, offs, offs, prefixes, wl.sm_scale)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    out = nv.fp8_extend_attn(_bf16(q).to(DEV), t(offs), kw, vw, t(offs), t(np.zeros(len(lens), np.int32)),
                             float(s_wk), float(s_wv), wl.sm_scale, wl.h_kv, max(lens), 0)
    torch.cuda.synchronize()
    H.assert_attention_close(out.cpu().numpy(), want, f"prefill {lens}")


@pytest.mark.timeout(900)
def test_prefill_full_size_sampled(nv):
    """The bench's prefill workload at full size (one 16384-token prompt of an NVFP4 layer, 8 KV /
    32 query heads) through the bench's calls: the one-pass write's NVFP4 pool and FP8 copy are
    byte-exact against the oracle's quantizers, and sampled query rows (all heads) of the causal
    attention over the copy match the oracle's attention over the keys they see."""
    wl = workloads.config(4)
    layer = 1
    assert not wl.is_fp8(layer)
    n = wl.extend_prefix
    ext = workloads.Workload(name="prefill", seed=wl.seed, batch=1, h_kv=wl.h_kv, h_q=wl.h_q, seq_lens=[n],
                             chan=wl.chan)
    k = ext.kv("k", 0, layer)
    v = ext.kv("v", 0, layer)
    rng = np.random.default_rng(2025)
    q = _bf16(rng.standard_normal((n, wl.h_q, 128)))
    print("prefill full size: inputs generated", flush=True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    slots = ext.slots(0, 0, n)
    kd, vd = k.to(DEV), v.to(DEV)
    gk = float(nv.global_scale(kd).item())
    gv = float(nv.global_scale(vd).item())
    s_wk, s_wv = 6.0 * gk, 6.0 * gv
    pool = nv.alloc_nvfp4_pool(ext.num_pages, wl.h_kv, DEV)
    kw = torch.empty((n, wl.h_kv, 128), dtype=torch.uint8, device=DEV)
    vw = torch.empty_like(kw)
    nv.nvfp4_prefill_write(kd, vd, t(slots), gk, gv, pool, s_wk, s_wv, kw, vw)
    offs = torch.tensor([0, n], dtype=torch.int32, device=DEV)
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = nv.fp8_extend_attn(q.to(DEV), offs, kw, vw, offs, zero, s_wk, s_wv, wl.sm_scale, wl.h_kv, n, 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    got_kw, got_vw = kw.cpu().numpy(), vw.cpu().numpy()
    got_pool = H.pool_to_numpy(pool)
    print("prefill full size: GPU done", flush=True)
    kn, vn = k.float().numpy(), v.float().numpy()
    g_k, g_v = o_nv.global_scale(kn), o_nv.global_scale(vn)
    assert (np.float32(gk), np.float32(gv)) == (g_k, g_v)
    sw_k, sw_v = np.float32(6.0) * g_k, np.float32(6.0) * g_v
    # the FP8 copy, every byte
    want_kw, want_vw = o_fp8.fp8_quantize(kn, sw_k), o_fp8.fp8_quantize(vn, sw_v)
    assert np.array_equal(got_kw, want_kw)
    assert np.array_equal(got_vw, want_vw)
    # the NVFP4 pool, every byte of the prompt's pages
    want_pool = H.oracle_nvfp4_pool(ext, [kn], [vn], g_k, g_v)
    for key in ("k_data", "k_scale", "v_data", "v_scale"):
        assert np.array_equal(got_pool[key], want_pool[key]), key
    print("prefill full size: write bytes exact", flush=True)
    k_hat = o_fp8.fp8_dequantize(want_kw, sw_k)
    v_hat = o_fp8.fp8_dequantize(want_vw, sw_v)
    qn = q.float().numpy()
    rows = [0, 1, 63, 64, 4095, 8191, 16382, 16383] + list(rng.integers(0, n, 8))
    want = np.stack([o_att.decode_attention_one(qn[i], k_hat[:i + 1], v_hat[:i + 1], wl.sm_scale) for i in rows])
    err = H.assert_attention_close(got[rows], want, "prefill full size, sampled rows")
    print(f"prefill full size: sampled rows max-abs {err[0]:.2e} rel-L2 {err[1]:.2e}", flush=True)

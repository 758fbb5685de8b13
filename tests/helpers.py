"""Shared test glue: oracle-side references and GPU-side set-up for one workload.

The oracle side works only from the seeded inputs (workloads); the GPU side only through the
C-ABI binding.  Nothing computed by the GPU is ever fed to the oracle.
"""
from __future__ import annotations

import hashlib
import os

import numpy as np
import torch

import workloads
from oracle import attention as o_att
from oracle import fp8 as o_fp8
from oracle import layout as o_layout
from oracle import nvfp4 as o_nv

MAX_ABS = 2e-3     # attention tolerance: max |gpu - oracle| over the whole output
REL_L2 = 1e-3      # and ||gpu - oracle||_2 / ||oracle||_2


def assert_attention_close(got: np.ndarray, want: np.ndarray, tag: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{tag}: non-finite output"
    err = np.abs(got - want)
    max_abs = float(err.max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{tag}: max-abs {max_abs:.3e} rel-L2 {rel:.3e}"
    return max_abs, rel


# ------------------------------------------------------------------------------------------------
# oracle side
# ------------------------------------------------------------------------------------------------
def oracle_inputs(wl: workloads.Workload, layer: int = 0, with_new: bool | None = None):
    """fp32 K/V per sequence (cache + appended token when the workload appends)."""
    with_new = wl.append if with_new is None else with_new
    ks, vs = [], []
    nk = wl.new_token("k", layer).float().numpy() if with_new else None
    nv = wl.new_token("v", layer).float().numpy() if with_new else None
    for b in range(wl.batch):
        k = wl.kv("k", b, layer).float().numpy()
        v = wl.kv("v", b, layer).float().numpy()
        if with_new:
            k = np.concatenate([k, nk[b:b + 1]], axis=0)
            v = np.concatenate([v, nv[b:b + 1]], axis=0)
        ks.append(k)
        vs.append(v)
    return ks, vs


def oracle_nvfp4_scales(wl, layer=0):
    """Global scales from the cached tokens only (appended tokens reuse them)."""
    ks, vs = oracle_inputs(wl, layer, with_new=False)
    return o_nv.global_scale(np.concatenate(ks)), o_nv.global_scale(np.concatenate(vs))


def oracle_nvfp4_pool(wl, ks, vs, gk, gv, fill=0):
    """Oracle pool bytes after writing every token of ks/vs (lists of [n][H][128] fp32)."""
    dshape, sshape = o_layout.nvfp4_pool_shapes(wl.num_pages, wl.h_kv)
    pool = {k: np.full(s, fill, dtype=np.uint8) for k, s in
            (("k_data", dshape), ("k_scale", sshape), ("v_data", dshape), ("v_scale", sshape))}
    for b in range(wl.batch):
        n = ks[b].shape[0]
        slots = wl.slots(b, 0, n)
        ck, sk = o_nv.quantize_blocks(ks[b], gk)
        cv, sv = o_nv.quantize_blocks(vs[b], gv)
        o_layout.write_nvfp4_tokens(pool["k_data"], pool["k_scale"], "k", slots, ck, sk)
        o_layout.write_nvfp4_tokens(pool["v_data"], pool["v_scale"], "v", slots, cv, sv)
    return pool


def oracle_nvfp4_decode(wl, q, ks, vs, gk, gv):
    """fp64 attention over the oracle's own dequantized cache."""
    kh, vh = [], []
    for b in range(wl.batch):
        ck, sk = o_nv.quantize_blocks(ks[b], gk)
        cv, sv = o_nv.quantize_blocks(vs[b], gv)
        kh.append(o_nv.dequantize_blocks(ck, sk, gk))
        vh.append(o_nv.dequantize_blocks(cv, sv, gv))
    return o_att.decode_attention(q, kh, vh, wl.sm_scale)


def oracle_fp8_decode(wl, q, ks, vs, sk, sv):
    kh = [o_fp8.fp8_dequantize(o_fp8.fp8_quantize(k, sk), sk) for k in ks]
    vh = [o_fp8.fp8_dequantize(o_fp8.fp8_quantize(v, sv), sv) for v in vs]
    return o_att.decode_attention(q, kh, vh, wl.sm_scale)


# ------------------------------------------------------------------------------------------------
# GPU side
# ------------------------------------------------------------------------------------------------
def gpu_all_tokens(wl, layer, dev):
    """Concatenated cached K, V ([sum L][H][128] bf16) and slots on the GPU."""
    k = torch.cat([wl.kv("k", b, layer) for b in range(wl.batch)]).to(dev)
    v = torch.cat([wl.kv("v", b, layer) for b in range(wl.batch)]).to(dev)
    slots = torch.from_numpy(np.concatenate([wl.slots(b) for b in range(wl.batch)])).to(dev)
    return k, v, slots


def gpu_nvfp4_layer(wl, layer, dev, fill=0):
    from bit_paged_kv_amd import paged
    k, v, slots = gpu_all_tokens(wl, layer, dev)
    return paged.build_nvfp4_cache(k, v, slots, wl.num_pages, fill=fill)


def gpu_tables(wl, dev, seq_lens=None):
    pt = torch.from_numpy(wl.page_table).to(dev)
    sl = torch.from_numpy((wl.total_lens if seq_lens is None else seq_lens).astype(np.int32)).to(dev)
    return pt, sl


def pool_to_numpy(pool):
    return {k: t.cpu().numpy() for k, t in pool.items()}


# ------------------------------------------------------------------------------------------------
# whole full-size caches: every stream's code and scale bytes, compared through digests
# ------------------------------------------------------------------------------------------------
def host_workers() -> int:
    """Worker processes for oracle work on the host: the cores this process may use, at most 16
    (the host-CPU share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def stream_digest(*arrays) -> str:
    """sha256 over one (sequence, kv head) stream's bytes, each array as contiguous uint8 in token
    order: NVFP4 K codes [n][128], K scale bytes [n][8], V codes, V scale bytes; or FP8 K and V
    bytes [n][128]."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a, dtype=np.uint8).tobytes())
    return h.hexdigest()


def oracle_stream_digests(task) -> dict:
    """Host worker: digests of the oracle's cache bytes for the streams (b, hk), hk in `heads`, of a
    workload (a config index or a Workload) and layer, from its seeded inputs alone (the appended
    token included when the workload appends), under the oracle's scales s_k, s_v: NVFP4 global
    scales, or FP8 per-tensor scales when `fp8`.  task = (which, b, heads, s_k, s_v[, layer, fp8])."""
    which, b, heads, s_k, s_v, layer, fp8 = (tuple(task) + (0, False))[:7]
    wl = workloads.config(which) if isinstance(which, int) else which
    k, v = wl.kv("k", b, layer), wl.kv("v", b, layer)
    nk = wl.new_token("k", layer)[b] if wl.append else None
    nv = wl.new_token("v", layer)[b] if wl.append else None
    out = {}
    for hk in heads:
        kh, vh = k[:, hk].float().numpy(), v[:, hk].float().numpy()
        if wl.append:
            kh = np.concatenate([kh, nk[hk][None].float().numpy()])
            vh = np.concatenate([vh, nv[hk][None].float().numpy()])
        if fp8:
            out[(b, hk)] = stream_digest(o_fp8.fp8_quantize(kh, s_k), o_fp8.fp8_quantize(vh, s_v))
        else:
            ck, sk = o_nv.quantize_blocks(kh, s_k)
            cv, sv = o_nv.quantize_blocks(vh, s_v)
            out[(b, hk)] = stream_digest(ck, sk, cv, sv)
    return out


def digest_tasks(wl, which, s_k, s_v, layer=0, fp8=False) -> list:
    """oracle_stream_digests tasks covering every stream of a workload: one per sequence, or per
    pair of kv heads for sequences long enough to keep a worker busy on their own."""
    return [(which, b, heads, s_k, s_v, layer, fp8) for b in range(wl.batch)
            for heads in ([list(range(wl.h_kv))] if wl.seq_lens[b] <= 32768 else
                          [[h, h + 1] for h in range(0, wl.h_kv, 2)])]


def pool_stream_digest(rows, n_tok: int, fp8: bool = False) -> str:
    """Digest of one stream's bytes as a GPU pool holds them: `rows` is {key: [pages][1][bytes]}
    of the stream's pages in sequence order (token t at local slot t)."""
    local = np.arange(n_tok)
    if fp8:
        return stream_digest(o_layout.read_fp8_tokens(rows["k"], "k", local)[:, 0],
                             o_layout.read_fp8_tokens(rows["v"], "v", local)[:, 0])
    ck, sk = o_layout.read_nvfp4_tokens(rows["k_data"], rows["k_scale"], "k", local)
    cv, sv = o_layout.read_nvfp4_tokens(rows["v_data"], rows["v_scale"], "v", local)
    return stream_digest(ck[:, 0], sk[:, 0], cv[:, 0], sv[:, 0])

"""Precision studies built from the library's own calls (run by ``bench.py --config sweep``).

Not part of the library: the studies need a reference attention on the unquantized K/V, which
lives here, beside the bench, rather than in the binding package.

* layer_sensitivity -- the per-layer sweep behind the mixed-precision rule of [O] "03 Mixed-precision
  KV Cache" (sensitive layers keep FP8): for every layer, the decode output with the layer's cache in
  NVFP4 and in FP8, each compared with attention on the unquantized bf16 K/V, and NVFP4 against FP8.
* gscale_variants -- the per-tensor scale the pages leave uncalibrated ([S] "The Core of the Ledger"
  paragraph 1; the summary notes the global scaling is not calibrated): the whole-tensor amax (the
  default), a static scale calibrated on a prefix of the tokens (later, larger values saturate), and
  one scale per KV head (each head quantized and decoded by its own call: the same kernels, more
  launches).  Each variant reports its error and its decode time.

Every quantization and decode runs in the HIP kernels; the reference attention is plain fp32 torch
on the GPU and the error metrics are reductions over the outputs (analysis, not the decode path).
"""
from __future__ import annotations

import torch

from bit_paged_kv_amd import _lib, paged


def attention_reference(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens, sm_scale: float) -> torch.Tensor:
    """fp32 attention on unquantized K/V: q [B][H_q][128]; k, v [sum L][H_kv][128] (sequences
    concatenated in order); seq_lens: host list.  Returns [B][H_q][128] fp32."""
    b, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
    start = 0
    for i, n in enumerate(seq_lens):
        kb = k[start:start + n].float().permute(1, 0, 2).contiguous()      # [H_kv][L][D]
        vb = v[start:start + n].float().permute(1, 0, 2).contiguous()
        qb = q[i].float().view(hkv, g, d)                                  # [H_kv][G][D]
        s = torch.matmul(qb, kb.transpose(1, 2).contiguous()) * sm_scale   # [H_kv][G][L]
        p = torch.softmax(s, dim=-1)
        out[i] = torch.matmul(p, vb).reshape(hq, d)
        start += n
    return out


def errors(out: torch.Tensor, ref: torch.Tensor, num_kv_heads: int | None = None) -> dict:
    """max-abs and rel-L2 of out against ref ([B][H_q][128]); with num_kv_heads, also the rel-L2 of
    each kv head's query group (heads of very different scale would otherwise hide each other)."""
    diff = (out.double() - ref.double())
    res = {"max_abs": float(diff.abs().max()), "rel_l2": float(diff.norm() / ref.double().norm().clamp_min(1e-300))}
    if num_kv_heads:
        g = out.shape[1] // num_kv_heads
        res["rel_l2_per_kv_head"] = [
            float(diff[:, h * g:(h + 1) * g].norm() / ref[:, h * g:(h + 1) * g].double().norm().clamp_min(1e-300))
            for h in range(num_kv_heads)]
    return res


def _decode_timed(fn, reps: int = 5):
    """Run fn() once (result) and reps more times between events; returns (result, us per call)."""
    out = fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return out, e0.elapsed_time(e1) * 1e3 / reps


def layer_sensitivity(layers: list, slots: torch.Tensor, num_pages: int, page_table: torch.Tensor,
                      seq_lens: torch.Tensor, sm_scale: float, num_kv_heads: int) -> list:
    """layers: list of dict(q [B][H_q][128] bf16, k, v [sum L][H_kv][128] bf16), all on the GPU.
    Returns one dict per layer: errors of the NVFP4 and FP8 decode against the bf16 reference, and
    of NVFP4 against FP8."""
    lens = [int(x) for x in seq_lens.cpu()]
    plan = _lib.plan_decode(len(lens), num_kv_heads, max(lens), sum(lens))
    rows = []
    for i, L in enumerate(layers):
        ref = attention_reference(L["q"], L["k"], L["v"], lens, sm_scale)
        pool4, gk, gv = paged.build_nvfp4_cache(L["k"], L["v"], slots, num_pages)
        o4 = _lib.nvfp4_decode(L["q"], pool4, gk, gv, page_table, seq_lens, sm_scale, plan, num_kv_heads)
        del pool4
        pool8, sk, sv = paged.build_fp8_cache(L["k"], L["v"], slots, num_pages)
        o8 = _lib.fp8_decode(L["q"], pool8, sk, sv, page_table, seq_lens, sm_scale, plan, num_kv_heads)
        del pool8
        torch.cuda.synchronize()
        rows.append({"layer": i, "nvfp4_vs_bf16": errors(o4, ref), "fp8_vs_bf16": errors(o8, ref),
                     "nvfp4_vs_fp8": errors(o4, o8)})
    return rows


def gscale_variants(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor, num_pages: int,
                    page_table: torch.Tensor, seq_lens: torch.Tensor, sm_scale: float, num_kv_heads: int,
                    calib_tokens: int) -> dict:
    """Error and decode time of the per-tensor scale variants for one layer (see the module notes).
    calib_tokens: the first calib_tokens rows of k / v form the calibration sample."""
    lens = [int(x) for x in seq_lens.cpu()]
    b, hq, _ = q.shape
    g = hq // num_kv_heads
    plan = _lib.plan_decode(b, num_kv_heads, max(lens), sum(lens))
    ref = attention_reference(q, k, v, lens, sm_scale)
    res = {}
    # whole-tensor amax (the default) and a static scale from a calibration prefix
    calib = (float(_lib.global_scale(k[:calib_tokens]).item()), float(_lib.global_scale(v[:calib_tokens]).item()))
    for name, gs in (("tensor_amax", None), ("calibrated_prefix", calib)):
        pool, gk, gv = paged.build_nvfp4_cache(k, v, slots, num_pages, gscales=gs)
        out, us = _decode_timed(lambda: _lib.nvfp4_decode(q, pool, gk, gv, page_table, seq_lens, sm_scale, plan,
                                                         num_kv_heads))
        res[name] = {"k_gscale": gk, "v_gscale": gv, **errors(out, ref, num_kv_heads), "decode_us": us}
        del pool
    # one scale per kv head: each head in its own pool, decoded by its own call
    plan1 = _lib.plan_decode(b, 1, max(lens), sum(lens))
    pools, scales, qs, outs = [], [], [], []
    for h in range(num_kv_heads):
        kh = k[:, h:h + 1].contiguous()
        vh = v[:, h:h + 1].contiguous()
        pool, gk, gv = paged.build_nvfp4_cache(kh, vh, slots, num_pages)
        pools.append(pool)
        scales.append((gk, gv))
        qs.append(q[:, h * g:(h + 1) * g].contiguous())
        outs.append(torch.empty((b, g, 128), dtype=torch.float32, device=q.device))
    ws = _lib.alloc_decode_workspace(b, g, 1, plan1[1], q.device)

    def per_head():
        for h in range(num_kv_heads):
            _lib.nvfp4_decode(qs[h], pools[h], scales[h][0], scales[h][1], page_table, seq_lens, sm_scale, plan1, 1,
                              out=outs[h], workspace=ws)
        return outs
    _, us = _decode_timed(per_head)
    out = torch.cat(outs, dim=1)
    res["per_head"] = {"k_gscale": [s[0] for s in scales], "v_gscale": [s[1] for s in scales],
                       **errors(out, ref, num_kv_heads), "decode_us": us}
    return res

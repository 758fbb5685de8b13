"""Paged-cache set-up on the device: per-tensor scales (a1) and quantize-on-write (a2 / FP8).

Thin conveniences over the binding for callers that hold whole K/V tensors on the GPU.  The one
host synchronisation is reading the two per-tensor scales back, once, when a cache is created.
"""
from __future__ import annotations

import torch

from . import _lib


def build_nvfp4_cache(k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor, num_pages: int,
                      fill: int | None = 0, gscales=None):
    """Quantize k, v ([n][H_kv][128] bf16, GPU) to a new NVFP4 pool at `slots`.

    The global scales are fp32(max|x| / 2688) over k and over v unless `gscales` = (gk, gv) is
    given.  Returns (pool, gk, gv).
    """
    h_kv = k.shape[1]
    pool = _lib.alloc_nvfp4_pool(num_pages, h_kv, k.device, fill)
    if gscales is None:
        gk_t = _lib.global_scale(k)
        gv_t = _lib.global_scale(v)
        gk, gv = float(gk_t.item()), float(gv_t.item())
    else:
        gk, gv = gscales
    _lib.nvfp4_quantize_append(k, v, slots, gk, gv, pool)
    return pool, gk, gv


def build_fp8_cache(k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor, num_pages: int,
                    fill: int | None = 0, scales=None):
    """Quantize k, v to a new per-tensor-scaled FP8 pool; scales fp32(max|x| / 448).  Returns (pool, sk, sv)."""
    h_kv = k.shape[1]
    pool = _lib.alloc_fp8_pool(num_pages, h_kv, k.device, fill)
    if scales is None:
        sk = float(_lib.global_scale(k, divisor=_lib.FP8_DIVISOR).item())
        sv = float(_lib.global_scale(v, divisor=_lib.FP8_DIVISOR).item())
    else:
        sk, sv = scales
    _lib.fp8_quantize_append(k, v, slots, sk, sv, pool)
    return pool, sk, sv

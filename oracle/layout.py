"""Where each byte of a token lives in the paged pools (oracle, test infrastructure).

The pages fix the format (two E2M1 codes per byte, one E4M3 scale per 16
values) and that the cache is paged (SGLang x Qwen x NVIDIA story, "Three
Paths" paragraphs 1-3), not the order of bytes inside a page.  The order below
is this library's documented contract; the oracle restates it independently of
the GPU code, from the index formulas alone.

All pools are indexed [page][kv_head][block], one block per (page, head) for
16 tokens of head_dim 128.  ``o`` is the token's offset in its page
(slot = page * 16 + o), ``d`` the channel, ``j = d // 16`` the scale block.

NVFP4 K data  (1024 B)  byte ((d//32)*16 + o)*16 + (d%32)//2,   nibble d%2
NVFP4 K scale (128 B)   byte ((j//2)*16 + o)*2 + j%2
NVFP4 V data  (1024 B)  byte ((o//4)*16 + d%16)*16 + 2*(d//16) + (o%4)//2,  nibble o%2
NVFP4 V scale (128 B)   byte ((o//4)*8 + j)*4 + o%4
FP8   K       (2048 B)  byte ((d//32)*16 + o)*32 + d%32
FP8   V       (2048 B)  byte ((o//4)*16 + d%16)*32 + (d//16)*4 + o%4
nibble 0 is the low nibble.  In V data two tokens (o even, o+1) share a byte.
"""

from __future__ import annotations

import numpy as np

PAGE = 16
HEAD_DIM = 128
NVFP4_DATA_BYTES = PAGE * HEAD_DIM // 2     # 1024
NVFP4_SCALE_BYTES = PAGE * HEAD_DIM // 16   # 128
FP8_BYTES = PAGE * HEAD_DIM                 # 2048


def _idx_nvfp4_data(kind: str, o, d):
    o = np.asarray(o)
    d = np.asarray(d)
    if kind == "k":
        return ((d // 32) * 16 + o) * 16 + (d % 32) // 2, d % 2
    if kind == "v":
        return ((o // 4) * 16 + d % 16) * 16 + 2 * (d // 16) + (o % 4) // 2, o % 2
    raise ValueError(kind)


def _idx_nvfp4_scale(kind: str, o, j):
    o = np.asarray(o)
    j = np.asarray(j)
    if kind == "k":
        return ((j // 2) * 16 + o) * 2 + j % 2
    if kind == "v":
        return ((o // 4) * 8 + j) * 4 + o % 4
    raise ValueError(kind)


def _idx_fp8(kind: str, o, d):
    o = np.asarray(o)
    d = np.asarray(d)
    if kind == "k":
        return ((d // 32) * 16 + o) * 32 + d % 32
    if kind == "v":
        return ((o // 4) * 16 + d % 16) * 32 + (d // 16) * 4 + o % 4
    raise ValueError(kind)


def nvfp4_pool_shapes(num_pages: int, h_kv: int):
    """(data shape, scale shape) of one NVFP4 pool (K or V)."""
    return (num_pages, h_kv, NVFP4_DATA_BYTES), (num_pages, h_kv, NVFP4_SCALE_BYTES)


def fp8_pool_shape(num_pages: int, h_kv: int):
    return (num_pages, h_kv, FP8_BYTES)


def write_nvfp4_tokens(data, scale, kind, slots, codes, scale_bytes):
    """Store codes [N][H][128] and scale bytes [N][H][8] of N tokens at their slots.

    ``data``/``scale`` are uint8 pools shaped as :func:`nvfp4_pool_shapes`;
    they are modified in place.  Slots must be distinct.
    """
    slots = np.asarray(slots, dtype=np.int64)
    n, h, d = codes.shape
    assert d == HEAD_DIM and scale_bytes.shape == (n, h, d // 16)
    page = slots // PAGE
    o = slots % PAGE
    heads = np.arange(h)
    dd = np.arange(d)
    jj = np.arange(d // 16)
    bidx, nib = _idx_nvfp4_data(kind, o[:, None, None], dd[None, None, :])
    bidx = np.broadcast_to(bidx, (n, h, d))
    nib = np.broadcast_to(nib, (n, h, d))
    pg = np.broadcast_to(page[:, None, None], (n, h, d))
    hh = np.broadcast_to(heads[None, :, None], (n, h, d))
    # nibble writes: do low and high nibbles in separate passes so that no two
    # writes of one pass touch the same byte
    for which in (0, 1):
        m = nib == which
        b = data[pg[m], hh[m], bidx[m]]
        v = codes[m] & 0xF
        if which == 0:
            b = (b & 0xF0) | v
        else:
            b = (b & 0x0F) | (v << 4)
        data[pg[m], hh[m], bidx[m]] = b
    sidx = _idx_nvfp4_scale(kind, o[:, None, None], jj[None, None, :])
    sidx = np.broadcast_to(sidx, (n, h, d // 16))
    pg = np.broadcast_to(page[:, None, None], (n, h, d // 16))
    hh = np.broadcast_to(heads[None, :, None], (n, h, d // 16))
    scale[pg, hh, sidx] = scale_bytes


def read_nvfp4_tokens(data, scale, kind, slots):
    """Codes [N][H][128] and scale bytes [N][H][8] of the tokens at ``slots``."""
    slots = np.asarray(slots, dtype=np.int64)
    h = data.shape[1]
    page = slots // PAGE
    o = slots % PAGE
    dd = np.arange(HEAD_DIM)
    jj = np.arange(HEAD_DIM // 16)
    bidx, nib = _idx_nvfp4_data(kind, o[:, None, None], dd[None, None, :])
    heads = np.arange(h)[None, :, None]
    b = data[page[:, None, None], heads, bidx]
    codes = ((b >> (4 * nib)) & 0xF).astype(np.uint8)
    sidx = _idx_nvfp4_scale(kind, o[:, None, None], jj[None, None, :])
    sc = scale[page[:, None, None], heads, sidx].astype(np.uint8)
    return codes, sc


def write_fp8_tokens(cache, kind, slots, codes):
    """Store E4M3 bytes [N][H][128] of N tokens at their slots (in place)."""
    slots = np.asarray(slots, dtype=np.int64)
    n, h, d = codes.shape
    page = slots // PAGE
    o = slots % PAGE
    idx = _idx_fp8(kind, o[:, None, None], np.arange(d)[None, None, :])
    cache[page[:, None, None], np.arange(h)[None, :, None], idx] = codes


def read_fp8_tokens(cache, kind, slots):
    slots = np.asarray(slots, dtype=np.int64)
    h = cache.shape[1]
    page = slots // PAGE
    o = slots % PAGE
    idx = _idx_fp8(kind, o[:, None, None], np.arange(HEAD_DIM)[None, None, :])
    return cache[page[:, None, None], np.arange(h)[None, :, None], idx].astype(np.uint8)


def sequence_slots(page_table_row, length: int) -> np.ndarray:
    """Slots of tokens 0..length-1 of a sequence: page_table[t // 16] * 16 + t % 16."""
    t = np.arange(length, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[t // PAGE]
    return pages * PAGE + t % PAGE

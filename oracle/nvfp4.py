"""NVFP4 two-level quantization, step by step (oracle, test infrastructure).

Follows the SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "The Core of the
Ledger: 4-bit Does Not Equal 2x" paragraph 1 (E2M1 values, one E4M3 scale per
16 values, one FP32 scale per tensor) and "The Ledger of 4-bit KV Cache"
bullet 1 (16 values take 8 packed bytes + 1 scale byte), and SOAR Notes 05,
"02 NVFP4 KV Cache" (two values packed per byte; dequantization multiplies by
the scale).

Readings of points the pages leave open (each repeated where it is applied):

* R1  a block is 16 consecutive channels of one (token, head) row;
* R2  scales multiply on dequantization: x_hat = e2m1 * s_block * g;
* R3  the global scale is g = fp32(amax / 2688), 2688 = 6 * 448, one per tensor
      (per layer, separately for K and V), set once and reused by appends;
* R5  the block scale is u = fp32(a / fp32(6 * g)) rounded to E4M3 by RNE with
      saturation, a = max |x| over the block;
* R6  element codes come from y = fp32(x / fp32(s * g)) (correctly rounded fp32
      division) rounded to E2M1 by RNE with saturation;
* R7  the sign bit is copied from x, also when the magnitude rounds to zero;
      a block whose scale rounds to zero stores signed zeros;
* R8  in the packed form element 2i goes to the low nibble of byte i, element
      2i+1 to the high one (where each byte sits in a page is the layout's
      business, see ``layout``).
"""

from __future__ import annotations

import numpy as np

from .codecs import e2m1_decode, e2m1_encode_magnitude, e4m3_decode, e4m3_encode

BLOCK = 16
GLOBAL_DIVISOR = np.float32(6.0 * 448.0)  # amax / (6 * 448): E2M1 max times E4M3 max


def global_scale(x) -> np.float32:
    """R3: g = fp32(max |x| / 2688) over the whole tensor (fp32 division, correctly rounded)."""
    a = np.max(np.abs(np.asarray(x, dtype=np.float32)))
    return np.float32(np.float32(a) / GLOBAL_DIVISOR)


def quantize_blocks(x, g):
    """Quantize rows of fp32 values into E2M1 codes and E4M3 block-scale bytes.

    ``x``: fp32 array [..., D] with D a multiple of 16 (R1: blocks run along the
    last axis).  ``g``: the fp32 global scale (> 0, finite).
    Returns (codes uint8 [..., D] with the sign in bit 3, scale bytes uint8 [..., D/16]).
    Blocks are independent; large inputs are processed a slice of blocks at a time.
    """
    x = np.asarray(x, dtype=np.float32)
    g = np.float32(g)
    if not (np.isfinite(g) and g > 0):
        raise ValueError("global scale must be finite and > 0")
    d = x.shape[-1]
    if d % BLOCK:
        raise ValueError("last axis must be a multiple of 16")
    flat = x.reshape(-1, BLOCK)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty(flat.shape[0], dtype=np.uint8)
    step = 1 << 16
    for s in range(0, flat.shape[0], step):
        codes[s:s + step], scales[s:s + step] = _quantize_block_rows(flat[s:s + step], g)
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1] + (d // BLOCK,))


def _quantize_block_rows(xb, g):
    """Blocks [n][16] -> (codes [n][16], scale bytes [n]); the steps R5, R6, R7."""
    # R5: block amax -> u = a / fp32(6 g) -> E4M3 (RNE, saturating)
    a = np.max(np.abs(xb), axis=-1)
    six_g = np.float32(np.float32(6.0) * g)
    u = (a / six_g).astype(np.float32)
    scale_bytes = e4m3_encode(u)
    s = e4m3_decode(scale_bytes).astype(np.float32)       # exact: E4M3 values are fp32 values
    # R6: y = x / fp32(s g), correctly rounded fp32 division -> E2M1 (RNE, saturating)
    den = (s * g).astype(np.float32)
    zero_scale = s == 0
    safe_den = np.where(zero_scale, np.float32(1.0), den).astype(np.float32)
    y = (xb / safe_den[..., None]).astype(np.float32)
    mag = e2m1_encode_magnitude(np.abs(y))
    mag = np.where(zero_scale[..., None], np.uint8(0), mag).astype(np.uint8)
    # R7: sign copied from x
    sign = np.signbit(xb).astype(np.uint8) << 3
    return mag | sign, scale_bytes


def dequantize_blocks(codes, scale_bytes, g) -> np.ndarray:
    """R2: x_hat = e2m1(code) * e4m3(scale) * g, in fp64 (exact: at most 2 + 4 + 24 significant bits)."""
    codes = np.asarray(codes, dtype=np.uint8)
    d = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (d // BLOCK, BLOCK))
    s = e4m3_decode(scale_bytes)[..., None]
    return (vals * s * np.float64(np.float32(g))).reshape(codes.shape)


def pack_nibbles(codes) -> np.ndarray:
    """R8: two 4-bit codes per byte, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def bytes_per_values(n_values: int) -> int:
    """Storage of n values (n a multiple of 16): n/2 packed bytes + n/16 scale bytes ("9 bytes per 16")."""
    if n_values % BLOCK:
        raise ValueError("n must be a multiple of 16")
    return n_values // 2 + n_values // BLOCK

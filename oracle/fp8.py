"""FP8 E4M3 KV (sensitive layers) and the NVFP4 -> FP8 workspace transcode (oracle, test infrastructure).

* SOAR Notes 05, "03 Mixed-precision KV Cache": the most sensitive layers (the
  first and the last few) keep an FP8 KV cache, the rest use NVFP4.
* SGLang x Qwen x NVIDIA story, "Three Paths" paragraph 2: for chunked
  prefill / extend the cached prefix is gathered and dequantized into a
  cross-layer shared FP8 workspace, then joined with the chunk's FP8 K/V.

Readings (repeated in the design notes):

* R13 the FP8 cache is per-tensor scaled: s = fp32(amax / 448); a value is
      stored as E4M3(fp32(x / s)) (RNE, saturating, sign kept) and read back as
      e4m3 * s;
* R14 the workspace uses the FP8 scale of the layer (passed in, ``s_ws``); each
      prefix value is first dequantized in fp32 -- v = fp32(fp32(e2m1 * s_blk) * g)
      -- then stored as E4M3(fp32(v / s_ws)) with the sign of its E2M1 code.
"""

from __future__ import annotations

import numpy as np

from .codecs import e2m1_decode, e4m3_decode, e4m3_encode

FP8_DIVISOR = np.float32(448.0)


def fp8_scale(x) -> np.float32:
    """R13: per-tensor scale s = fp32(max |x| / 448)."""
    a = np.max(np.abs(np.asarray(x, dtype=np.float32)))
    return np.float32(np.float32(a) / FP8_DIVISOR)


def fp8_quantize(x, s) -> np.ndarray:
    """R13: E4M3 byte of fp32(x / s) for every element (RNE, saturating, sign copied)."""
    x = np.asarray(x, dtype=np.float32)
    s = np.float32(s)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("FP8 scale must be finite and > 0")
    return e4m3_encode((x / s).astype(np.float32))


def fp8_dequantize(codes, s) -> np.ndarray:
    """x_hat = e4m3(code) * s in fp64 (exact)."""
    return e4m3_decode(codes) * np.float64(np.float32(s))


def nvfp4_to_fp8_workspace(codes, scale_bytes, g, s_ws) -> np.ndarray:
    """R14: FP8 workspace bytes for NVFP4 codes [..., D] with block-scale bytes [..., D/16]."""
    codes = np.asarray(codes, dtype=np.uint8)
    d = codes.shape[-1]
    e = e2m1_decode(codes).astype(np.float32)             # exact
    s = e4m3_decode(scale_bytes).astype(np.float32)       # exact
    es = (e.reshape(codes.shape[:-1] + (d // 16, 16)) * s[..., None]).astype(np.float32)  # exact (<= 6 bits)
    v = (es * np.float32(g)).astype(np.float32).reshape(codes.shape)    # one fp32 rounding
    w = (v / np.float32(s_ws)).astype(np.float32)                       # one fp32 rounding
    out = e4m3_encode(np.abs(w))
    sign = ((codes >> 3) & 1).astype(np.uint8) << 7                     # sign of the E2M1 code
    return out | sign

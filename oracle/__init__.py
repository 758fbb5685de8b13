"""CPU oracle for NVFP4 / FP8 paged-KV decode attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct statement of what the GPU
path computes.  It exists to check the HIP kernels; it is never part of the
product path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code, table
or constant with ``bit_paged_kv_amd`` and imports nothing from it.

Sources (the web pages this method is described on):

* "SGLang x Qwen x NVIDIA Collaboration: NVFP4 KV Cache Breaks Long-Context and
  Agentic Inference Bottlenecks" (ai.synthepulse.app story), sections
  "The Ledger of 4-bit KV Cache" (bullet 1: two-level scaling, 9 bytes per
  16 values), "The Core of the Ledger: 4-bit Does Not Equal 2x" (E2M1 values,
  one E4M3 scale per 16 values, one FP32 scale per tensor) and "Three Paths"
  (quantized write, FP8 workspace for extend, decode that reads NVFP4 and
  dequantizes on the fly).
* "SOAR Weekly Champion Notes 05: NVFP4 KV Cache and Mixed-Precision Practice"
  (openbmb.cn), sections "02 NVFP4 KV Cache" (E2M1 bit layout, two values per
  byte, dequantization multiplies by the scale) and "03 Mixed-precision KV
  Cache" (FP8 KV for the sensitive layers).

Modules:

* ``codecs``    -- E2M1 and OCP E4M3 decode tables and round-to-nearest-even
                   encoders, written from the format definitions.
* ``nvfp4``     -- global scale, block quantization, dequantization.
* ``fp8``       -- per-tensor FP8 quantization and the NVFP4 -> FP8 workspace
                   transcode used by chunked extend.
* ``layout``    -- where each byte of a token lives in the paged pools.
* ``attention`` -- fp64 softmax attention for one decode step.

Every function states which passage it follows.  Points the pages leave open
are resolved by the readings listed in the design notes; each is repeated in
the docstring of the function that applies it.  All functions here are pinned
by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.
"""

from . import codecs, nvfp4, fp8, layout, attention  # noqa: F401

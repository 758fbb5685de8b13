"""bit_paged_kv_amd: NVFP4 / FP8 paged KV cache for decode attention on MI355X (gfx950).

The product is the C-ABI library ``libnvkv.so`` (include/nvkv.h) built from the HIP kernels in
``csrc/``; this package is its thin Python binding (torch tensors in, raw pointers out).
"""
from ._lib import (  # noqa: F401
    EXPORTED, FP8_BYTES, FP8_DIVISOR, HEAD_DIM, LIB_PATH, NVFP4_DATA_BYTES, NVFP4_GLOBAL_DIVISOR,
    NVFP4_SCALE_BYTES, PAGE_SIZE, PREC_FP8, PREC_NVFP4, alloc_decode_workspace, alloc_fp8_pool, alloc_nvfp4_pool, decode_layers,
    decode_workspace_size, default_sm_scale, dequant_to_workspace, fp8_decode, fp8_extend_attn, fp8_quantize_append,
    fp8_workspace_append, global_scale, prepare_fp8_extend_attn, prepare_fp8_workspace_append,
    nvfp4_decode, nvfp4_decode_noalloc, decode_noalloc_max_bytes, nvfp4_pool_bytes, nvfp4_prefill_write, nvfp4_quantize_append, plan_decode, prepare_decode_layers,
    prepare_nvfp4_prefill_write,
    prepare_dequant_to_workspace, prepare_nvfp4_decode, prepare_nvfp4_quantize_append, read_probe, status_string,
    version,
    PreparedCall, PreparedDecode,
)

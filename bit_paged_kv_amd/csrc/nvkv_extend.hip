// The extend chunk's FP8 append to the shared workspace.
//
// SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "Three Paths" paragraph 2: an extend step gathers the
// cached NVFP4 prefix into an FP8 workspace (nvfp4_to_fp8_ws_kernel) and the new chunk's K/V join it
// there, after the prefix rows of their sequence; the attention over prefix || chunk is
// extend_attn_kernel (nvkv_extend_attn.hip).
#include <hip/hip_runtime.h>

#include "nvkv_device.h"
#include "nvkv_launch.h"

namespace nvkv {

// ---------------------------------------------------------------------------------------------
// Chunk K/V (bf16) -> FP8 workspace rows after each sequence's prefix: E4M3 of fp32(x / s), one
// thread per 16 values.  grid.y = sequence.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_ws_append_kernel(const uint8_t* __restrict__ k_in,
                                                            const uint8_t* __restrict__ v_in,
                                                            const int32_t* __restrict__ q_offsets,
                                                            const int32_t* __restrict__ ws_offsets,
                                                            const int32_t* __restrict__ prefix_lens, int hkv,
                                                            float sk, float sv, uint8_t* __restrict__ k_ws,
                                                            uint8_t* __restrict__ v_ws) {
  const int b = blockIdx.y;
  const int row0 = q_offsets[b];
  const int n = q_offsets[b + 1] - row0;
  const size_t groups = (size_t)max(n, 0) * hkv * 8;         // 16-value groups of one tensor
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 2 * groups) return;
  const bool is_v = idx >= groups;
  const size_t gi = is_v ? idx - groups : idx;
  const size_t tok = gi / ((size_t)hkv * 8);
  const size_t rest = gi - tok * hkv * 8;                      // head * 8 + group within the row
  float x[16];
  const uint4* src = reinterpret_cast<const uint4*>((is_v ? v_in : k_in) + (((size_t)row0 + tok) * hkv * 128 + rest * 16) * 2);
  bf16x8_to_f32(src[0], x);
  bf16x8_to_f32(src[1], x + 8);
  const float s = is_v ? sv : sk;
  const float r = 1.0f / s;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = e4m3x4_div(x + 4 * i, s, r);
  const size_t dst_row = (size_t)ws_offsets[b] + (size_t)prefix_lens[b] + tok;
  *reinterpret_cast<uint4*>((is_v ? v_ws : k_ws) + (dst_row * hkv * 128 + rest * 16)) =
      make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t launch_fp8_ws_append(const void* k, const void* v, const int32_t* q_offsets, const int32_t* ws_offsets,
                                const int32_t* prefix_lens, int batch, int hkv, int max_chunk, float sk, float sv,
                                uint8_t* k_ws, uint8_t* v_ws, hipStream_t stream) {
  const size_t threads = 2 * (size_t)max_chunk * hkv * 8;
  dim3 grid((unsigned)std::max<size_t>(1, (threads + 255) / 256), batch);
  hipLaunchKernelGGL(fp8_ws_append_kernel, grid, dim3(256), 0, stream, (const uint8_t*)k, (const uint8_t*)v, q_offsets,
                     ws_offsets, prefix_lens, hkv, sk, sv, k_ws, v_ws);
  return hipGetLastError();
}

}  // namespace nvkv

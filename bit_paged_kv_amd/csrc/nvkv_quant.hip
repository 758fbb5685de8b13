// Write-side kernels: per-tensor scale, NVFP4 / FP8 quantize-on-write into the paged pools, and the
// NVFP4 -> FP8 prefix gather used by chunked extend.
//
// SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "Three Paths" paragraphs 1-2: prefill and extend
// quantize K/V into the persistent NVFP4 cache; extend gathers the cached prefix and dequantizes it
// into a cross-layer shared FP8 workspace.  All kernels are memory-bound streaming passes.
#include "nvkv_device.h"
#include "nvkv_launch.h"

namespace nvkv {

// ---------------------------------------------------------------------------------------------
// Per-tensor absolute maximum -> scale = fp32(amax / divisor)
// ---------------------------------------------------------------------------------------------
// Non-negative bf16 / E4M3 magnitudes order like their bit patterns, so the maximum is taken on
// integers: (bits & 0x7FFF) for bf16, (byte & 0x7F) for E4M3.
__global__ __launch_bounds__(256) void amax_partial_kernel(const uint8_t* __restrict__ x, int in_dtype,
                                                           size_t n, uint32_t* __restrict__ partial) {
  const size_t elem_bytes = in_dtype == 0 ? 2 : 1;
  const size_t nbytes = n * elem_bytes;
  const size_t nvec = nbytes / 16;
  uint32_t m = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (size_t)gridDim.x * blockDim.x) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (in_dtype == 0) {
        m = max(m, w[k] & 0x7FFFu);
        m = max(m, (w[k] >> 16) & 0x7FFFu);
      } else {
        m = max(m, w[k] & 0x7Fu);
        m = max(m, (w[k] >> 8) & 0x7Fu);
        m = max(m, (w[k] >> 16) & 0x7Fu);
        m = max(m, (w[k] >> 24) & 0x7Fu);
      }
    }
  }
  if (blockIdx.x == 0) {  // tail bytes past the last 16-byte vector
    for (size_t byte = nvec * 16 + threadIdx.x * elem_bytes; byte < nbytes; byte += blockDim.x * elem_bytes) {
      uint32_t v = in_dtype == 0 ? (uint32_t)x[byte] | ((uint32_t)x[byte + 1] << 8) : (uint32_t)x[byte];
      m = max(m, in_dtype == 0 ? (v & 0x7FFFu) : (v & 0x7Fu));
    }
  }
  // block reduction: wave butterflies, then across the 4 waves through LDS
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
}

__global__ __launch_bounds__(256) void amax_finalize_kernel(const uint32_t* __restrict__ partial, int nblocks,
                                                            int in_dtype, float in_scale, float divisor,
                                                            float* __restrict__ out) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nblocks; i += blockDim.x) m = max(m, partial[i]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    const float amax = in_dtype == 0 ? __uint_as_float(m << 16) : e4m3_value(m) * in_scale;
    out[0] = amax / divisor;
  }
}

// ---------------------------------------------------------------------------------------------
// Input block loader: 16 consecutive channels of one (token, head) as fp32.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void load_block16(const uint8_t* base, int in_dtype, float in_scale, size_t elem_index,
                                             float (&x)[16]) {
  if (in_dtype == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(base + elem_index * 2);
    bf16x8_to_f32(p[0], x);
    bf16x8_to_f32(p[1], x + 8);
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(base + elem_index);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b = (w[k] >> (8 * i)) & 0xFFu;
        const float mag = e4m3_value(b & 0x7Fu) * in_scale;
        x[4 * k + i] = (b & 0x80u) ? -mag : mag;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// NVFP4 quantize-append: one thread per (token, head, 16-channel block); blockIdx.y = 0 K, 1 V.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(
    const uint8_t* __restrict__ k_in, const uint8_t* __restrict__ v_in, int in_dtype, float k_in_scale,
    float v_in_scale, const int32_t* __restrict__ slots, int n_tok, int hkv, float gk, float gv,
    uint8_t* __restrict__ k_data, uint8_t* __restrict__ k_scale, uint8_t* __restrict__ v_data,
    uint8_t* __restrict__ v_scale) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)n_tok * hkv * 8) return;
  const bool is_v = blockIdx.y == 1;
  const int j = (int)(idx & 7);
  const size_t th = idx >> 3;
  const int h = (int)(th % hkv);
  const size_t t = th / hkv;
  float x[16];
  load_block16(is_v ? v_in : k_in, in_dtype, is_v ? v_in_scale : k_in_scale, (th * 128) + 16 * j, x);
  uint32_t codes[16];
  const uint32_t sc = nvfp4_quantize_block(x, is_v ? gv : gk, codes);
  const int slot = slots[t];
  const int o = slot & 15;
  const size_t blk = (size_t)(slot >> 4) * hkv + h;
  if (!is_v) {
    // 8 contiguous bytes: ((j/2)*16 + o)*16 + 8*(j%2)
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) lo |= codes[i] << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hi |= codes[8 + i] << (4 * i);
    uint2* dst = reinterpret_cast<uint2*>(k_data + blk * kNvfp4DataBytes + ((j >> 1) * 16 + o) * 16 + 8 * (j & 1));
    *dst = make_uint2(lo, hi);
    k_scale[blk * kNvfp4ScaleBytes + ((j >> 1) * 16 + o) * 2 + (j & 1)] = (uint8_t)sc;
  } else {
    // channel d = 16j + i sits in byte ((o/4)*16 + i)*16 + 2j + (o%4)/2, nibble o%2; the other
    // nibble of that byte belongs to token o^1, so update ours with two word atomics.
    uint8_t* base = v_data + blk * kNvfp4DataBytes;
    const int shift_in_byte = 4 * (o & 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const size_t byte = (size_t)(((o >> 2) * 16 + i) * 16 + 2 * j + ((o & 3) >> 1));
      unsigned int* word = reinterpret_cast<unsigned int*>(base + (byte & ~(size_t)3));
      const int shift = (int)(byte & 3) * 8 + shift_in_byte;
      atomicAnd(word, ~(0xFu << shift));
      atomicOr(word, codes[i] << shift);
    }
    v_scale[blk * kNvfp4ScaleBytes + ((o >> 2) * 8 + j) * 4 + (o & 3)] = (uint8_t)sc;
  }
}

// ---------------------------------------------------------------------------------------------
// FP8 quantize-append (per-tensor scale): one thread per (token, head, 16-channel block).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_quantize_kernel(
    const uint8_t* __restrict__ k_in, const uint8_t* __restrict__ v_in, const int32_t* __restrict__ slots,
    int n_tok, int hkv, float sk, float sv, uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)n_tok * hkv * 8) return;
  const bool is_v = blockIdx.y == 1;
  const int j = (int)(idx & 7);
  const size_t th = idx >> 3;
  const int h = (int)(th % hkv);
  const size_t t = th / hkv;
  float x[16];
  load_block16(is_v ? v_in : k_in, 0, 1.0f, th * 128 + 16 * j, x);
  const float s = is_v ? sv : sk;
  uint32_t b[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) b[i] = e4m3_encode(x[i] / s);
  const int slot = slots[t];
  const int o = slot & 15;
  const size_t blk = (size_t)(slot >> 4) * hkv + h;
  if (!is_v) {
    uint4 w;
    w.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    w.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    w.z = b[8] | (b[9] << 8) | (b[10] << 16) | (b[11] << 24);
    w.w = b[12] | (b[13] << 8) | (b[14] << 16) | (b[15] << 24);
    *reinterpret_cast<uint4*>(k_cache + blk * kFp8Bytes + ((j >> 1) * 16 + o) * 32 + 16 * (j & 1)) = w;
  } else {
    uint8_t* base = v_cache + blk * kFp8Bytes;
#pragma unroll
    for (int i = 0; i < 16; ++i) base[((o >> 2) * 16 + i) * 32 + j * 4 + (o & 3)] = (uint8_t)b[i];
  }
}

// ---------------------------------------------------------------------------------------------
// NVFP4 prefix -> dense FP8 workspace.  One thread per (prefix token, head, block); grid.y = seq.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t transcode_e2m1(uint32_t code, float s, float g, float s_ws) {
  // magnitude codes 0..3 are 0, .5, 1, 1.5 (= code / 2); 4..7 are (2 + m) * 2^(e - 2) = 2, 3, 4, 6
  const float mag_e2m1 = (code & 4u) ? __builtin_ldexpf((float)(2u + (code & 1u)), (int)((code >> 1) & 3u) - 2)
                                     : 0.5f * (float)(code & 3u);
  const float es = mag_e2m1 * s;          // exact: at most 6 significant bits
  const float v = es * g;                 // one rounding
  const float w = v / s_ws;               // one rounding (correctly rounded division)
  return e4m3_encode(w) | ((code & 8u) << 4);
}

__global__ __launch_bounds__(256) void nvfp4_to_fp8_ws_kernel(
    const uint8_t* __restrict__ k_data, const uint8_t* __restrict__ k_scale, const uint8_t* __restrict__ v_data,
    const uint8_t* __restrict__ v_scale, float gk, float gv, const int32_t* __restrict__ page_table, int max_pages,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ ws_offsets, int hkv, int max_prefix,
    float sk_ws, float sv_ws, uint8_t* __restrict__ k_ws, uint8_t* __restrict__ v_ws) {
  const int b = blockIdx.y;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int len = min(prefix_lens[b], max_prefix);
  if (idx >= (size_t)len * hkv * 8) return;
  const bool is_v = blockIdx.z == 1;
  const int j = (int)(idx & 7);
  const size_t th = idx >> 3;
  const int h = (int)(th % hkv);
  const int t = (int)(th / hkv);
  const int page = page_table[(size_t)b * max_pages + (t >> 4)];
  const int o = t & 15;
  const size_t blk = (size_t)page * hkv + h;
  uint32_t out[16];
  if (!is_v) {
    const uint2 w = *reinterpret_cast<const uint2*>(k_data + blk * kNvfp4DataBytes + ((j >> 1) * 16 + o) * 16 + 8 * (j & 1));
    const float s = e4m3_value(k_scale[blk * kNvfp4ScaleBytes + ((j >> 1) * 16 + o) * 2 + (j & 1)] & 0x7Fu);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = transcode_e2m1((w.x >> (4 * i)) & 0xFu, s, gk, sk_ws);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[8 + i] = transcode_e2m1((w.y >> (4 * i)) & 0xFu, s, gk, sk_ws);
  } else {
    const uint8_t* base = v_data + blk * kNvfp4DataBytes;
    const float s = e4m3_value(v_scale[blk * kNvfp4ScaleBytes + ((o >> 2) * 8 + j) * 4 + (o & 3)] & 0x7Fu);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t byte = base[((o >> 2) * 16 + i) * 16 + 2 * j + ((o & 3) >> 1)];
      out[i] = transcode_e2m1((byte >> (4 * (o & 1))) & 0xFu, s, gv, sv_ws);
    }
  }
  uint4 w;
  w.x = out[0] | (out[1] << 8) | (out[2] << 16) | (out[3] << 24);
  w.y = out[4] | (out[5] << 8) | (out[6] << 16) | (out[7] << 24);
  w.z = out[8] | (out[9] << 8) | (out[10] << 16) | (out[11] << 24);
  w.w = out[12] | (out[13] << 8) | (out[14] << 16) | (out[15] << 24);
  uint8_t* dst = (is_v ? v_ws : k_ws) + ((size_t)(ws_offsets[b] + t) * hkv + h) * kHeadDim + 16 * j;
  *reinterpret_cast<uint4*>(dst) = w;
}

// ---------------------------------------------------------------------------------------------
// launchers (validated arguments only; called from the C ABI layer)
// ---------------------------------------------------------------------------------------------
constexpr int kAmaxBlocks = 1024;

size_t global_scale_workspace_bytes() { return kAmaxBlocks * sizeof(uint32_t); }

hipError_t launch_global_scale(const void* x, int in_dtype, float in_scale, size_t n, float divisor, float* out,
                               void* workspace, hipStream_t stream) {
  const size_t nbytes = n * (in_dtype == 0 ? 2 : 1);
  int blocks = (int)std::min<size_t>(kAmaxBlocks, std::max<size_t>(1, (nbytes / 16 + 255) / 256));
  hipLaunchKernelGGL(amax_partial_kernel, dim3(blocks), dim3(256), 0, stream, (const uint8_t*)x, in_dtype, n,
                     (uint32_t*)workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(256), 0, stream, (const uint32_t*)workspace, blocks,
                     in_dtype, in_scale, divisor, out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_quantize(const void* k_in, const void* v_in, int in_dtype, float k_in_scale, float v_in_scale,
                                 const int32_t* slots, int n_tok, int hkv, float gk, float gv, uint8_t* k_data,
                                 uint8_t* k_scale, uint8_t* v_data, uint8_t* v_scale, hipStream_t stream) {
  const size_t threads = (size_t)n_tok * hkv * 8;
  dim3 grid((unsigned)((threads + 255) / 256), 2);
  hipLaunchKernelGGL(nvfp4_quantize_kernel, grid, dim3(256), 0, stream, (const uint8_t*)k_in, (const uint8_t*)v_in,
                     in_dtype, k_in_scale, v_in_scale, slots, n_tok, hkv, gk, gv, k_data, k_scale, v_data, v_scale);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void* k_in, const void* v_in, const int32_t* slots, int n_tok, int hkv, float sk,
                               float sv, uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream) {
  const size_t threads = (size_t)n_tok * hkv * 8;
  dim3 grid((unsigned)((threads + 255) / 256), 2);
  hipLaunchKernelGGL(fp8_quantize_kernel, grid, dim3(256), 0, stream, (const uint8_t*)k_in, (const uint8_t*)v_in,
                     slots, n_tok, hkv, sk, sv, k_cache, v_cache);
  return hipGetLastError();
}

hipError_t launch_dequant_to_ws(const uint8_t* k_data, const uint8_t* k_scale, const uint8_t* v_data,
                                const uint8_t* v_scale, float gk, float gv, const int32_t* page_table, int max_pages,
                                const int32_t* prefix_lens, const int32_t* ws_offsets, int batch, int hkv,
                                int max_prefix, float sk_ws, float sv_ws, uint8_t* k_ws, uint8_t* v_ws,
                                hipStream_t stream) {
  const size_t threads = (size_t)max_prefix * hkv * 8;
  dim3 grid((unsigned)((threads + 255) / 256), batch, 2);
  hipLaunchKernelGGL(nvfp4_to_fp8_ws_kernel, grid, dim3(256), 0, stream, k_data, k_scale, v_data, v_scale, gk, gv,
                     page_table, max_pages, prefix_lens, ws_offsets, hkv, max_prefix, sk_ws, sv_ws, k_ws, v_ws);
  return hipGetLastError();
}

}  // namespace nvkv

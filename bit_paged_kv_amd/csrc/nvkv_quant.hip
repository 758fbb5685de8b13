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
// The four lanes of a lane quad take four consecutive input tokens of one (head, block).
//
// In V data two tokens share each byte, so V bytes can be written with plain stores only by a
// writer that owns every token in them.  When the four tokens of a lane quad fill one aligned token
// quad of one page (slots s, s+1, s+2, s+3 with s % 4 == 0: the usual case for a prefill or extend
// chunk) the lanes merge their nibbles with lane swaps and own the quad's V bits of their block: one
// 16-bit store per channel row and one 32-bit store for the four scales.  Otherwise (single appended
// tokens, chunks that start mid-quad) each token's nibbles are merged into their bytes with atomic
// word updates.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bool aligned_quad(const int32_t* slots, int t0, int nt) {
  if (nt != 4) return false;
  const int s0 = slots[t0];
  return (s0 & 3) == 0 && slots[t0 + 1] == s0 + 1 && slots[t0 + 2] == s0 + 2 && slots[t0 + 3] == s0 + 3;
}

// OR of a value over the four lanes of a lane quad (DPP quad permutations xor 1, xor 2)
__device__ __forceinline__ uint32_t quad_or(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  return v;
}

__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(
    const uint8_t* __restrict__ k_in, const uint8_t* __restrict__ v_in, int in_dtype, float k_in_scale,
    float v_in_scale, const int32_t* __restrict__ slots, int n_tok, int hkv, float gk, float gv,
    uint8_t* __restrict__ k_data, uint8_t* __restrict__ k_scale, uint8_t* __restrict__ v_data,
    uint8_t* __restrict__ v_scale) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n_groups = ((size_t)n_tok + 3) / 4;
  if (idx >= n_groups * hkv * 32) return;          // a multiple of 4: lane quads stay whole
  const bool is_v = blockIdx.y == 1;
  const int k = (int)(idx & 3);                    // token within the group
  const int j = (int)((idx >> 2) & 7);
  const size_t gh = idx >> 5;
  const int h = (int)(gh % hkv);
  const int t0 = (int)(gh / hkv) * 4;
  const int nt = min(4, n_tok - t0);
  const int t = t0 + k;
  const bool has_token = k < nt;
  float x[16];
  uint32_t codes[16];
  uint32_t sc = 0;
  int slot = 0;
  if (has_token) {
    load_block16(is_v ? v_in : k_in, in_dtype, is_v ? v_in_scale : k_in_scale, ((size_t)t * hkv + h) * 128 + 16 * j, x);
    sc = nvfp4_quantize_block(x, is_v ? gv : gk, codes);
    slot = slots[t];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) codes[i] = 0;
  }
  const int o = slot & 15;
  const size_t blk = (size_t)(slot >> 4) * hkv + h;
  if (!is_v) {
    if (!has_token) return;
    // 8 contiguous bytes: ((j/2)*16 + o)*16 + 8*(j%2)
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) lo |= codes[i] << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hi |= codes[8 + i] << (4 * i);
    *reinterpret_cast<uint2*>(k_data + blk * kNvfp4DataBytes + ((j >> 1) * 16 + o) * 16 + 8 * (j & 1)) =
        make_uint2(lo, hi);
    k_scale[blk * kNvfp4ScaleBytes + ((j >> 1) * 16 + o) * 2 + (j & 1)] = (uint8_t)sc;
    return;
  }
  if (aligned_quad(slots, t0, nt)) {           // uniform over the lane quad
    // channel row r of token quad o/4: the 16-bit word at ((o/4)*16 + r)*16 + 2j holds the nibbles
    // of tokens 4(o/4) .. +3 in bits 0-3, 4-7, 8-11, 12-15
    uint32_t rows[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) rows[i] = quad_or(codes[i] << (4 * k));
    const uint32_t scales = quad_or(sc << (8 * k));
    uint8_t* base = v_data + blk * kNvfp4DataBytes + (o >> 2) * 256 + 2 * j;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint16_t*>(base + (4 * k + i) * 16) = (uint16_t)rows[4 * k + i];
    if (k == 0) *reinterpret_cast<uint32_t*>(v_scale + blk * kNvfp4ScaleBytes + ((o >> 2) * 8 + j) * 4) = scales;
    return;
  }
  if (!has_token) return;
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

// ---------------------------------------------------------------------------------------------
// FP8 quantize-append (per-tensor scale): one thread per (group of four input tokens, head,
// 16-channel block).  For an aligned token quad the four V bytes of each channel row are adjacent
// and go out as one 32-bit store.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fp8_quantize_kernel(
    const uint8_t* __restrict__ k_in, const uint8_t* __restrict__ v_in, const int32_t* __restrict__ slots,
    int n_tok, int hkv, float sk, float sv, uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n_groups = ((size_t)n_tok + 3) / 4;
  if (idx >= n_groups * hkv * 8) return;
  const bool is_v = blockIdx.y == 1;
  const int j = (int)(idx & 7);
  const size_t gh = idx >> 3;
  const int h = (int)(gh % hkv);
  const int t0 = (int)(gh / hkv) * 4;
  const int nt = min(4, n_tok - t0);
  const float s = is_v ? sv : sk;
  const bool quad = is_v && aligned_quad(slots, t0, nt);
  uint32_t rows[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) rows[i] = 0;
  for (int k = 0; k < nt; ++k) {
    const size_t t = (size_t)t0 + k;
    float x[16];
    load_block16(is_v ? v_in : k_in, 0, 1.0f, (t * hkv + h) * 128 + 16 * j, x);
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
    } else if (quad) {
#pragma unroll
      for (int i = 0; i < 16; ++i) rows[i] |= b[i] << (8 * k);
    } else {
      uint8_t* base = v_cache + blk * kFp8Bytes;
#pragma unroll
      for (int i = 0; i < 16; ++i) base[((o >> 2) * 16 + i) * 32 + j * 4 + (o & 3)] = (uint8_t)b[i];
    }
  }
  if (quad) {
    const int s0 = slots[t0];
    uint8_t* base = v_cache + ((size_t)(s0 >> 4) * hkv + h) * kFp8Bytes + ((s0 & 15) >> 2) * 512 + j * 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<uint32_t*>(base + i * 32) = rows[i];
  }
}

// ---------------------------------------------------------------------------------------------
// NVFP4 prefix -> dense FP8 workspace.  One thread per (prefix token quad, head, block);
// grid.y = sequence, grid.z = 0 K, 1 V.
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

// Eight 4-bit codes that share one block scale -> their eight workspace bytes, from the 8-byte
// table row of that scale (byte m = output for magnitude m): two byte permutations look up the
// even and the odd codes, the code signs are copied to bit 7, two more permutations interleave.
__device__ __forceinline__ uint2 ws_bytes8(uint2 row, uint32_t w) {
  const uint32_t ev = __builtin_amdgcn_perm(row.y, row.x, w & 0x07070707u) | ((w & 0x08080808u) << 4);
  const uint32_t od = __builtin_amdgcn_perm(row.y, row.x, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
  return make_uint2(__builtin_amdgcn_perm(od, ev, 0x05010400u), __builtin_amdgcn_perm(od, ev, 0x07030602u));
}

// One wavefront per (prefix page, head), K and V: every lane loads 16 bytes of the page's K and of
// its V (the decode kernel's access pattern) and ends up with 32 consecutive channels of one token
// (token lane % 16, channels 32 (lane / 16) .. +31, i.e. two blocks), looks their codes up in the
// per-scale tables and writes 32 contiguous workspace bytes.  K arrives in that order; V (channel
// rows of token quads) is staged in a per-wave LDS slot and regathered.  grid.y = sequence.
constexpr int kWsWaves = 16;   // 1024 threads: two table entries each
__global__ __launch_bounds__(64 * kWsWaves) void nvfp4_to_fp8_ws_kernel(
    const uint8_t* __restrict__ k_data, const uint8_t* __restrict__ k_scale, const uint8_t* __restrict__ v_data,
    const uint8_t* __restrict__ v_scale, float gk, float gv, const int32_t* __restrict__ page_table, int max_pages,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ ws_offsets, int hkv, int max_prefix,
    float sk_ws, float sv_ws, uint8_t* __restrict__ k_ws, uint8_t* __restrict__ v_ws) {
  // The workspace byte of every E2M1 magnitude under every non-negative E4M3 block scale (128 x 8),
  // for K and V: each workgroup transcodes these 2048 cases once instead of dividing per value.
  __shared__ uint2 lut[2][128];
  __shared__ uint4 stage[kWsWaves][64];
  for (int e = threadIdx.x; e < 2048; e += blockDim.x) {
    const bool v = e >= 1024;
    reinterpret_cast<uint8_t*>(lut)[e] = (uint8_t)transcode_e2m1((uint32_t)(e & 7), e4m3_value((uint32_t)((e >> 3) & 127)),
                                                                 v ? gv : gk, v ? sv_ws : sk_ws);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int len = min(prefix_lens[b], max_prefix);
  const int units = ((len + 15) >> 4) * hkv;
  const size_t off = (size_t)ws_offsets[b];
  const size_t row_bytes = (size_t)hkv * kHeadDim;
  const int o = lane & 15, grp = lane >> 4;                // token and 32-channel group of this lane
  const int q = o >> 2, k = o & 3;
  const uint8_t* vst = reinterpret_cast<const uint8_t*>(stage[wave]);
  for (int u = blockIdx.x * kWsWaves + wave; u < units; u += gridDim.x * kWsWaves) {
    const int p = u / hkv, h = u - p * hkv;
    const int page = page_table[(size_t)b * max_pages + p];
    const int nv = min(16, len - 16 * p);
    const size_t blk = (size_t)page * hkv + h;
    const uint4 kd = *reinterpret_cast<const uint4*>(k_data + blk * kNvfp4DataBytes + lane * 16);
    const uint32_t ks = *reinterpret_cast<const uint16_t*>(k_scale + blk * kNvfp4ScaleBytes + lane * 2);
    const uint4 vd = *reinterpret_cast<const uint4*>(v_data + blk * kNvfp4DataBytes + lane * 16);
    // V scales of this token for blocks 2 grp, 2 grp + 1: bytes ((q*8 + n)*4 + k)
    const uint8_t* vsb = v_scale + blk * kNvfp4ScaleBytes + (q * 8 + 2 * grp) * 4 + k;
    const uint32_t vs_a = vsb[0], vs_b = vsb[4];
    // K: already token-major
    const uint2 r0 = lut[0][ks & 0x7Fu], r1 = lut[0][(ks >> 8) & 0x7Fu];
    const uint2 ka = ws_bytes8(r0, kd.x), kb = ws_bytes8(r0, kd.y), kc = ws_bytes8(r1, kd.z), ke = ws_bytes8(r1, kd.w);
    // V: byte ((o/4)*16 + r)*16 + 4 grp + i of the page holds channel 32 grp + 16 (i/2) + r for tokens
    // 4q + 2(i%2) + {0, 1}; the 32-bit word at 4 grp therefore has token k's nibble of channel
    // 32 grp + r in bits 4k and of channel 32 grp + 16 + r in bits 16 + 4k
    stage[wave][lane] = vd;                  // LDS operations of one wave complete in order
    uint32_t va0 = 0, va1 = 0, vb0 = 0, vb1 = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(vst + (q * 16 + r) * 16 + 4 * grp);
      const uint32_t na = (w >> (4 * k)) & 0xFu, nb = (w >> (16 + 4 * k)) & 0xFu;
      if (r < 8) {
        va0 |= na << (4 * r);
        vb0 |= nb << (4 * r);
      } else {
        va1 |= na << (4 * (r - 8));
        vb1 |= nb << (4 * (r - 8));
      }
    }
    const uint2 s0 = lut[1][vs_a & 0x7Fu], s1 = lut[1][vs_b & 0x7Fu];
    const uint2 va = ws_bytes8(s0, va0), vb = ws_bytes8(s0, va1), vc = ws_bytes8(s1, vb0), ve = ws_bytes8(s1, vb1);
    if (o < nv) {
      const size_t row = (off + 16 * p + o) * row_bytes + (size_t)h * kHeadDim + 32 * grp;
      *reinterpret_cast<uint4*>(k_ws + row) = make_uint4(ka.x, ka.y, kb.x, kb.y);
      *reinterpret_cast<uint4*>(k_ws + row + 16) = make_uint4(kc.x, kc.y, ke.x, ke.y);
      *reinterpret_cast<uint4*>(v_ws + row) = make_uint4(va.x, va.y, vb.x, vb.y);
      *reinterpret_cast<uint4*>(v_ws + row + 16) = make_uint4(vc.x, vc.y, ve.x, ve.y);
    }
  }
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
  const size_t threads = (((size_t)n_tok + 3) / 4) * hkv * 32;
  dim3 grid((unsigned)((threads + 255) / 256), 2);
  hipLaunchKernelGGL(nvfp4_quantize_kernel, grid, dim3(256), 0, stream, (const uint8_t*)k_in, (const uint8_t*)v_in,
                     in_dtype, k_in_scale, v_in_scale, slots, n_tok, hkv, gk, gv, k_data, k_scale, v_data, v_scale);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void* k_in, const void* v_in, const int32_t* slots, int n_tok, int hkv, float sk,
                               float sv, uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream) {
  const size_t threads = (((size_t)n_tok + 3) / 4) * hkv * 8;
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
  // one wave per (page, head); a few pages per wave so that each workgroup's tables serve many
  const size_t units = (((size_t)max_prefix + 15) / 16) * hkv;
  const size_t want = (units + kWsWaves - 1) / kWsWaves;
  const size_t cap = std::max<size_t>(1, 512 / (size_t)batch);
  dim3 grid((unsigned)std::max<size_t>(1, std::min(want, cap)), batch);
  hipLaunchKernelGGL(nvfp4_to_fp8_ws_kernel, grid, dim3(64 * kWsWaves), 0, stream, k_data, k_scale, v_data, v_scale,
                     gk, gv, page_table, max_pages, prefix_lens, ws_offsets, hkv, max_prefix, sk_ws, sv_ws, k_ws,
                     v_ws);
  return hipGetLastError();
}

}  // namespace nvkv

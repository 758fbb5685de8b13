// Chunked-extend attention over the shared FP8 workspace, and the chunk's FP8 append to it.
//
// SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "Three Paths" paragraph 2 and summary bullet 2: an
// extend step gathers the cached NVFP4 prefix into an FP8 workspace (nvfp4_to_fp8_ws_kernel), the
// new chunk's K/V join it there, and the chunk's queries (BF16) attend over prefix || chunk with
// FP8 K/V, causally; the chunk is then quantized into the NVFP4 cache.  Unlike decode this is
// compute-bound (the chunk's queries share every key), so the design centres on the matrix cores:
//
//  * one workgroup of four waves per (sequence, kv head, block of query tokens); its 128 score
//    columns are (query token, query head of the group) pairs, 32 per wave, so every K/V tile
//    staged in LDS serves all G query heads of the kv head;
//  * K/V tiles of 32 keys are read from HBM once per workgroup, converted from E4M3 (exactly) to
//    bf16 (K) and fp16 (V) while being written to LDS, in three buffers with one barrier per tile:
//    the PV products of a tile are issued after the next tile's QK products, so each wave has
//    independent matrix work in flight while its softmax runs;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys as rows, bf16 q as the B operand straight from
//    registers): each lane ends with 4 keys x 1 column of scores -- exactly the B operand layout of
//    O^T += V^T P^T on v_mfma_f32_16x16x32_f16, so softmax needs no data movement between the two;
//  * online softmax in the exp2 domain with lazy rescaling (the running maximum is raised only when
//    a weight would exceed 2^8); P enters PV as an fp16 hi + lo pair (two MFMAs sharing the V
//    operand), so it keeps ~22 significant bits; accumulation is fp32;
//  * the workspace scales are folded into fp32 factors: s_K into the score scale, s_V into the
//    output.
#include <hip/hip_runtime.h>

#include "nvkv_device.h"
#include "nvkv_launch.h"

namespace nvkv {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

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
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[i] = e4m3_encode(x[4 * i] / s) | (e4m3_encode(x[4 * i + 1] / s) << 8) |
           (e4m3_encode(x[4 * i + 2] / s) << 16) | (e4m3_encode(x[4 * i + 3] / s) << 24);
  }
  const size_t dst_row = (size_t)ws_offsets[b] + (size_t)prefix_lens[b] + tok;
  *reinterpret_cast<uint4*>((is_v ? v_ws : k_ws) + (dst_row * hkv * 128 + rest * 16)) =
      make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------------------------
// Extend attention
// ---------------------------------------------------------------------------------------------
constexpr int kXWaves = 4;
constexpr int kXCols = 32 * kXWaves;     // score columns per workgroup
constexpr int kXKeys = 32;               // keys per tile
constexpr int kKRow = 128 + 8;           // bf16 elements per K row in LDS (16-byte pad: conflict-free reads)
// V in LDS: [g][channel][8 keys] fp16 with keys 4 g .. 4 g + 3 then 16 + 4 g .. 16 + 4 g + 3 of the tile,
// i.e. exactly the 16-byte A operand (V^T row, k = 8 g .. 8 g + 7) lane group g reads for a channel
// (+ 8 elements of pad per group: the staging writes of one pass then fall in 32 distinct bank pairs)
constexpr int kVGroup = 128 * 8 + 8;     // fp16 elements per lane group
constexpr float kXSlack = 8.0f;          // weights may reach 2^8 before the running maximum is raised

typedef unsigned int u4x __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float xmax16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp16 of (p - hi) for a pair of values with a single rounding (mixed-precision fma)
__device__ __forceinline__ h2 lo_pair(float p0, float p1, h2 hi) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(r)
      : "v"(p0), "v"(p1), "v"(hi));
  return __builtin_bit_cast(h2, r);
}

// E4M3 pair (one 16-bit half of w) -> bf16 pair / fp16 pair, exactly (scale 1.0)
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH));
}

struct ExtendArgs {
  const uint16_t* q;            // bf16 [total_q][hq][128]
  const int32_t* q_offsets;     // [batch + 1]
  const uint8_t* k_ws;          // E4M3 [rows][hkv][128]
  const uint8_t* v_ws;
  const int32_t* ws_offsets;    // [batch (+1)]
  const int32_t* prefix_lens;   // [batch]
  float qk_scale;               // sm_scale * s_K * log2(e)
  float inv_qk_scale;           // 1 / qk_scale (raw-score threshold of the lazy rescale)
  float v_scale;                // s_V
  int hq, hkv, group, tokens_per_wg;
  float* out;                   // fp32 [total_q][hq][128]
};

__global__ __launch_bounds__(64 * kXWaves, 2) void extend_attn_kernel(ExtendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[3][kXKeys * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[3][4 * kVGroup];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.z, hk = blockIdx.y;
  const int row0 = a.q_offsets[b];
  const int chunk = a.q_offsets[b + 1] - row0;
  const int qt0 = blockIdx.x * a.tokens_per_wg;                // first query token (chunk row) of the workgroup
  if (qt0 >= chunk) return;                                     // uniform over the workgroup
  const int prefix = a.prefix_lens[b];
  const int total = prefix + chunk;                             // keys of this sequence
  const int qt_last = min(chunk, qt0 + a.tokens_per_wg) - 1;
  const int key_end = prefix + qt_last + 1;                     // keys any column of the workgroup sees
  const int n_tiles = (key_end + kXKeys - 1) / kXKeys;
  const size_t row_stride = (size_t)a.hkv * 128;                // bytes per workspace row
  const uint8_t* kbase = a.k_ws + (size_t)a.ws_offsets[b] * row_stride + (size_t)hk * 128;
  const uint8_t* vbase = a.v_ws + (size_t)a.ws_offsets[b] * row_stride + (size_t)hk * 128;
  // the sequence's rows as buffers: keys past `total` read as zeros
  const uint32_t span = (uint32_t)((size_t)(total - 1) * row_stride + 128);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kbase), 0, span, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vbase), 0, span, 0x00020000);

  // ---- this lane's two score columns (one per 16-column tile) ----
  const int g = lane >> 4, col16 = lane & 15;
  int lim[2];          // keys < lim[ct] are visible to the column (0: padding column)
  bf8v qop[2][4];      // B operands of S^T = K Q^T: Q^T[32 ks + 8 g .. + 7][column]
  size_t orow[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int c = 32 * wave + 16 * ct + col16;
    const int tk = c / a.group, hc = c - tk * a.group;
    const int qt = qt0 + tk;
    const bool ok = tk < a.tokens_per_wg && qt < chunk;
    lim[ct] = ok ? prefix + qt + 1 : 0;
    orow[ct] = ok ? ((size_t)(row0 + qt) * a.hq + (size_t)hk * a.group + hc) * 128 : 0;
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + orow[ct]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = ok ? qp[4 * ks + g] : make_uint4(0, 0, 0, 0);
      qop[ct][ks] = __builtin_bit_cast(bf8v, v);
    }
  }

  // ---- staging: thread t loads 16 K bytes (key t / 8, channels 16 (t % 8) ..) and 4 x 4 V bytes
  //      (keys 4 (t % 8) .. + 3, channels 4 (t / 8) .. + 3) of a tile ----
  const int t = threadIdx.x;
  const int sk_key = t >> 3, sk_ch = (t & 7) * 16;
  const int sv_q = t & 7, sv_ch = (t >> 3) * 4;
  uint4 kreg;
  uint32_t vreg[4];
  auto load_tile = [&](int tile) {
    const int key0 = tile * kXKeys;
    const u4x kv = __builtin_amdgcn_raw_buffer_load_b128(krs, (uint32_t)((size_t)(key0 + sk_key) * row_stride) + sk_ch, 0, 0);
    kreg = make_uint4(kv[0], kv[1], kv[2], kv[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vreg[r] = __builtin_amdgcn_raw_buffer_load_b32(vrs, (uint32_t)((size_t)(key0 + 4 * sv_q + r) * row_stride) + sv_ch, 0, 0);
  };
  auto store_tile = [&](int buf) {
    // K: 16 E4M3 -> 16 bf16 at row sk_key, columns sk_ch ..
    uint16_t* kd = &k_lds[buf][sk_key * kKRow + sk_ch];
    const uint32_t kw[4] = {kreg.x, kreg.y, kreg.z, kreg.w};
    uint32_t kb[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb[2 * i] = fp8x2_to_bf16x2<false>(kw[i]);
      kb[2 * i + 1] = fp8x2_to_bf16x2<true>(kw[i]);
    }
    *reinterpret_cast<uint4*>(kd) = make_uint4(kb[0], kb[1], kb[2], kb[3]);
    *reinterpret_cast<uint4*>(kd + 8) = make_uint4(kb[4], kb[5], kb[6], kb[7]);
    // V: keys 4 sv_q + r (r = 0..3) x channels sv_ch + c (c = 0..3) -> fp16 [quad][channel][r]
    uint32_t h[4][2];   // h[r]: fp16 pairs of key r, channels (0,1), (2,3)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r][0] = fp8x2_to_f16x2<false>(vreg[r]);
      h[r][1] = fp8x2_to_f16x2<true>(vreg[r]);
    }
    // key quad sv_q is half sv_q / 4 of lane group sv_q % 4's 8-key rows
    uint16_t* vd = &v_lds[buf][(sv_q & 3) * kVGroup + sv_ch * 8 + (sv_q >> 2) * 4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int wi = c >> 1;
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;   // high or low fp16 of each pair
      const uint32_t k01 = __builtin_amdgcn_perm(h[1][wi], h[0][wi], sel);
      const uint32_t k23 = __builtin_amdgcn_perm(h[3][wi], h[2][wi], sel);
      *reinterpret_cast<uint2*>(vd + c * 8) = make_uint2(k01, k23);
    }
  };

  // a finite floor for the running maximum: exp2(score - m_run) needs no guard for columns that
  // have seen no visible key yet (their weights are exp2(-inf) = 0, and the first real maximum
  // rescales the empty state by exp2(-1e30 - m) = 0)
  constexpr float kFloor = -1.0e30f;
  float m_run[2] = {kFloor, kFloor}, l_run[2] = {0.0f, 0.0f}, thr[2] = {-INFINITY, -INFINITY};
  f4 o[8][2];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n][0] = o[n][1] = f4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over three LDS buffers: iteration i computes S(i) = K(i) Q^T, then the PV
  // products of tile i - 1 (independent of S(i), so the matrix cores stay busy while S(i) drains),
  // then the softmax of tile i; tile i + 1 is staged meanwhile.  Buffers in use in iteration i:
  // i % 3 (QK), (i - 1) % 3 (PV) and (i + 1) % 3 (staging) -- all distinct.
  h8 phi[2], plo[2];   // B operands of PV for the previous tile: P^T hi / lo, keys 4 g + r then 16 + 4 g + r
  auto pv = [&](int vb) {
    // O^T += V^T P^T: A = V^T[16 n + lane % 16][keys 4 g + r, 16 + 4 g + r], one 16-byte read
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int ch = 16 * n + col16;
      const h8 vop = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(&v_lds[vb][g * kVGroup + ch * 8]));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, phi[ct], o[n][ct], 0, 0, 0);
        o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, plo[ct], o[n][ct], 0, 0, 0);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  int buf = 0, prev = 2;
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int next = (buf == 2) ? 0 : buf + 1;
    if (tile + 1 < n_tiles) load_tile(tile + 1);
    const int key0 = tile * kXKeys;
    // S^T = K Q^T: rows are keys 16 rt + (lane % 16) of the tile
    f4 s[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      s[rt][0] = s[rt][1] = f4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* kr = &k_lds[buf][(16 * rt + col16) * kKRow + 8 * g];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf8v kop = __builtin_bit_cast(bf8v, *reinterpret_cast<const uint4*>(kr + 32 * ks));
        s[rt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[0][ks], s[rt][0], 0, 0, 0);
        s[rt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[1][ks], s[rt][1], 0, 0, 0);
      }
    }
    if (tile > 0) pv(prev);
    // softmax of this tile; this lane's keys: key0 + 16 rt + 4 g + r
    const bool edge = key0 + kXKeys > prefix + qt0;   // some column may not see every key of the tile
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float x[8];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[4 * rt + r] = s[rt][ct][r];
      if (edge) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + 16 * rt + 4 * g + r >= lim[ct]) x[4 * rt + r] = -INFINITY;
      }
      float xm = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) xm = fmaxf(xm, x[i]);
      if (__any(xm > thr[ct])) {
        const float hmax = xmax32(xmax16(xm));
        const float m_new = fmaxf(m_run[ct], hmax * a.qk_scale);
        const float alpha = __builtin_amdgcn_exp2f(m_run[ct] - m_new);
        l_run[ct] *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) o[n][ct] *= alpha;
        m_run[ct] = m_new;
        thr[ct] = (m_new + kXSlack) * a.inv_qk_scale;
      }
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], a.qk_scale, -m_run[ct]));
      l_run[ct] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      // P = hi + lo in fp16: hi rounds toward zero, lo = fp16(P - hi) keeps ~11 more bits
      h2 hp[4], lp[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hp[k] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(p[2 * k], p[2 * k + 1]));
        lp[k] = lo_pair(p[2 * k], p[2 * k + 1], hp[k]);
      }
      phi[ct] = cat4(hp[0], hp[1], hp[2], hp[3]);
      plo[ct] = cat4(lp[0], lp[1], lp[2], lp[3]);
    }
    if (tile + 1 < n_tiles) store_tile(next);
    __syncthreads();
    prev = buf;
    buf = next;
  }
  pv(prev);   // the last tile's products (no buffer is written any more)

  // ---- normalise and write: lane holds O^T[16 n + 4 g + r][column] ----
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float l = xsum32(xsum16(l_run[ct]));
    if (lim[ct] == 0) continue;
    const float f = a.v_scale / l;
    float* dst = a.out + orow[ct];
#pragma unroll
    for (int n = 0; n < 8; ++n) *reinterpret_cast<f4*>(dst + 16 * n + 4 * g) = o[n][ct] * f;
  }
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

hipError_t launch_extend_attn(const void* q, const int32_t* q_offsets, const uint8_t* k_ws, const uint8_t* v_ws,
                              const int32_t* ws_offsets, const int32_t* prefix_lens, float k_ws_scale,
                              float v_ws_scale, float sm_scale, int batch, int hq, int hkv, int max_chunk,
                              float* out, hipStream_t stream) {
  ExtendArgs a;
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.q_offsets = q_offsets;
  a.k_ws = k_ws;
  a.v_ws = v_ws;
  a.ws_offsets = ws_offsets;
  a.prefix_lens = prefix_lens;
  a.qk_scale = sm_scale * k_ws_scale * 1.44269504088896341f;
  a.inv_qk_scale = 1.0f / a.qk_scale;
  a.v_scale = v_ws_scale;
  a.hq = hq;
  a.hkv = hkv;
  a.group = hq / hkv;
  a.tokens_per_wg = kXCols / a.group;
  a.out = out;
  dim3 grid((unsigned)((max_chunk + a.tokens_per_wg - 1) / a.tokens_per_wg), hkv, batch);
  hipLaunchKernelGGL(extend_attn_kernel, grid, dim3(64 * kXWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvkv

// Decode attention over a paged NVFP4 (or FP8 E4M3) KV cache, reading the packed cache directly.
//
// SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "Three Paths" paragraphs 3-4: decode is memory-bound,
// so the kernel reads the packed K/V and the E4M3 block scales straight from HBM and dequantizes on
// the fly instead of materialising a dequantized copy.  The Blackwell kernel described there
// stages tiles in shared memory and converts E2M1 pairs to bf16; this one is designed for gfx950:
//
//  * one wavefront owns one (sequence, kv head, split of pages); pages are consumed two at a time
//    (32 tokens = the K depth of one v_mfma_f32_16x16x32_f16);
//  * every lane issues one 16-byte load per page for K and one for V (the in-page byte layout puts
//    each lane's MFMA operand in 16 contiguous bytes), plus its scale bytes -- no LDS staging;
//  * E2M1 pairs and E4M3 scale pairs become fp16 with the gfx950 pair converts; e2m1 * scale is
//    exact in fp16 (<= 6 significant bits, range 2^-10 .. 2688), applied with packed fp16 multiplies;
//  * S^T = K_hat q^T runs on the matrix cores with tokens as rows, so each lane ends up holding the
//    scores of 4 tokens x 1 query head -- exactly the B operand it needs for O^T = V_hat^T P^T;
//  * the global scales are folded into fp32 factors: g_K into the score scale, g_V into the output;
//  * online softmax in the exp2 domain with wave butterfly reductions; P enters PV as an fp16
//    hi + lo pair so that it keeps ~22 significant bits; accumulation is fp32;
//  * splits write unnormalised partial outputs + (max, sum); a second kernel merges them.
#include <type_traits>
#include <utility>

#include "nvkv_device.h"
#include "nvkv_launch.h"

namespace nvkv {

constexpr int kWaves = 4;  // independent splits per workgroup

template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// Per-lane registers of one page of one kv head.
struct PageNv4 {
  uint4 kd;      // 32 E2M1 codes of token (lane % 16), channels 32*(lane/16) .. +31
  uint32_t ks;   // their two E4M3 block scales (low 16 bits)
  uint4 vd;      // 32 E2M1 codes: tokens 4*(lane/16) .. +3 at channels 16n + lane%16, n = 0..7
  uint4 vs0, vs1;  // E4M3 scales of tokens 4*(lane/16) .. +3, blocks 0..7 (dword n = block n)
};
struct PageFp8 {
  uint4 k0, k1;  // 32 E4M3 values of token (lane % 16), channels 32*(lane/16) .. +31
  uint4 v0, v1;  // dword n: tokens 4*(lane/16) .. +3 at channel 16n + lane % 16
};

__device__ __forceinline__ void zero_page(PageNv4& p) {
  p.kd = make_uint4(0, 0, 0, 0);
  p.ks = 0;
  p.vd = make_uint4(0, 0, 0, 0);
  p.vs0 = make_uint4(0, 0, 0, 0);
  p.vs1 = make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void zero_page(PageFp8& p) {
  p.k0 = p.k1 = p.v0 = p.v1 = make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void load_page(PageNv4& p, const DecodeArgs& a, size_t blk, int lane) {
  p.kd = *reinterpret_cast<const uint4*>(a.k_data + blk * kNvfp4DataBytes + lane * 16);
  p.ks = *reinterpret_cast<const uint16_t*>(a.k_scale + blk * kNvfp4ScaleBytes + lane * 2);
  p.vd = *reinterpret_cast<const uint4*>(a.v_data + blk * kNvfp4DataBytes + lane * 16);
  const uint4* vs = reinterpret_cast<const uint4*>(a.v_scale + blk * kNvfp4ScaleBytes + (lane >> 4) * 32);
  p.vs0 = vs[0];
  p.vs1 = vs[1];
}
__device__ __forceinline__ void load_page(PageFp8& p, const DecodeArgs& a, size_t blk, int lane) {
  const uint4* k = reinterpret_cast<const uint4*>(a.k_data + blk * kFp8Bytes + lane * 32);
  const uint4* v = reinterpret_cast<const uint4*>(a.v_data + blk * kFp8Bytes + lane * 32);
  p.k0 = k[0];
  p.k1 = k[1];
  p.v0 = v[0];
  p.v1 = v[1];
}

__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

// Zero what belongs to tokens at or past `nvalid` in a partly filled page, so that bytes never
// written (possibly NaN scale patterns) cannot reach the arithmetic.
__device__ __forceinline__ void mask_page(PageNv4& p, int nvalid, int lane) {
  if ((lane & 15) >= nvalid) p.ks = 0;                     // K: scale 0 -> exact zeros
  const int t0 = 4 * (lane >> 4);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m |= (t0 + i < nvalid ? 0xFFu : 0u) << (8 * i);
  p.vs0 = and4(p.vs0, m);                                  // V: per-token scale bytes
  p.vs1 = and4(p.vs1, m);
}
__device__ __forceinline__ void mask_page(PageFp8& p, int nvalid, int lane) {
  if ((lane & 15) >= nvalid) p.k0 = p.k1 = make_uint4(0, 0, 0, 0);
  const int t0 = 4 * (lane >> 4);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m |= (t0 + i < nvalid ? 0xFFu : 0u) << (8 * i);
  p.v0 = and4(p.v0, m);
  p.v1 = and4(p.v1, m);
}

// --- K operands: A[token][k] for k-step S covers channels 32*(lane/16) + 8S + 0..7 -------------
template <int S>
__device__ __forceinline__ h8 k_operand(const PageNv4& p, h2 sc2) {
  const uint32_t w = u4get(p.kd, S);
  const _Float16 s = (S < 2) ? sc2[0] : sc2[1];           // block 2*(lane/16) + S/2
  const h2 ss = {s, s};
  return cat4(fp4x2_to_h2<0>(w) * ss, fp4x2_to_h2<1>(w) * ss, fp4x2_to_h2<2>(w) * ss, fp4x2_to_h2<3>(w) * ss);
}
template <int S>
__device__ __forceinline__ h8 k_operand(const PageFp8& p, h2) {
  const uint32_t w0 = (S < 2) ? u4get(p.k0, 2 * S) : u4get(p.k1, 2 * S - 4);
  const uint32_t w1 = (S < 2) ? u4get(p.k0, 2 * S + 1) : u4get(p.k1, 2 * S - 3);
  return cat4(fp8x2_to_h2<false>(w0), fp8x2_to_h2<true>(w0), fp8x2_to_h2<false>(w1), fp8x2_to_h2<true>(w1));
}
__device__ __forceinline__ h2 k_scales(const PageNv4& p) { return fp8x2_to_h2<false>(p.ks); }
__device__ __forceinline__ h2 k_scales(const PageFp8&) { return h2{(_Float16)1.0f, (_Float16)1.0f}; }

// --- V operands: A[channel 16N + lane%16][k], k = tokens 4*(lane/16)+0..3 of page 0, then page 1 ---
template <int N>
__device__ __forceinline__ h8 v_operand(const PageNv4& p0, const PageNv4& p1) {
  constexpr int W = N >> 1;           // dword holding block N
  constexpr int B0 = 2 * (N & 1);     // byte of tokens (+0,+1); B0 + 1 holds tokens (+2,+3)
  const uint32_t d0 = u4get(p0.vd, W), d1 = u4get(p1.vd, W);
  const uint32_t s0 = (N < 4) ? u4get(p0.vs0, N & 3) : u4get(p0.vs1, N & 3);
  const uint32_t s1 = (N < 4) ? u4get(p1.vs0, N & 3) : u4get(p1.vs1, N & 3);
  return cat4(fp4x2_to_h2<B0>(d0) * fp8x2_to_h2<false>(s0), fp4x2_to_h2<B0 + 1>(d0) * fp8x2_to_h2<true>(s0),
              fp4x2_to_h2<B0>(d1) * fp8x2_to_h2<false>(s1), fp4x2_to_h2<B0 + 1>(d1) * fp8x2_to_h2<true>(s1));
}
template <int N>
__device__ __forceinline__ h8 v_operand(const PageFp8& p0, const PageFp8& p1) {
  const uint32_t a = (N < 4) ? u4get(p0.v0, N & 3) : u4get(p0.v1, N & 3);
  const uint32_t b = (N < 4) ? u4get(p1.v0, N & 3) : u4get(p1.v1, N & 3);
  return cat4(fp8x2_to_h2<false>(a), fp8x2_to_h2<true>(a), fp8x2_to_h2<false>(b), fp8x2_to_h2<true>(b));
}

template <typename Page>
__device__ __forceinline__ f4 qk_page(const Page& p, const h8 (&qb)[4]) {
  const h2 sc2 = k_scales(p);
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<0>(p, sc2), qb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<1>(p, sc2), qb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<2>(p, sc2), qb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<3>(p, sc2), qb[3], acc, 0, 0, 0);
  return acc;
}

// Fused quantize-append of one new token (position pos) of kv head hk into the NVFP4 pools.
// Lanes 0..31 handle K, 32..63 V; four lanes share a 16-channel block (4 channels each).
__device__ void append_token_nvfp4(const DecodeArgs& a, int b, int hk, int pos, int page, int lane) {
  const bool is_v = lane >= 32;
  const int j = (lane & 31) >> 2, qq = lane & 3;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(is_v ? a.new_v : a.new_k) +
                        ((size_t)b * a.hkv + hk) * kHeadDim + 16 * j + 4 * qq;
  const uint2 raw = *reinterpret_cast<const uint2*>(src);
  const float x[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                      __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u)};
  float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  amax = wave_max_xor(amax, 1);
  amax = wave_max_xor(amax, 2);
  float den;
  const uint32_t sc = nvfp4_block_scale(amax, is_v ? a.v_gscale : a.k_gscale, &den);
  uint32_t code[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) code[i] = nvfp4_code(x[i], den);
  const int o = pos & 15;
  const size_t blk = (size_t)page * a.hkv + hk;
  if (!is_v) {
    uint8_t* kd = const_cast<uint8_t*>(a.k_data) + blk * kNvfp4DataBytes;
    const uint32_t two = code[0] | (code[1] << 4) | (code[2] << 8) | (code[3] << 12);
    *reinterpret_cast<uint16_t*>(kd + ((j >> 1) * 16 + o) * 16 + 8 * (j & 1) + 2 * qq) = (uint16_t)two;
    if (qq == 0)
      const_cast<uint8_t*>(a.k_scale)[blk * kNvfp4ScaleBytes + ((j >> 1) * 16 + o) * 2 + (j & 1)] = (uint8_t)sc;
  } else {
    uint8_t* vd = const_cast<uint8_t*>(a.v_data) + blk * kNvfp4DataBytes;
    const int sh = 4 * (o & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the other nibble belongs to token o^1, which no other lane of this launch writes
      uint8_t* p = vd + ((o >> 2) * 16 + 4 * qq + i) * 16 + 2 * j + ((o & 3) >> 1);
      *p = (uint8_t)((*p & ~(0xFu << sh)) | (code[i] << sh));
    }
    if (qq == 0)
      const_cast<uint8_t*>(a.v_scale)[blk * kNvfp4ScaleBytes + ((o >> 2) * 8 + j) * 4 + (o & 3)] = (uint8_t)sc;
  }
}

template <typename Page>
__global__ __launch_bounds__(64 * kWaves) void decode_split_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (split >= a.num_splits) return;
  const int hk = blockIdx.y, b = blockIdx.z;
  const int group = a.hq / a.hkv;
  const int seq_len = a.seq_lens[b];
  const int n_pages = (seq_len + kPageSize - 1) / kPageSize;
  const int pg_begin = split * a.pages_per_split;
  const int pg_end = (split == a.num_splits - 1) ? n_pages : min(n_pages, pg_begin + a.pages_per_split);
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  const int jh = lane & 15, c = lane >> 4;
  const bool head_ok = jh < group;
  const int hq = hk * group + (head_ok ? jh : 0);
  const size_t row = (size_t)b * a.hq + hq;

  if constexpr (std::is_same<Page, PageNv4>::value) {
    if (a.new_k != nullptr) {
      const int pos = seq_len - 1;
      const int owner = min((pos / kPageSize) / a.pages_per_split, a.num_splits - 1);
      if (split == owner) {
        append_token_nvfp4(a, b, hk, pos, pt[pos / kPageSize], lane);
        __threadfence();   // the stores must be visible to this wave's loads of the page below
      }
    }
  }

  float* part_o = reinterpret_cast<float*>(a.workspace);
  float* part_ml = part_o + (size_t)a.batch * a.hq * a.num_splits * kHeadDim;
  if (pg_begin >= pg_end) {   // a split past the end of a short sequence (num_splits > 1 only)
    if (head_ok && c == 0) {
      float2 ml = make_float2(-INFINITY, 0.0f);
      *reinterpret_cast<float2*>(part_ml + (row * a.num_splits + split) * 2) = ml;
    }
    return;
  }

  // q row -> fp16 B operands, rescaled by a power of two so the row maximum sits in [2^13, 2^14)
  float qf[32];
  if (head_ok) {
    const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + row * kHeadDim + 32 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) bf16x8_to_f32(qp[i], qf + 8 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) qf[i] = 0.0f;
  }
  float qmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qmax = fmaxf(qmax, fabsf(qf[i]));
  qmax = wave_max_xor(qmax, 16);
  qmax = wave_max_xor(qmax, 32);
  int qexp = 0;
  if (qmax > 0.0f) {
    int ex;
    (void)frexpf(qmax, &ex);          // qmax = f * 2^ex, f in [0.5, 1)
    qexp = min(max(14 - ex, -100), 100);
  }
  h8 qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) qb[s][i] = (_Float16)__builtin_ldexpf(qf[8 * s + i], qexp);
  // scores in log2 units: <q, K_hat> * sm_scale * log2(e); K_hat = (e2m1 * s_blk) * g_K
  const float qk_scale = a.sm_scale * 1.44269504088896341f * a.k_gscale * __builtin_ldexpf(1.0f, -qexp);

  float m_run = -INFINITY, l_run = 0.0f;
  f4 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f4{0.f, 0.f, 0.f, 0.f};

  Page cur0, cur1, nxt0, nxt1;
  auto load_pair = [&](Page& p0, Page& p1, int pg, int id0, int id1) {
    load_page(p0, a, (size_t)id0 * a.hkv + hk, lane);
    if (pg + 1 < pg_end) load_page(p1, a, (size_t)id1 * a.hkv + hk, lane);
    else zero_page(p1);
  };
  int id_n0 = pt[pg_begin], id_n1 = pt[min(pg_begin + 1, pg_end - 1)];
  load_pair(cur0, cur1, pg_begin, id_n0, id_n1);
  id_n0 = pt[min(pg_begin + 2, pg_end - 1)];
  id_n1 = pt[min(pg_begin + 3, pg_end - 1)];

  for (int pg = pg_begin; pg < pg_end; pg += 2) {
    // issue the next pair's loads (and the page ids after it) before computing this pair
    const int id_f0 = pt[min(pg + 4, pg_end - 1)];
    const int id_f1 = pt[min(pg + 5, pg_end - 1)];
    if (pg + 2 < pg_end) load_pair(nxt0, nxt1, pg + 2, id_n0, id_n1);

    const int nv0 = min(kPageSize, seq_len - pg * kPageSize);
    const int nv1 = (pg + 1 < pg_end) ? min(kPageSize, seq_len - (pg + 1) * kPageSize) : 0;
    if (nv0 < kPageSize) mask_page(cur0, nv0, lane);
    if (nv1 < kPageSize && nv1 > 0) mask_page(cur1, nv1, lane);

    const f4 s0 = qk_page(cur0, qb);
    const f4 s1 = (nv1 > 0) ? qk_page(cur1, qb) : f4{0.f, 0.f, 0.f, 0.f};
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = (4 * c + r < nv0) ? s0[r] * qk_scale : -INFINITY;
      x[4 + r] = (4 * c + r < nv1) ? s1[r] * qk_scale : -INFINITY;
    }
    float mloc = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mloc = fmaxf(mloc, x[i]);
    mloc = wave_max_xor(mloc, 16);
    mloc = wave_max_xor(mloc, 32);
    const float m_new = fmaxf(m_run, mloc);
    if (__any(m_new > m_run)) {     // rescale only when some head's running max moved
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n] *= alpha;
    }
    m_run = m_new;
    float pr[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
      psum += pr[i];
    }
    l_run += psum;
    h8 ph, pl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ph[i] = (_Float16)pr[i];
      pl[i] = (_Float16)(pr[i] - (float)ph[i]);
    }
    static_for<0, 8>([&](auto nc) {
      constexpr int N = decltype(nc)::value;
      const h8 va = v_operand<N>(cur0, cur1);
      o[N] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, o[N], 0, 0, 0);
      o[N] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl, o[N], 0, 0, 0);
    });

    cur0 = nxt0;
    cur1 = nxt1;
    id_n0 = id_f0;
    id_n1 = id_f1;
  }

  l_run = wave_sum_xor(l_run, 16);
  l_run = wave_sum_xor(l_run, 32);
  if (!head_ok) return;
  // lane holds O^T[16n + 4c + r][head]
  if (a.num_splits == 1) {
    const float f = a.v_gscale / l_run;
    float* dst = a.out + row * kHeadDim + 4 * c;
#pragma unroll
    for (int n = 0; n < 8; ++n) *reinterpret_cast<f4*>(dst + 16 * n) = o[n] * f;
  } else {
    float* dst = part_o + (row * a.num_splits + split) * kHeadDim + 4 * c;
#pragma unroll
    for (int n = 0; n < 8; ++n) *reinterpret_cast<f4*>(dst + 16 * n) = o[n] * a.v_gscale;
    if (c == 0) *reinterpret_cast<float2*>(part_ml + (row * a.num_splits + split) * 2) = make_float2(m_run, l_run);
  }
}

// Log-sum-exp merge of the splits of one (sequence, query head): 128 threads, one channel each.
__global__ __launch_bounds__(128) void merge_splits_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, int num_splits,
                                                           float* __restrict__ out) {
  const size_t row = blockIdx.x;
  const float* ml = part_ml + row * num_splits * 2;
  float m = -INFINITY;
  for (int s = 0; s < num_splits; ++s)
    if (ml[2 * s + 1] > 0.0f) m = fmaxf(m, ml[2 * s]);
  float den = 0.0f, acc = 0.0f;
  for (int s = 0; s < num_splits; ++s) {
    const float l = ml[2 * s + 1];
    if (l > 0.0f) {   // empty splits carry no partial output
      const float w = __builtin_amdgcn_exp2f(ml[2 * s] - m);
      den += w * l;
      acc += w * part_o[(row * num_splits + s) * kHeadDim + threadIdx.x];
    }
  }
  out[row * kHeadDim + threadIdx.x] = acc / den;
}

size_t decode_workspace_bytes(int batch, int hq, int num_splits) {
  if (num_splits <= 1) return 0;
  return (size_t)batch * hq * num_splits * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid((a.num_splits + kWaves - 1) / kWaves, a.hkv, a.batch);
  if (a.format == kFmtNvfp4)
    hipLaunchKernelGGL(decode_split_kernel<PageNv4>, grid, dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_split_kernel<PageFp8>, grid, dim3(64 * kWaves), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  const float* part_o = reinterpret_cast<const float*>(a.workspace);
  const float* part_ml = part_o + (size_t)a.batch * a.hq * a.num_splits * kHeadDim;
  hipLaunchKernelGGL(merge_splits_kernel, dim3(a.batch * a.hq), dim3(kHeadDim), 0, stream, part_o, part_ml,
                     a.num_splits, a.out);
  return hipGetLastError();
}

}  // namespace nvkv

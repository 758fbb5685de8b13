// Decode attention over a paged NVFP4 (or FP8 E4M3) KV cache, reading the packed cache directly.
//
// SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "Three Paths" paragraphs 3-4: decode is memory-bound,
// so the kernel reads the packed K/V and the E4M3 block scales straight from HBM and dequantizes on
// the fly instead of materialising a dequantized copy.  The Blackwell kernel described there
// stages tiles in shared memory and converts E2M1 pairs to bf16; this one is designed for gfx950:
//
//  * the step's pages are cut into pieces of equal cost, one workgroup of four wavefronts each (on
//    a ragged batch every stream also costs a fixed start-up; on equal lengths the two pieces of
//    the two workgroups that share a compute unit are split 9 : 7); a wavefront owns a quarter of
//    each stream's part of its piece and consumes pages two at a time (32 tokens = the K depth of
//    one v_mfma_f32_16x16x32_f16);
//  * every lane issues one 16-byte load per page for K and one for V (the in-page byte layout puts
//    each lane's MFMA operand in 16 contiguous bytes), plus its scale bytes -- no LDS staging;
//  * E2M1 pairs and E4M3 scale pairs become fp16 with the gfx950 pair converts; e2m1 * scale is
//    exact in fp16 (<= 6 significant bits, range 2^-10 .. 2688), applied with packed fp16 multiplies;
//  * S^T = K_hat q^T runs on the matrix cores with tokens as rows, so each lane ends up holding the
//    scores of 4 tokens x 1 query head -- exactly the B operand it needs for O^T = V_hat^T P^T;
//  * the global scales are folded into fp32 factors: g_K into the score scale, g_V into the output;
//  * online softmax in the exp2 domain with wave butterfly reductions; P enters PV as an fp16
//    hi + lo pair so that it keeps ~22 significant bits; accumulation is fp32;
//  * a stream split over several pieces leaves unnormalised partial outputs + (max, sum); the last
//    of its pieces to finish merges them, so a decode is a single launch.
#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>

#include <hip/hip_ext.h>

#include "nvkv_device.h"
#include "nvkv_launch.h"

namespace nvkv {

constexpr int kWaves = 4;  // waves per workgroup, each on a quarter of a segment

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
  uint32_t vs;   // V scale bytes 2*lane, 2*lane+1: tokens 4*(lane/16) + 2*(lane%2) + {0,1}, block (lane%16)/2
};
struct PageFp8 {
  uint4 k0, k1;  // 32 E4M3 values of token (lane % 16), channels 32*(lane/16) .. +31
  uint4 v0, v1;  // dword n: tokens 4*(lane/16) .. +3 at channel 16n + lane % 16
};

__device__ __forceinline__ void zero_page(PageNv4& p) {
  p.kd = make_uint4(0, 0, 0, 0);
  p.ks = 0;
  p.vd = make_uint4(0, 0, 0, 0);
  p.vs = 0;
}
__device__ __forceinline__ void zero_page(PageFp8& p) {
  p.k0 = p.k1 = p.v0 = p.v1 = make_uint4(0, 0, 0, 0);
}

// Raw buffer loads: the page address lives in a scalar buffer resource (built with scalar adds)
// and each lane supplies only a 32-bit offset, so no vector instruction is spent on addresses.
// The resource covers exactly one (page, head) block; reads past it return zeros.
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;   // raw (untyped, unswizzled) buffer on gfx9-family GPUs

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* base, size_t blk, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + blk * bytes, 0, bytes, kBufferWord3);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  const u4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// blk is wave-uniform: (page id) * num_kv_heads + head.
__device__ __forceinline__ void load_page(PageNv4& p, const DecodeArgs& a, size_t blk, unsigned lane) {
  p.kd = ld16(block_rsrc(a.k_data, blk, kNvfp4DataBytes), lane * 16u);
  p.ks = __builtin_amdgcn_raw_buffer_load_b16(block_rsrc(a.k_scale, blk, kNvfp4ScaleBytes), lane * 2u, 0, 0);
  p.vd = ld16(block_rsrc(a.v_data, blk, kNvfp4DataBytes), lane * 16u);
  p.vs = __builtin_amdgcn_raw_buffer_load_b16(block_rsrc(a.v_scale, blk, kNvfp4ScaleBytes), lane * 2u, 0, 0);
}
__device__ __forceinline__ void load_page(PageFp8& p, const DecodeArgs& a, size_t blk, unsigned lane) {
  const __amdgpu_buffer_rsrc_t rk = block_rsrc(a.k_data, blk, kFp8Bytes);
  const __amdgpu_buffer_rsrc_t rv = block_rsrc(a.v_data, blk, kFp8Bytes);
  p.k0 = ld16(rk, lane * 32u);
  p.k1 = ld16(rk, lane * 32u + 16u);
  p.v0 = ld16(rv, lane * 32u);
  p.v1 = ld16(rv, lane * 32u + 16u);
}

__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

// Zero what belongs to tokens at or past `nvalid` in a partly filled page, so that bytes never
// written (possibly NaN scale patterns) cannot reach the arithmetic.
__device__ __forceinline__ void mask_page(PageNv4& p, int nvalid, int lane) {
  if ((lane & 15) >= nvalid) p.ks = 0;                     // K: scale 0 -> exact zeros
  const int t0 = 4 * (lane >> 4) + 2 * (lane & 1);         // V: the two tokens of this lane's scale bytes
  p.vs &= (t0 < nvalid ? 0xFFu : 0u) | (t0 + 1 < nvalid ? 0xFF00u : 0u);
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
// q0 / q1: this lane's token quad in the LDS slot of page 0 / page 1 (16 fp16 scale pairs; dword
// 2n + h = tokens +2h, +2h+1 of block n), written by v_scale_publish below.  Each block's two
// dwords are read right where they are used, which keeps few of them live.
template <int N>
__device__ __forceinline__ h8 v_operand(const PageNv4& p0, const PageNv4& p1, const uint32_t* q0,
                                        const uint32_t* q1) {
  constexpr int W = N >> 1;           // dword holding block N
  constexpr int B0 = 2 * (N & 1);     // byte of tokens (+0,+1); B0 + 1 holds tokens (+2,+3)
  const uint32_t d0 = u4get(p0.vd, W), d1 = u4get(p1.vd, W);
  const uint2 a = *reinterpret_cast<const uint2*>(q0 + 2 * N);
  const uint2 b = *reinterpret_cast<const uint2*>(q1 + 2 * N);
  return cat4(fp4x2_to_h2<B0>(d0) * __builtin_bit_cast(h2, a.x), fp4x2_to_h2<B0 + 1>(d0) * __builtin_bit_cast(h2, a.y),
              fp4x2_to_h2<B0>(d1) * __builtin_bit_cast(h2, b.x), fp4x2_to_h2<B0 + 1>(d1) * __builtin_bit_cast(h2, b.y));
}
template <int N>
__device__ __forceinline__ h8 v_operand(const PageFp8& p0, const PageFp8& p1, const uint32_t*, const uint32_t*) {
  const uint32_t a = (N < 4) ? u4get(p0.v0, N & 3) : u4get(p0.v1, N & 3);
  const uint32_t b = (N < 4) ? u4get(p1.v0, N & 3) : u4get(p1.v1, N & 3);
  return cat4(fp8x2_to_h2<false>(a), fp8x2_to_h2<true>(a), fp8x2_to_h2<false>(b), fp8x2_to_h2<true>(b));
}

// Each lane converts the E4M3 pair it loaded (tokens 4c + 2(lane%2) + {0,1} of block (lane%16)/2)
// and publishes it in this wave's LDS slot, where the 16 lanes of token quad c read the 16 pairs of
// the quad in (block, half) order.  LDS operations of one wave complete in order, so no barrier is
// needed.
__device__ __forceinline__ void v_scale_publish(const PageNv4& p, uint32_t* slot, int lane) {
  slot[lane] = __builtin_bit_cast(uint32_t, fp8x2_to_h2<false>(p.vs));
}
__device__ __forceinline__ void v_scale_publish(const PageFp8&, uint32_t*, int) {}

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

// Cross-lane partners without an LDS round trip: the gfx950 lane-swap instructions pair lane l with
// l ^ 16 (permlane16_swap) or l ^ 32 (permlane32_swap).  With both inputs equal, each lane of a pair
// receives the two values in the same order, so both compute bit-identical results.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The value lane l ^ 8 holds (same row of 16 lanes): DPP rotation of the row by 8.
__device__ __forceinline__ float from_lane_xor8(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x128, 0xF, 0xF, false));
}

// fp16 of (p - hi) for a pair of values with a single rounding (mixed-precision fma): hi + lo then
// carries about 22 significant bits of p.
__device__ __forceinline__ h2 lo_part(float p0, float p1, h2 hi) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(r)
      : "v"(p0), "v"(p1), "v"(hi));
  return __builtin_bit_cast(h2, r);
}

// Softmax weights may grow to 2^kSlack (log2 units) above the running maximum before it is raised,
// so the cross-lane maximum is needed only in the rare pairs that raise it.
constexpr float kSlack = 8.0f;

// Lane index computed where it is used: the masking of a partial page runs once per wave, and
// values derived from a loop-invariant lane index would otherwise stay in registers all loop long.
__device__ __forceinline__ int opaque_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Issue priority of a wave from the work it has left (four levels, the most left first).  Each SIMD
// runs waves of two or more workgroups, and among equal priorities the oldest wave issues first:
// the older workgroup then races ahead and the younger one finishes its pages alone, with no other
// wave to hide its memory latency (measured on the long context: 77 against 112 us for the two
// halves of the grid).  Raising the waves that have more left keeps the waves of a SIMD closer
// together: 117.1 against 118.5 us per step, side by side.
__device__ __forceinline__ void issue_priority(int left, int total) {
  const int lvl = (4 * left - 1) / total;
  if (lvl >= 3)
    __builtin_amdgcn_s_setprio(3);
  else if (lvl == 2)
    __builtin_amdgcn_s_setprio(2);
  else if (lvl == 1)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Pages of a sequence of `len` tokens (lengths are >= 1).
__device__ __forceinline__ int seq_pages(int len) { return (len + kPageSize - 1) / kPageSize; }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = min(v, __shfl_xor(v, d, 64));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v = max(v, __shfl_xor(v, d, 64));
  return __builtin_amdgcn_readfirstlane(v);
}

// ---- merge of a stream's partials, by the last of its pieces to publish ----
// Workspace of a decode with several pieces: partial outputs [slots][group][128] fp32, (max, sum)
// pairs [slots][group], slots = num_splits + B * Hkv, then one 64-bit arrival word per stream
// (generation in the high half, pieces arrived in the low half).
__device__ __forceinline__ size_t partial_slots(const DecodeArgs& a) { return (size_t)a.num_splits + (size_t)a.batch * a.hkv; }
__device__ __forceinline__ unsigned long long* arrival_words(const DecodeArgs& a) {
  const size_t bytes = partial_slots(a) * (a.hq / a.hkv) * (kHeadDim + 2) * sizeof(float);
  return reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(a.workspace) + ((bytes + 15) & ~size_t(15)));
}

// Arrival words.  A segment that holds part of a stream reads the stream's word when it starts
// and, when it ends, counts itself in: if the word it read carries another generation (an earlier
// launch's, or any value in a fresh workspace), it first tries to replace exactly that value by
// (generation, 0), then adds one.  The word keeps its old value until some workgroup's exchange
// succeeds, so the first exchange to reach it succeeds and later ones fail harmlessly; each add
// follows its own workgroup's exchange to the same word (or a read that already saw this
// generation), so every add lands on a word of this generation.  Nothing waits on another
// workgroup.
__device__ __forceinline__ unsigned long long read_arrival_word(unsigned long long* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned arrive(unsigned long long* w, unsigned long long seen, unsigned gen) {
  if ((unsigned)(seen >> 32) != gen)
    __hip_atomic_compare_exchange_strong(w, &seen, (unsigned long long)gen << 32, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
  return (unsigned)__hip_atomic_fetch_add(w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// Device-coherent (sc1) buffer stores and loads of the workspace: they are written through to, and
// read from, the level every XCD shares, so partials pass between workgroups on different XCDs
// without a cache-wide writeback or invalidation.  Offsets are bytes from the workspace base (the
// host keeps the workspace under 2^31 bytes).
constexpr int kCoherent = 16;   // cache-policy operand of the buffer builtins: sc1 (device scope)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const DecodeArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc(a.workspace, 0, 0x7FFFFFFF, kBufferWord3);
}

__device__ __forceinline__ void merge_one(float2 vc, const f4& oc, float& m, float& den, f4& acc) {
  if (vc.y > 0.0f) {   // a partial of zero weight contributes nothing
    const float m_new = fmaxf(m, vc.x);
    const float f_old = __builtin_amdgcn_exp2f(m - m_new);   // 0 while m is -inf
    const float f_new = __builtin_amdgcn_exp2f(vc.x - m_new);
    den = den * f_old + vc.y * f_new;
    acc = acc * f_old + oc * f_new;
    m = m_new;
  }
}

// Log-sum-exp merge of the n partials of stream (b, hk) (pieces first .. first + n - 1, partial
// slots first + stream ..) into the output rows of its query heads: thread t takes head t / 32,
// channels 4 (t % 32) .. + 3, sixteen partials per memory round trip.
__device__ void merge_stream(const DecodeArgs& a, int b, int hk, int first, int n) {
  constexpr int kBatch = 16;
  const int group = a.hq / a.hkv;
  const size_t slots = partial_slots(a);
  const unsigned ml_base = (unsigned)(slots * group * kHeadDim * sizeof(float));
  const unsigned slot0 = (unsigned)(first + b * a.hkv + hk);
  const __amdgpu_buffer_rsrc_t ws = ws_rsrc(a);
  for (int e = threadIdx.x; e < group * 32; e += 64 * kWaves) {
    const int j = e >> 5, d = (e & 31) * 4;
    float m = -INFINITY, den = 0.0f;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n; i0 += kBatch) {
      float2 v[kBatch];
      f4 o[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const unsigned ent = (slot0 + (unsigned)min(i0 + k, n - 1)) * (unsigned)group + (unsigned)j;   // re-reads past n
        const auto mv = __builtin_amdgcn_raw_buffer_load_b64(ws, ml_base + ent * 8u, 0, kCoherent);
        const u4v ov = __builtin_amdgcn_raw_buffer_load_b128(ws, (ent * kHeadDim + d) * 4u, 0, kCoherent);
        v[k] = make_float2(__uint_as_float(mv[0]), __uint_as_float(mv[1]));
        o[k] = f4{__uint_as_float(ov[0]), __uint_as_float(ov[1]), __uint_as_float(ov[2]), __uint_as_float(ov[3])};
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (i0 + k < n) merge_one(v[k], o[k], m, den, acc);
    }
    *reinterpret_cast<f4*>(a.out + ((size_t)b * a.hq + (size_t)hk * group + j) * kHeadDim + d) = acc * (1.0f / den);
  }
}

// The step's work is the sequence of units of the streams s = b * Hkv + h in order; stream s owns
// pages(b) + extra units, extra = kStreamCostPages when the lengths differ (else 0): virtual units
// at its start that stand for the fixed cost of starting a segment (the page-id and first page
// round trips, the combine), followed by one unit per page.  The units are cut into `pieces`
// consecutive pieces of piece_pages(...) units, an even count of at least min_pages, and
// workgroup i takes piece i: every workgroup of a grid that fits the GPU at once then has about
// the same cost, whatever the length mix (a piece that holds many short streams gets fewer pages).
__device__ __forceinline__ int piece_pages(int total_units, int pieces, int min_pages) {
  return max(min_pages, (((total_units + pieces - 1) / pieces) + 1) & ~1);
}

// Pieces of an equal-length batch come in pairs: workgroups i and i + G/2 of a grid of two per
// compute unit share a unit, and the older of the two (the first dispatched) is favoured by the
// wave arbiter, so it finishes first and the younger ends alone.  Pair k (units 2k pp .. 2k pp +
// 2 pp) is split 9 : 7 -- piece 2k, the older workgroup k's, takes pp + pp / 8 -- which keeps
// pairs aligned to stream boundaries whenever single pieces were (long contexts, 4 x 131072:
// 118.4 against 120.0 us per step, side by side).  Pieces are numbered in unit order.
struct Pieces {
  int pp;      // units per piece (the pair's mean)
  int first;   // units of the first piece of a pair (pp unless paired)
  bool paired;
  __device__ int start(int piece) const {
    return paired ? (piece >> 1) * 2 * pp + (piece & 1) * first : piece * pp;
  }
  __device__ int of(int u) const {   // the piece holding unit u
    if (!paired) return u / pp;
    const int k = u / (2 * pp);
    return 2 * k + (u - k * 2 * pp >= first ? 1 : 0);
  }
};
__device__ __forceinline__ Pieces make_pieces(int units, int pieces, int min_pages, bool equal_lengths) {
  Pieces p;
  p.pp = piece_pages(units, pieces, min_pages);
  p.paired = equal_lengths && pieces >= 2 && (pieces & 1) == 0;
  p.first = p.paired ? (p.pp + p.pp / 8) & ~1 : p.pp;
  return p;
}

// One workgroup of four waves per piece.  A piece is walked as segments (the pages of one stream
// it holds); each wave takes a contiguous, even-sized quarter of a segment and the four combine in
// LDS.  A segment holding a whole stream writes the normalised output; the others write their
// unnormalised partial output (times g_V) and (max, sum) in log2 units at partial slot
// (piece + stream) -- unique, since both grow along the unit order -- and count themselves in on
// the stream's arrival word; the last of a stream's pieces merges its partials (merge_stream).
// Partials are written before they are read and arrival words carry the launch's generation, so
// the workspace needs no initialisation.
//
// kPack (query heads per kv head <= 8): score columns 8..15 repeat heads 0..7, and those lanes feed
// the low fp16 part of P into the PV product while columns 0..7 feed the high part, so one MFMA per
// 16 channels accumulates both; the two halves of the output are added once at the end.
template <typename Page, bool kPack>
__global__ __launch_bounds__(64 * kWaves, 3) void decode_split_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = a.hq / a.hkv;

  // ---- this workgroup's piece: lanes hold the lengths of sequences base .. base + 63 ----
  int len_l = 0, incl_l = 0, total = 0, lmin = 0x7FFFFFFF, lmax = 0;
  for (int base = 0; base < a.batch; base += 64) {
    const bool ok = base + lane < a.batch;
    len_l = ok ? a.seq_lens[base + lane] : 0;
    lmin = min(lmin, wave_min(ok ? len_l : 0x7FFFFFFF));
    lmax = max(lmax, wave_max(len_l));
    incl_l = wave_incl_scan(ok ? seq_pages(len_l) : 0, lane);
    total += __builtin_amdgcn_readlane(incl_l, 63);   // readlane: a wave-uniform (scalar) value
  }
  const int extra = lmin == lmax ? 0 : kStreamCostPages;
  const int units = (total + extra * a.batch) * a.hkv;
  const Pieces pcs = make_pieces(units, (int)gridDim.x, a.pages_per_split, extra == 0);
  const int half = (int)gridDim.x / 2;
  const int piece = !pcs.paired ? (int)blockIdx.x
                                : (int)blockIdx.x < half ? 2 * (int)blockIdx.x : 2 * ((int)blockIdx.x - half) + 1;
  int u0 = pcs.start(piece);
  if (u0 >= units) return;
  const int u1 = min(units, pcs.start(piece + 1));
  // the sequence holding unit u0: the first with Hkv * (cost up to and including it) > u0
  int base = 0, before = 0;   // before: cost of the sequences before `base`
  if (a.batch > 64) {
    for (;; base += 64) {
      len_l = base + lane < a.batch ? a.seq_lens[base + lane] : 0;
      incl_l = wave_incl_scan(base + lane < a.batch ? seq_pages(len_l) : 0, lane);
      const int chunk = __builtin_amdgcn_readlane(incl_l, 63) + extra * min(64, a.batch - base);
      if ((before + chunk) * a.hkv > u0) break;
      before += chunk;
    }
  }
  const int cost_l = incl_l + extra * (lane + 1);   // cost of sequences base .. base + lane
  const unsigned long long hit = __ballot(base + lane < a.batch && (before + cost_l) * a.hkv > u0);
  const int lb = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  int b = base + lb;
  int seq_len = __builtin_amdgcn_readlane(len_l, lb);
  int n_pages = seq_pages(seq_len);
  const int seq_start = (before + __builtin_amdgcn_readlane(cost_l, lb) - n_pages - extra) * a.hkv;   // first unit of b
  int hk = (u0 - seq_start) / (n_pages + extra);
  int s_start = seq_start + hk * (n_pages + extra);                                                 // of stream (b, hk)

  __shared__ uint32_t vs_lds[kWaves][128];                  // per-wave exchange slot for V scale pairs
  __shared__ float red_o[kWaves][16][kHeadDim];             // per-wave partial outputs
  __shared__ float red_ml[kWaves][16][2];                   // per-wave (max, sum) per query head

  for (;;) {
    // the length of the sequence after b, read ahead (scalar) for the step to the next stream
    const int next_len = b + 1 < a.batch ? a.seq_lens[b + 1] : 0;
    // segment: pages [seg_begin, seg_end) of stream (b, hk), whose pages are units r0 .. r0 + n_pages
    const int r0 = s_start + extra;
    const int seg_begin = max(u0, r0) - r0, seg_end = min(u1 - r0, n_pages);
    const bool has_pages = seg_begin < seg_end;   // a piece may end inside the virtual units
    if (has_pages) {
      const bool whole = seg_begin == 0 && seg_end == n_pages;
      unsigned long long* arrival = arrival_words(a) + (size_t)b * a.hkv + hk;
      unsigned long long seen = 0;
      if (!whole && threadIdx.x == 0) seen = read_arrival_word(arrival);   // used only when the segment ends
      // lane-derived values are recomputed for every segment (the lane index is opaque to the
      // compiler), so that none of them is hoisted and kept in a register across the whole piece
      const int lane = opaque_lane_id();
      const int col = lane & 15, c = lane >> 4;
      const int jh = kPack ? (col & 7) : col;          // query head (within the group) of this lane's column
      const bool lo_lane = kPack && col >= 8;          // packed: this column carries the low part of P
      uint32_t* vs_slot = vs_lds[wave];
      const bool head_ok = jh < group;
      // each wave takes a contiguous, even-sized quarter of the segment
      const int quarter = (((seg_end - seg_begin + kWaves - 1) / kWaves) + 1) & ~1;
      const int pg_begin = min(seg_end, seg_begin + wave * quarter);
      const int pg_end = min(seg_end, pg_begin + quarter);
      const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
      const int hq = hk * group + (head_ok ? jh : 0);
      const size_t row = (size_t)b * a.hq + hq;

      if constexpr (std::is_same<Page, PageNv4>::value) {
        if (a.new_k != nullptr) {
          const int pos = seq_len - 1;
          if (pos / kPageSize >= pg_begin && pos / kPageSize < pg_end) {
            append_token_nvfp4(a, b, hk, pos, pt[pos / kPageSize], lane);
            // only this wave reads the page back; its stores reach L2 (L1 writes through, and L1 holds no
            // copy of the page: it is invalidated at kernel start), so waiting for them suffices
            __threadfence_block();
          }
        }
      }

      float m_run = -INFINITY, l_run = 0.0f;
      f4 o[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n] = f4{0.f, 0.f, 0.f, 0.f};

      if (pg_begin < pg_end) {
        // q row -> fp16 B operands, rescaled by a power of two so the row maximum sits in [2^13, 2^14).
        // The raw row is loaded with the first page ids (every lane reads a valid row: absent heads
        // read head 0 and zero it), and converted while the first pages are in flight, so the wave
        // waits for two memory round trips before its first scores, not three.
        h8 qb[4];
        float qk_scale = 0.0f;
        uint4 q_raw[4];
        auto load_q = [&] {
          const uint4* qp =
              reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + row * kHeadDim + 32 * c);
#pragma unroll
          for (int i = 0; i < 4; ++i) q_raw[i] = qp[i];
        };
        auto prep_q = [&] {
          float qf[32];
#pragma unroll
          for (int i = 0; i < 4; ++i) bf16x8_to_f32(q_raw[i], qf + 8 * i);
#pragma unroll
          for (int i = 0; i < 32; ++i) qf[i] = head_ok ? qf[i] : 0.0f;
          float qmax = 0.0f;
#pragma unroll
          for (int i = 0; i < 32; ++i) qmax = fmaxf(qmax, fabsf(qf[i]));
          qmax = max_xor16(qmax);
          qmax = max_xor32(qmax);
          int qexp = 0;
          if (qmax > 0.0f) {
            int ex;
            (void)frexpf(qmax, &ex);          // qmax = f * 2^ex, f in [0.5, 1)
            qexp = min(max(14 - ex, -100), 100);
          }
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) qb[s][i] = (_Float16)__builtin_ldexpf(qf[8 * s + i], qexp);
          // scores in log2 units: <q, K_hat> * sm_scale * log2(e); K_hat = (e2m1 * s_blk) * g_K
          qk_scale = a.sm_scale * 1.44269504088896341f * a.k_gscale * __builtin_ldexpf(1.0f, -qexp);
        };
        float thr = -INFINITY;    // raw score above which the running maximum must be raised

        // Every load below is unconditional: a pair index past the end is clamped to the last pair (a
        // re-read that hits in cache) and an odd trailing page is masked, so no branch separates a load
        // from its use and the waits on the vector-memory counter stay precise while two pairs are in flight.
        const int npairs = (pg_end - pg_begin + 1) >> 1;
        // the wave's slice of the page table as a buffer; ids are read with a scalar offset
        const __amdgpu_buffer_rsrc_t ids_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t*>(pt + pg_begin), 0, (pg_end - pg_begin) * 4, kBufferWord3);
        int vzero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));   // per-lane zero offset: keeps these on the vector path
        auto load_ids = [&](int pair, int& i0, int& i1) {
          const int rel = 2 * min(pair, npairs - 1);
          i0 = (int)__builtin_amdgcn_raw_buffer_load_b32(ids_rsrc, vzero, rel * 4, 0);
          i1 = (int)__builtin_amdgcn_raw_buffer_load_b32(ids_rsrc, vzero, min(rel + 1, pg_end - pg_begin - 1) * 4, 0);
        };
        auto issue = [&](Page& p0, Page& p1, int i0, int i1) {
          load_page(p0, a, (size_t)__builtin_amdgcn_readfirstlane(i0) * a.hkv + hk, (unsigned)lane);
          load_page(p1, a, (size_t)__builtin_amdgcn_readfirstlane(i1) * a.hkv + hk, (unsigned)lane);
        };

        // S^T = K_hat q^T for one pair of pages (two independent MFMA chains).  Only the last pair of a
        // wave's range can hold a partly filled or missing page (tail): masking runs only there.
        auto scores = [&](Page& p0, Page& p1, int pair, bool tail, float (&x)[8]) {
          const int pg = pg_begin + 2 * pair;
          int nv0 = kPageSize, nv1 = kPageSize;
          if (tail) {
            asm volatile("" ::: "memory");   // keep this a branch: the masking must not run on every pair
            nv0 = min(kPageSize, seq_len - pg * kPageSize);
            nv1 = (pg + 1 < pg_end) ? min(kPageSize, seq_len - (pg + 1) * kPageSize) : 0;
            const int ln = opaque_lane_id();
            if (nv0 < kPageSize) mask_page(p0, nv0, ln);
            if (nv1 < kPageSize) mask_page(p1, nv1, ln);   // nv1 == 0: a duplicated page, all masked
          }
          const h2 sc0 = k_scales(p0), sc1 = k_scales(p1);
          f4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<0>(p0, sc0), qb[0], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<0>(p1, sc1), qb[0], s1, 0, 0, 0);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<1>(p0, sc0), qb[1], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<1>(p1, sc1), qb[1], s1, 0, 0, 0);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<2>(p0, sc0), qb[2], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<2>(p1, sc1), qb[2], s1, 0, 0, 0);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<3>(p0, sc0), qb[3], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<3>(p1, sc1), qb[3], s1, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[r] = s0[r];
            x[4 + r] = s1[r];
          }
          if (tail) {
            asm volatile("" ::: "memory");
            const int t0 = 4 * (opaque_lane_id() >> 4);   // first token row of this lane
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (t0 + r >= nv0) x[r] = -INFINITY;
              if (t0 + r >= nv1) x[4 + r] = -INFINITY;
            }
          }
        };

        // Online softmax over one pair's raw scores, then O^T += V_hat^T P^T.
        auto accumulate = [&](const Page& p0, const Page& p1, const float (&x)[8]) {
          v_scale_publish(p0, vs_slot, lane);
          v_scale_publish(p1, vs_slot + 64, lane);
          const uint32_t* vq0 = vs_slot + 16 * c;
          const uint32_t* vq1 = vs_slot + 64 + 16 * c;
          const float xm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
          if (__any(xm > thr)) {   // some weight would exceed 2^kSlack: raise every head's running maximum
            const float hmax = max_xor32(max_xor16(xm));
            const float m_new = fmaxf(m_run, hmax * qk_scale);   // qk_scale > 0: the max commutes with it
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int n = 0; n < 8; ++n) o[n] *= alpha;
            m_run = m_new;
            thr = (m_run + kSlack) / qk_scale;
          }
          float pr[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], qk_scale, -m_run));
          l_run += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
          // P = hi + lo in fp16: hi rounds toward zero, lo = fp16(P - hi) keeps ~11 more bits
          h2 ph2[4], pl2[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            ph2[k] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pr[2 * k], pr[2 * k + 1]));
            pl2[k] = lo_part(pr[2 * k], pr[2 * k + 1], ph2[k]);
          }
          if constexpr (kPack) {
            h2 pp[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) pp[k] = lo_lane ? pl2[k] : ph2[k];
            const h8 pb = cat4(pp[0], pp[1], pp[2], pp[3]);
            static_for<0, 8>([&](auto nc) {
              constexpr int N = decltype(nc)::value;
              o[N] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand<N>(p0, p1, vq0, vq1), pb, o[N], 0, 0, 0);
            });
          } else {
            const h8 ph = cat4(ph2[0], ph2[1], ph2[2], ph2[3]);
            const h8 pl = cat4(pl2[0], pl2[1], pl2[2], pl2[3]);
            // hi product of block N issued next to the lo product of block N-1
            h8 va_prev;
            static_for<0, 8>([&](auto nc) {
              constexpr int N = decltype(nc)::value;
              const h8 va = v_operand<N>(p0, p1, vq0, vq1);
              o[N] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, o[N], 0, 0, 0);
              if constexpr (N > 0) o[N - 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va_prev, pl, o[N - 1], 0, 0, 0);
              va_prev = va;
            });
            o[7] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va_prev, pl, o[7], 0, 0, 0);
          }
        };

        // Software pipeline: the scores of pair p+1 are computed right after pair p's PV products are
        // issued, so the matrix cores and the next pair's decode overlap the softmax dependency chain.
        float x[8];
        if constexpr (std::is_same<Page, PageNv4>::value) {
          // Three register buffers in rotation: two pairs are in flight while one is computed; page ids
          // are fetched one pair ahead of the data that needs them.
          Page pa0, pa1, pb0, pb1, pc0, pc1;
          int a0, a1, b0, b1, c0, c1;
          load_ids(0, a0, a1);
          load_ids(1, b0, b1);
          load_ids(2, c0, c1);
          load_q();
          issue(pa0, pa1, a0, a1);
          issue(pb0, pb1, b0, b1);
          prep_q();
          scores(pa0, pa1, 0, npairs <= 1, x);
          for (int pr = 0;; pr += 3) {
            issue_priority(npairs - pr, npairs);
            load_ids(pr + 3, a0, a1);
            issue(pc0, pc1, c0, c1);
            accumulate(pa0, pa1, x);
            if (pr + 1 >= npairs) break;
            scores(pb0, pb1, pr + 1, pr + 2 >= npairs, x);
            load_ids(pr + 4, b0, b1);
            issue(pa0, pa1, a0, a1);
            accumulate(pb0, pb1, x);
            if (pr + 2 >= npairs) break;
            scores(pc0, pc1, pr + 2, pr + 3 >= npairs, x);
            load_ids(pr + 5, c0, c1);
            issue(pb0, pb1, b0, b1);
            accumulate(pc0, pc1, x);
            if (pr + 3 >= npairs) break;
            scores(pa0, pa1, pr + 3, pr + 4 >= npairs, x);
          }
        } else {
          // FP8 pages take twice the registers: two buffers, one pair in flight while one is computed.
          Page pa0, pa1, pb0, pb1;
          int a0, a1, b0, b1;
          load_ids(0, a0, a1);
          load_ids(1, b0, b1);
          load_q();
          issue(pa0, pa1, a0, a1);
          prep_q();
          scores(pa0, pa1, 0, npairs <= 1, x);
          for (int pr = 0;; pr += 2) {
            issue_priority(npairs - pr, npairs);
            load_ids(pr + 2, a0, a1);
            issue(pb0, pb1, b0, b1);
            accumulate(pa0, pa1, x);
            if (pr + 1 >= npairs) break;
            scores(pb0, pb1, pr + 1, pr + 2 >= npairs, x);
            load_ids(pr + 3, b0, b1);
            issue(pa0, pa1, a0, a1);
            accumulate(pb0, pb1, x);
            if (pr + 2 >= npairs) break;
            scores(pa0, pa1, pr + 2, pr + 3 >= npairs, x);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        l_run = sum_xor32(sum_xor16(l_run));
        if constexpr (kPack) {
#pragma unroll
          for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[n][r] += from_lane_xor8(o[n][r]);
        }
      }

      // ---- combine the 4 waves of this workgroup (lane holds O^T[16n + 4c + r][head jh]) ----
      if (!lo_lane) {
#pragma unroll
        for (int n = 0; n < 8; ++n) *reinterpret_cast<f4*>(&red_o[wave][jh][16 * n + 4 * c]) = o[n];
        if (c == 0) {
          red_ml[wave][jh][0] = m_run;
          red_ml[wave][jh][1] = l_run;
        }
      }
      __syncthreads();
      const int tid = (wave << 6) | opaque_lane_id();
      const int tj = tid >> 4;                    // query head (within the group) of this thread
      const int td = (tid & 15) * 8;              // first of its 8 channels
      if (tj < group) {
        float cm = -INFINITY, cl = 0.0f, co[8];
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (red_ml[w][tj][1] > 0.0f) cm = fmaxf(cm, red_ml[w][tj][0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) co[i] = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float lw = red_ml[w][tj][1];
          if (lw > 0.0f) {
            const float wt = __builtin_amdgcn_exp2f(red_ml[w][tj][0] - cm);
            cl += wt * lw;
#pragma unroll
            for (int i = 0; i < 8; ++i) co[i] += wt * red_o[w][tj][td + i];
          }
        }
        if (whole) {
          const float f = a.v_gscale / cl;
          float* dst = a.out + ((size_t)b * a.hq + hk * group + tj) * kHeadDim + td;
          *reinterpret_cast<f4*>(dst) = f4{co[0], co[1], co[2], co[3]} * f;
          *reinterpret_cast<f4*>(dst + 4) = f4{co[4], co[5], co[6], co[7]} * f;
        } else {
          const size_t slots = partial_slots(a);
          const size_t e = ((size_t)piece + (size_t)b * a.hkv + hk) * group + tj;
          float* part_o = reinterpret_cast<float*>(a.workspace);
          float* part_ml = part_o + slots * group * kHeadDim;
          // device-coherent stores: the merging workgroup may run on another XCD
          const __amdgpu_buffer_rsrc_t ws = ws_rsrc(a);
          const unsigned off = (unsigned)((e * kHeadDim + td) * sizeof(float));
          const float g = a.v_gscale;
          __builtin_amdgcn_raw_buffer_store_b128(
              u4v{__float_as_uint(co[0] * g), __float_as_uint(co[1] * g), __float_as_uint(co[2] * g), __float_as_uint(co[3] * g)},
              ws, off, 0, kCoherent);
          __builtin_amdgcn_raw_buffer_store_b128(
              u4v{__float_as_uint(co[4] * g), __float_as_uint(co[5] * g), __float_as_uint(co[6] * g), __float_as_uint(co[7] * g)},
              ws, off + 16u, 0, kCoherent);
          if (td == 0) {
            typedef unsigned int u2v __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(u2v{__float_as_uint(cm), __float_as_uint(cl)}, ws,
                                                  (unsigned)((part_ml - part_o) * sizeof(float) + e * 8), 0, kCoherent);
          }
        }
      }
      if (!whole) {
        // ---- the last piece of the stream to publish its partial merges the stream ----
        __shared__ int merge_here;
        const int r0 = s_start + extra;                        // unit of the stream's first page
        const int first = pcs.of(r0), n_pieces = pcs.of(r0 + n_pages - 1) - first + 1;
        // every thread's partial stores have completed (vmcnt 0) before the workgroup counts itself in
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) merge_here = arrive(arrival, seen, a.gen) == (unsigned)n_pieces;
        __syncthreads();
        if (merge_here) merge_stream(a, b, hk, first, n_pieces);
      }
    }

    // ---- next stream of the piece ----
    u0 = s_start + n_pages + extra;
    if (u0 >= u1) return;
    s_start = u0;
    if (++hk == a.hkv) {
      hk = 0;
      ++b;
      seq_len = next_len;
      n_pages = seq_pages(seq_len);
    }
    if (has_pages) __syncthreads();   // the combine above has read red_o / red_ml before they are written again
  }
}

// Library-held split partials and arrival words for callers that cannot allocate: one array per
// device, reached by the kernels only through the device address hipGetSymbolAddress returns (the
// array's name is a host-side stand-in in this code).  The partials are written before they are
// read and the arrival words carry each launch's generation, so the array needs no clearing; calls
// that overlap on one device share it and race.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  static std::atomic<void*> cache[kMaxScratchDevices];
  static std::mutex lock;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> g(lock);
    p = cache[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // this device is current
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      cache[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const dim3 grid((unsigned)a.num_splits);
  // the extended launch lets the dispatch packet itself record the events: no extra stream commands
  const bool pack = a.hq / a.hkv <= 8;
  const dim3 block(64 * kWaves);
  if (a.format == kFmtNvfp4) {
    if (pack)
      hipExtLaunchKernelGGL(decode_split_kernel<PageNv4, true>, grid, block, 0, stream, start, stop, 0, a);
    else
      hipExtLaunchKernelGGL(decode_split_kernel<PageNv4, false>, grid, block, 0, stream, start, stop, 0, a);
  } else {
    if (pack)
      hipExtLaunchKernelGGL(decode_split_kernel<PageFp8, true>, grid, block, 0, stream, start, stop, 0, a);
    else
      hipExtLaunchKernelGGL(decode_split_kernel<PageFp8, false>, grid, block, 0, stream, start, stop, 0, a);
  }
  return hipGetLastError();
}

}  // namespace nvkv

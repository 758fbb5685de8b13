// Chunked-extend (and prefill) attention over FP8 E4M3 K/V: the chunk's BF16 queries attend over
// prefix || chunk, causally.
//
// SGLang x Qwen x NVIDIA NVFP4 KV-cache story, "Three Paths" paragraphs 1-2 and summary bullet 2:
// initial prefill computes with BF16 Q x FP8 K/V; chunked prefill / extend gathers the cached NVFP4
// prefix into a shared FP8 workspace and attends over it.  Unlike decode this is compute-bound (the
// chunk's queries share every key), so the design centres on keeping the matrix cores busy:
//
//  * one workgroup of eight waves per (sequence, kv head, block of query tokens); its 256 or 384
//    score columns are (query token, query head of the group) pairs, 32 or 48 per wave (two or three
//    16-column tiles: three when the grid is long enough to fill the device anyway, since each K/V
//    operand read from LDS then serves 1.5x the columns), so every K/V tile
//    staged in LDS serves all G query heads of the kv head;
//  * the waves form two groups of four (one wave of each on every SIMD) that alternate between a
//    matrix phase (S = K Q^T for tile i and O += V P for tile i - 1) and a vector phase (the online
//    softmax of a tile, plus staging of the next tile).  A workgroup barrier separates the phases,
//    so while one group's MFMAs run, the other group's VALU work issues on the same SIMD;
//  * K/V tiles of 32 keys are read once per workgroup and converted exactly from E4M3 to bf16 (K,
//    staged by the first group) and fp16 (V, staged by the second) while being written to LDS,
//    three buffers deep;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys as rows, bf16 q as the B operand straight from
//    registers): each lane ends with 4 keys x 1 column of scores -- exactly the B operand layout of
//    O^T += V^T P^T on v_mfma_f32_16x16x32_f16, so the softmax needs no data movement;
//  * online softmax in the exp2 domain with lazy rescaling (the running maximum is raised only when
//    a weight would exceed 2^8); P enters PV as an fp16 hi + lo pair (two MFMAs sharing the V
//    operand), so it keeps ~22 significant bits; accumulation is fp32;
//  * the workspace scales are folded into fp32 factors: s_K into the score scale, s_V into the
//    output.
// Scores are finite or -inf (masked keys); the file is compiled without NaN semantics.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "nvkv_device.h"
#include "nvkv_launch.h"

namespace nvkv {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

constexpr int kXWaves = 8;               // two groups of four
constexpr int kXKeys = 32;               // keys per tile
constexpr int kKRow = 128 + 8;           // bf16 elements per K row in LDS (16-byte pad: conflict-free reads)
// V in LDS: [g][channel][8 keys] fp16 with keys 4 g .. 4 g + 3 then 16 + 4 g .. 16 + 4 g + 3 of the tile,
// i.e. exactly the 16-byte A operand (V^T row, k = 8 g .. 8 g + 7) lane group g reads for a channel
// (+ 8 elements of pad per group: the staging writes of one pass then fall in 32 distinct bank pairs)
constexpr int kVGroup = 128 * 8 + 8;     // fp16 elements per lane group
constexpr float kXSlack = 8.0f;          // weights may reach 2^8 before the running maximum is raised
constexpr int kRawBuffer = 0x00020000;   // buffer resource word 3: raw, unswizzled

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

// Lane index read where it is used: keeps index arithmetic that only the diagonal tiles need inside
// their branch (the compiler would otherwise hoist it and pay for it on every tile).
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Workgroup barrier that orders LDS only: prefetch loads from global memory stay in flight across
// it (a full barrier would wait for them, exposing their latency at every phase).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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
  int hq, hkv, group, tokens_per_wg, n_blocks;
  float* out;                   // fp32 [total_q][hq][128]
};

// kCT: 16-column score tiles per wave (2 or 3)
template <int kCT>
__global__ __launch_bounds__(64 * kXWaves, 2) void extend_attn_kernel(ExtendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[3][kXKeys * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[3][4 * kVGroup];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool group_a = wave < 4;          // matrix phase first; the other group is half a tile behind
  // token blocks in decreasing causal work (the last block of a chunk sees the most keys), all kv
  // heads of a block together
  const int b = blockIdx.y;
  const int hk = (int)(blockIdx.x % (unsigned)a.hkv);
  const int blk = a.n_blocks - 1 - (int)(blockIdx.x / (unsigned)a.hkv);
  const int row0 = a.q_offsets[b];
  const int chunk = a.q_offsets[b + 1] - row0;
  const int qt0 = blk * a.tokens_per_wg;                        // first query token (chunk row) of the workgroup
  if (qt0 >= chunk) return;                                     // uniform over the workgroup
  const int prefix = a.prefix_lens[b];
  const int total = prefix + chunk;                             // keys of this sequence
  const int qt_last = min(chunk, qt0 + a.tokens_per_wg) - 1;
  const int key_end = prefix + qt_last + 1;                     // keys any column of the workgroup sees
  const int n_tiles = (key_end + kXKeys - 1) / kXKeys;
  const uint32_t row_stride = (uint32_t)a.hkv * 128;            // bytes per workspace row
  const uint8_t* kbase = a.k_ws + (size_t)a.ws_offsets[b] * row_stride + (size_t)hk * 128;
  const uint8_t* vbase = a.v_ws + (size_t)a.ws_offsets[b] * row_stride + (size_t)hk * 128;
  // the sequence's rows from key `key` on, as a buffer (built with scalar arithmetic): keys past
  // `total` read as zeros, and a start at or past the end gives an empty buffer
  const uint32_t span = (uint32_t)(total - 1) * row_stride + 128;
  auto rows_from = [&](const uint8_t* base, int key) {
    const uint32_t off = (uint32_t)key * row_stride;
    // the clamped difference is selected as a vector instruction; reading it back as a scalar keeps
    // the whole resource in scalar registers (a vector resource would need a loop per load)
    const uint32_t n = __builtin_amdgcn_readfirstlane(off < span ? span - off : 0u);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + off, 0, n, kRawBuffer);
  };

  // ---- this lane's two score columns (one per 16-column tile) ----
  const int g = lane >> 4, col16 = lane & 15;
  bf8v qop[kCT][4];      // B operands of S^T = K Q^T: Q^T[32 ks + 8 g .. + 7][column]
  // Per-column facts, recomputed where they are needed (the diagonal tiles, the epilogue) rather
  // than kept in registers through the main loop: lim = keys < lim are visible to the column (0 for
  // a padding column), row = element offset of its q row (and of its output row).
  auto col_lim = [&](int ct, int l16) -> int {
    const int tk = (16 * kCT * wave + 16 * ct + l16) / a.group;
    const int qt = qt0 + tk;
    return (tk < a.tokens_per_wg && qt < chunk) ? prefix + qt + 1 : 0;
  };
  auto col_row = [&](int ct, int l16) -> size_t {
    const int c = 16 * kCT * wave + 16 * ct + l16;
    const int tk = c / a.group, hc = c - tk * a.group;
    return ((size_t)(row0 + qt0 + tk) * a.hq + (size_t)hk * a.group + hc) * 128;
  };
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    const bool ok = col_lim(ct, col16) != 0;
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + (ok ? col_row(ct, col16) : 0));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = ok ? qp[4 * ks + g] : make_uint4(0, 0, 0, 0);
      qop[ct][ks] = __builtin_bit_cast(bf8v, v);
    }
  }

  // ---- staging, 256 threads per group: the first group stages K (thread t: 16 bytes of key t / 8,
  //      channels 16 (t % 8) ..), the second V (4 x 4 bytes: keys 4 (t % 8) .. + 3, channels
  //      4 (t / 8) .. + 3) ----
  const int t = threadIdx.x & 255;
  const int sk_key = t >> 3, sk_ch = (t & 7) * 16;
  const int sv_q = t & 7, sv_ch = (t >> 3) * 4;
  const uint32_t k_off = (uint32_t)sk_key * row_stride + sk_ch;
  const uint32_t v_off = (uint32_t)(4 * sv_q) * row_stride + sv_ch;
  // staged bytes of this thread: 16 K bytes (group A) or 4 V dwords (group B)
  uint4 sreg;
  auto load_stage = [&](int tile) {
    const int key0 = tile * kXKeys;
    if (group_a) {
      const u4x kv = __builtin_amdgcn_raw_buffer_load_b128(rows_from(kbase, key0), k_off, 0, 0);
      sreg = make_uint4(kv[0], kv[1], kv[2], kv[3]);
    } else {
      // key 4 sv_q + r of the tile: the per-r row offset lives in the (scalar) buffer base
      sreg.x = __builtin_amdgcn_raw_buffer_load_b32(rows_from(vbase, key0), v_off, 0, 0);
      sreg.y = __builtin_amdgcn_raw_buffer_load_b32(rows_from(vbase, key0 + 1), v_off, 0, 0);
      sreg.z = __builtin_amdgcn_raw_buffer_load_b32(rows_from(vbase, key0 + 2), v_off, 0, 0);
      sreg.w = __builtin_amdgcn_raw_buffer_load_b32(rows_from(vbase, key0 + 3), v_off, 0, 0);
    }
  };
  auto store_k = [&](int buf) {
    // 16 E4M3 -> 16 bf16 at row sk_key, columns sk_ch ..
    uint16_t* kd = &k_lds[buf][sk_key * kKRow + sk_ch];
    const uint32_t kw[4] = {sreg.x, sreg.y, sreg.z, sreg.w};
    uint32_t kb[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb[2 * i] = fp8x2_to_bf16x2<false>(kw[i]);
      kb[2 * i + 1] = fp8x2_to_bf16x2<true>(kw[i]);
    }
    *reinterpret_cast<uint4*>(kd) = make_uint4(kb[0], kb[1], kb[2], kb[3]);
    *reinterpret_cast<uint4*>(kd + 8) = make_uint4(kb[4], kb[5], kb[6], kb[7]);
  };
  auto store_v = [&](int buf) {
    // keys 4 sv_q + r (r = 0..3) x channels sv_ch + c (c = 0..3) -> fp16 [quad][channel][r]
    const uint32_t vw[4] = {sreg.x, sreg.y, sreg.z, sreg.w};
    uint32_t h[4][2];   // h[r]: fp16 pairs of key r, channels (0,1), (2,3)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r][0] = fp8x2_to_f16x2<false>(vw[r]);
      h[r][1] = fp8x2_to_f16x2<true>(vw[r]);
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
  float m_run[kCT], l_run[kCT];
  f4 o[8][kCT];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    m_run[ct] = kFloor;
    l_run[ct] = 0.0f;
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n][ct] = f4{0.f, 0.f, 0.f, 0.f};
  }
  f4 s[2][kCT];          // scores of the tile awaiting its softmax: rows are keys 16 rt + 4 g + r
  h8 phi[kCT], plo[kCT];   // B operands of PV for the tile awaiting it: P^T hi / lo
  // A raise of the running maximum rescales O by alpha.  The vector phase only records alpha; the
  // next matrix phase applies it before its PV products, so O is only ever updated in matrix phases.
  float alpha_pend[kCT];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) alpha_pend[ct] = 1.0f;
  bool rescale_pend = false;   // wave-uniform
  auto apply_rescale = [&]() {
    if (rescale_pend) {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) o[n][ct] *= alpha_pend[ct];
      }
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) alpha_pend[ct] = 1.0f;   // a later raise of one column tile leaves the other at 1
      rescale_pend = false;
    }
  };

  // matrix phase: S(tile) = K Q^T, then O += V P for tile - 1 (kPV false for tile 0).  The compiler
  // issues the 16 operand reads two at a time, each pair just ahead of the products that use it;
  // pinning another order (all reads first, or reads interleaved with the QK products), or keeping
  // the products ahead of the phase-ending barrier, measured slower.
  auto matrix_phase = [&](int tile, auto pv_tag) {
    constexpr bool kPV = decltype(pv_tag)::value;
    if constexpr (kPV) apply_rescale();   // O is not read by the QK products: rescaling first is exact
    const int kb = tile % 3;
    bf8v kop[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const uint16_t* kr = &k_lds[kb][(16 * rt + col16) * kKRow + 8 * g];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kop[rt][ks] = __builtin_bit_cast(bf8v, *reinterpret_cast<const uint4*>(kr + 32 * ks));
    }
    h8 vop[8];
    if constexpr (kPV) {
      const int vb = (tile + 2) % 3;   // (tile - 1) % 3
      // A = V^T[16 n + lane % 16][keys 4 g + r, 16 + 4 g + r]: one 16-byte read per channel tile
#pragma unroll
      for (int n = 0; n < 8; ++n)
        vop[n] = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(&v_lds[vb][g * kVGroup + (16 * n + col16) * 8]));
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) s[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct)
          s[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[rt][ks], qop[ct][ks], s[rt][ct], 0, 0, 0);
    }
    if constexpr (kPV) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[n], phi[ct], o[n][ct], 0, 0, 0);
          o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[n], plo[ct], o[n][ct], 0, 0, 0);
        }
    }
  };
  using with_pv = std::integral_constant<bool, true>;
  using no_pv = std::integral_constant<bool, false>;
  // the last tile's PV (no buffer is written any more)
  auto last_pv = [&](int tile) {
    apply_rescale();
    const int vb = tile % 3;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const h8 vop =
          __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(&v_lds[vb][g * kVGroup + (16 * n + col16) * 8]));
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, phi[ct], o[n][ct], 0, 0, 0);
        o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, plo[ct], o[n][ct], 0, 0, 0);
      }
    }
  };
  // vector phase: online softmax of tile `tile` from s into phi / plo
  auto softmax_phase = [&](int tile) {
    const int key0 = tile * kXKeys;
    const bool edge = key0 + kXKeys > prefix + qt0;   // some column may not see every key of the tile
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      float x[8];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[4 * rt + r] = s[rt][ct][r];
      if (edge) {
        const int ln = lane_here();
        const int kr0 = key0 + 4 * (ln >> 4);             // this lane's first key row
        const int lim = col_lim(ct, ln & 15);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kr0 + 16 * rt + r >= lim) x[4 * rt + r] = -INFINITY;
      }
      float xm = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) xm = fmaxf(xm, x[i]);
      // raw score above which a weight would exceed 2^kXSlack (always met while m_run is the floor)
      const float thr = __builtin_fmaf(m_run[ct], a.inv_qk_scale, kXSlack * a.inv_qk_scale);
      if (__any(xm > thr)) {
        const float hmax = xmax32(xmax16(xm));
        const float m_new = fmaxf(m_run[ct], hmax * a.qk_scale);
        const float alpha = __builtin_amdgcn_exp2f(m_run[ct] - m_new);
        l_run[ct] *= alpha;
        alpha_pend[ct] = alpha;
        rescale_pend = true;
        m_run[ct] = m_new;
      }
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], a.qk_scale, -m_run[ct]));
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
  };

  // Schedule, tile i (each group runs its own loop; both pass two barriers per tile):
  //   phase 1:  A: S(i), PV(i-1)                              B: store V(i); load V(i+1); softmax(i-1)
  //   phase 2:  A: store K(i+1); load K(i+2); softmax(i)      B: S(i), PV(i-1)
  //   epilogue: A: PV(n-1)                                    B: softmax(n-1), PV(n-1)
  // A group's loads are issued early in its vector phase and written to LDS in its next vector
  // phase, two phases later.  LDS buffer i % 3 holds tile i: K(i+1) is written in phase 2 of tile i
  // over K(i-2), last read in phase 2 of tile i-2; V(i) is written in phase 1 of tile i over V(i-3),
  // last read in phase 2 of tile i-2.  The tiles read at the same time are K(i) and V(i-1), so every
  // write follows the last read of its buffer by at least one barrier.  The loop bodies carry no
  // conditions on the tile index: loads past the last tile read zeros (empty buffer), and the stores
  // of tile n land in buffer n % 3, which no phase reads any more.
  load_stage(0);
  if (group_a)
    store_k(0);
  else
    store_v(0);
  load_stage(1);
  // nothing is in flight when the loops start (the q loads and tile 1's loads included), so the
  // loops' only memory waits are the ones their own prefetches need
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  if (group_a) {
    auto vector_phase_a = [&](int tile) {
      store_k((tile + 1) % 3);
      // the next loads may not move above the store: their registers are the ones just stored from
      asm volatile("" ::: "memory");
      load_stage(tile + 2);
      softmax_phase(tile);
    };
    matrix_phase(0, no_pv{});
    lds_barrier();
    vector_phase_a(0);
    lds_barrier();
    for (int tile = 1; tile < n_tiles; ++tile) {
      matrix_phase(tile, with_pv{});
      lds_barrier();
      vector_phase_a(tile);
      lds_barrier();
    }
  } else {
    lds_barrier();
    matrix_phase(0, no_pv{});
    lds_barrier();
    for (int tile = 1; tile < n_tiles; ++tile) {
      store_v(tile % 3);
      asm volatile("" ::: "memory");
      load_stage(tile + 1);
      softmax_phase(tile - 1);
      lds_barrier();
      matrix_phase(tile, with_pv{});
      lds_barrier();
    }
  }
  if (!group_a) softmax_phase(n_tiles - 1);
  last_pv(n_tiles - 1);

  // ---- normalise and write: lane holds O^T[16 n + 4 g + r][column] ----
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    const float l = xsum32(xsum16(l_run[ct]));
    if (col_lim(ct, lane_here() & 15) == 0) continue;
    const float f = a.v_scale / l;
    float* dst = a.out + col_row(ct, lane_here() & 15);
#pragma unroll
    for (int n = 0; n < 8; ++n) *reinterpret_cast<f4*>(dst + 16 * n + 4 * g) = o[n][ct] * f;
  }
}

hipError_t launch_extend_attn(const void* q, const int32_t* q_offsets, const uint8_t* k_ws, const uint8_t* v_ws,
                              const int32_t* ws_offsets, const int32_t* prefix_lens, float k_ws_scale,
                              float v_ws_scale, float sm_scale, int batch, int hq, int hkv, int max_chunk,
                              int cus, float* out, hipStream_t stream) {
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
  // Three 16-column tiles per wave when that grid still gives every compute unit four workgroups or
  // more (each LDS operand read then serves 1.5x the columns: a 16384-token prefill, 62.5 against
  // 64.5 ms per 24 layers side by side); two otherwise, where fewer, wider workgroups would leave
  // units idle (a 2048-token chunk over 8 kv heads: 171 workgroups for 256 units, 24.8 against
  // 18.0 ms).
  const int tpw3 = 16 * 3 * kXWaves / a.group;
  const long long grid3 = (long long)((max_chunk + tpw3 - 1) / tpw3) * hkv * batch;
  const int ct = grid3 >= 4LL * cus ? 3 : 2;
  a.tokens_per_wg = 16 * ct * kXWaves / a.group;
  a.n_blocks = (max_chunk + a.tokens_per_wg - 1) / a.tokens_per_wg;
  a.out = out;
  dim3 grid((unsigned)a.n_blocks * hkv, batch);
  if (ct == 3)
    hipLaunchKernelGGL(extend_attn_kernel<3>, grid, dim3(64 * kXWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(extend_attn_kernel<2>, grid, dim3(64 * kXWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvkv

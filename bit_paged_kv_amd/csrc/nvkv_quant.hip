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
#pragma unroll 4
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
// NVFP4 quantize-append.  One workgroup per (window of kQWin consecutive input tokens, head).
//
// In V data two tokens share each byte (a 16-bit word holds one channel of an aligned token quad), so
// V bytes can be written with plain stores only by a writer that owns all four tokens of a quad.
// Phase 1 quantizes the window plus a halo of the next three tokens, K and V, one thread per
// (token, 16-channel block): K rows go straight to the pool, V codes and scales to LDS.  Phase 2
// writes V: a token whose slot starts an aligned quad whose four slots are taken by it and the next
// three input tokens ("leader") writes the quad's 16 channel words and its 32-bit scale word from
// LDS; tokens inside such a quad write nothing (its leader, in this window or in the previous one,
// whose halo holds them, covers them); any other token (single appends, irregular slot runs) merges
// its nibbles into their bytes with word atomics.  Input runs of any alignment thus write with plain
// stores except at run ends.
// ---------------------------------------------------------------------------------------------
#ifndef NVKV_Q_TOKENS
#define NVKV_Q_TOKENS 64
#endif
#ifndef NVKV_Q_THREADS
#define NVKV_Q_THREADS 512
#endif
constexpr int kQTok = NVKV_Q_TOKENS;      // tokens a workgroup quantizes (a power of two)
constexpr int kQWin = kQTok - 3;          // tokens it owns; the last three are the halo
constexpr int kQItems = kQTok * 16;       // (token, block, K|V) items of phase 1
constexpr int kQThreads = NVKV_Q_THREADS;
static_assert(kQWin <= 64, "the V writers of a window are listed by one wave");

// kWs: the prefill write -- every owned token's K and V also go, as E4M3 of fp32(x / s_ws) (the FP8
// encoding of the mixed-precision layers), to row t of a dense FP8 copy [n_tok][hkv][128] that the
// prefill attention reads, so the bf16 input is read once for both formats.
template <bool kWs>
__global__ __launch_bounds__(kQThreads) void nvfp4_quantize_kernel(
    const uint8_t* __restrict__ k_in, const uint8_t* __restrict__ v_in, int in_dtype, float k_in_scale,
    float v_in_scale, const int32_t* __restrict__ slots, int n_tok, int hkv, float gk, float gv,
    uint8_t* __restrict__ k_data, uint8_t* __restrict__ k_scale, uint8_t* __restrict__ v_data,
    uint8_t* __restrict__ v_scale, float sk_ws, float sv_ws, uint8_t* __restrict__ k_ws, uint8_t* __restrict__ v_ws) {
  __shared__ uint2 vcodes[kQTok][8];      // [token in window][block]: element i at bits 4 (i % 8) of word i / 8
  __shared__ uint8_t vscales[kQTok][8];
  __shared__ int32_t wslots[kQTok + 3];   // slots of input tokens w0 - 3 .. w0 + kQTok - 1 (-1: none)
  __shared__ int8_t vlist[kQWin];         // owned tokens that write V: quad leaders first, then lone tokens
  __shared__ int vcount[2];               // number of leaders, number of lone tokens
  const int h = blockIdx.y;
  const int w0 = blockIdx.x * kQWin;
  if (threadIdx.x < kQTok + 3) {
    const int t = w0 - 3 + (int)threadIdx.x;
    wslots[threadIdx.x] = (t >= 0 && t < n_tok) ? slots[t] : -1;
  }
  // phase 1: 64 tokens x 8 blocks x {K, V}; K only for owned tokens
#pragma unroll
  for (int it = 0; it < (kQItems + kQThreads - 1) / kQThreads; ++it) {
    const int item = it * kQThreads + (int)threadIdx.x;
    if (item >= kQItems) break;
    const bool is_v = item >= kQItems / 2;
    const int tr = (item >> 3) & (kQTok - 1), j = item & 7;
    const int t = w0 + tr;
    if (t >= n_tok || (!is_v && tr >= kQWin)) continue;
    float x[16];
    load_block16(is_v ? v_in : k_in, in_dtype, is_v ? v_in_scale : k_in_scale, ((size_t)t * hkv + h) * 128 + 16 * j, x);
    if constexpr (kWs) {
      if (tr < kQWin) {
        const float s = is_v ? sv_ws : sk_ws;
        const float r = 1.0f / s;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = e4m3x4_div(x + 4 * i, s, r);
        *reinterpret_cast<uint4*>((is_v ? v_ws : k_ws) + ((size_t)t * hkv + h) * 128 + 16 * j) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    uint32_t lo, hi;
    const uint32_t sc = nvfp4_quantize_block_packed(x, is_v ? gv : gk, lo, hi);
    if (is_v) {
      vcodes[tr][j] = make_uint2(lo, hi);
      vscales[tr][j] = (uint8_t)sc;
    } else {
      // from global memory: wslots is not complete before the barrier that ends this phase
      const int slot = slots[t];
      const int o = slot & 15;
      const size_t blk = (size_t)(slot >> 4) * hkv + h;
      // 8 contiguous bytes: ((j/2)*16 + o)*16 + 8*(j%2)
      *reinterpret_cast<uint2*>(k_data + blk * kNvfp4DataBytes + ((j >> 1) * 16 + o) * 16 + 8 * (j & 1)) =
          make_uint2(lo, hi);
      k_scale[blk * kNvfp4ScaleBytes + ((j >> 1) * 16 + o) * 2 + (j & 1)] = (uint8_t)sc;
    }
  }
  __syncthreads();
  // V writers of the window: an owned token is the leader of a complete quad (its slot starts an
  // aligned quad whose four slots are taken by it and the next three input tokens), inside one
  // (written by its leader, here or in the previous window, whose halo holds it), or lone.  The
  // first wave lists the leaders, then the lone tokens, so that phase 2 runs one thread per
  // (writer, block) with no idle lanes between them.
  if (threadIdx.x < 64) {
    const int tr = (int)threadIdx.x, t = w0 + tr;
    bool leader = false, lone = false;
    if (tr < kQWin && t < n_tok) {
      const int slot = wslots[tr + 3], r = slot & 3;
      // the quad is complete if input tokens t - r .. t - r + 3 hold exactly slots slot - r .. slot - r + 3
      // (wslots index of token t - r + m: tr + 3 - r + m, within 0 .. kQTok + 2)
      bool complete = t - r >= 0 && t - r + 3 < n_tok;
#pragma unroll
      for (int m = 0; m < 4; ++m) complete = complete && (m == r || wslots[tr + 3 - r + m] == slot - r + m);
      leader = complete && r == 0;
      lone = !complete;
    }
    const unsigned long long lm = __ballot(leader), am = __ballot(lone);
    const unsigned long long below = (1ull << tr) - 1ull;
    const int nl = __popcll(lm);
    if (leader) vlist[__popcll(lm & below)] = (int8_t)tr;
    if (lone) vlist[nl + __popcll(am & below)] = (int8_t)tr;
    if (tr == 0) {
      vcount[0] = nl;
      vcount[1] = __popcll(am);
    }
  }
  __syncthreads();
  // phase 2: V of the listed tokens, one thread per (writer, block)
  const int n_lead = vcount[0], n_writers = vcount[0] + vcount[1];
  for (int task = (int)threadIdx.x; task < n_writers * 8; task += kQThreads) {
    const int idx = task >> 3, j = task & 7;
    const int tr = vlist[idx];
    const int slot = wslots[tr + 3];
    const int o = slot & 15;
    const size_t blk = (size_t)(slot >> 4) * hkv + h;
    uint8_t* vd = v_data + blk * kNvfp4DataBytes;
    if (idx < n_lead) {
      // 4x16 nibble transpose: word of channel i = nibbles of tokens 0..3 at bits 0, 4, 8, 12
      const uint2 c0 = vcodes[tr][j], c1 = vcodes[tr + 1][j], c2 = vcodes[tr + 2][j], c3 = vcodes[tr + 3][j];
      uint8_t* base = vd + (o >> 2) * 256 + 2 * j;
      auto rows8 = [&](uint32_t a, uint32_t b, uint32_t c, uint32_t d, int r0) {
        // bytes of channel pairs: ab_e byte m = (a, b) nibbles of channel 2m; ab_o of channel 2m + 1
        const uint32_t ab_e = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
        const uint32_t ab_o = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
        const uint32_t cd_e = (c & 0x0F0F0F0Fu) | ((d & 0x0F0F0F0Fu) << 4);
        const uint32_t cd_o = ((c >> 4) & 0x0F0F0F0Fu) | (d & 0xF0F0F0F0u);
        // channel 2m: low byte from ab_e, high byte from cd_e
        const uint32_t e01 = __builtin_amdgcn_perm(cd_e, ab_e, 0x05010400u);   // channels 0, 2 (+2m)
        const uint32_t e23 = __builtin_amdgcn_perm(cd_e, ab_e, 0x07030602u);   // channels 4, 6
        const uint32_t o01 = __builtin_amdgcn_perm(cd_o, ab_o, 0x05010400u);   // channels 1, 3
        const uint32_t o23 = __builtin_amdgcn_perm(cd_o, ab_o, 0x07030602u);   // channels 5, 7
        const uint32_t w[8] = {e01 & 0xFFFFu, o01 & 0xFFFFu, e01 >> 16, o01 >> 16,
                               e23 & 0xFFFFu, o23 & 0xFFFFu, e23 >> 16, o23 >> 16};
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint16_t*>(base + (r0 + i) * 16) = (uint16_t)w[i];
      };
      rows8(c0.x, c1.x, c2.x, c3.x, 0);
      rows8(c0.y, c1.y, c2.y, c3.y, 8);
      const uint32_t scw = (uint32_t)vscales[tr][j] | ((uint32_t)vscales[tr + 1][j] << 8) |
                           ((uint32_t)vscales[tr + 2][j] << 16) | ((uint32_t)vscales[tr + 3][j] << 24);
      *reinterpret_cast<uint32_t*>(v_scale + blk * kNvfp4ScaleBytes + ((o >> 2) * 8 + j) * 4) = scw;
    } else {
      // channel d = 16j + i sits in byte ((o/4)*16 + i)*16 + 2j + (o%4)/2, nibble o%2; the other
      // nibble of that byte belongs to slot o^1, so update ours with two word atomics.
      const uint2 cw = vcodes[tr][j];
      const int shift_in_byte = 4 * (o & 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t code = ((i < 8 ? cw.x : cw.y) >> (4 * (i & 7))) & 0xFu;
        const size_t byte = (size_t)(((o >> 2) * 16 + i) * 16 + 2 * j + ((o & 3) >> 1));
        unsigned int* word = reinterpret_cast<unsigned int*>(vd + (byte & ~(size_t)3));
        const int shift = (int)(byte & 3) * 8 + shift_in_byte;
        atomicAnd(word, ~(0xFu << shift));
        atomicOr(word, code << shift);
      }
      v_scale[blk * kNvfp4ScaleBytes + ((o >> 2) * 8 + j) * 4 + (o & 3)] = vscales[tr][j];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// FP8 quantize-append (per-tensor scale): one thread per (group of four input tokens, head,
// 16-channel block).  For an aligned token quad the four V bytes of each channel row are adjacent
// and go out as one 32-bit store.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bool aligned_quad(const int32_t* slots, int t0, int nt) {
  if (nt != 4) return false;
  const int s0 = slots[t0];
  return (s0 & 3) == 0 && slots[t0 + 1] == s0 + 1 && slots[t0 + 2] == s0 + 2 && slots[t0 + 3] == s0 + 3;
}

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
  const float r = 1.0f / s;
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
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = e4m3x4_div(x + 4 * i, s, r);
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) b[4 * i + k2] = (w >> (8 * k2)) & 0xFFu;
    }
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
// NVFP4 prefix -> dense FP8 workspace.
// ---------------------------------------------------------------------------------------------
// Workspace byte of one E2M1 code under block scale s (an E4M3 value), global scale g and the
// workspace's FP8 scale s_ws.
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

// One wavefront per (prefix page, head) at a time, K and V: every lane loads 16 bytes of the page's K
// and of its V (the decode kernel's access pattern) and ends up with 32 consecutive channels of one
// token (token lane % 16, channels 32 (lane / 16) .. +31, i.e. two blocks), looks their codes up in
// the per-scale tables and writes 32 contiguous workspace bytes.  K arrives in that order; V (channel
// rows of token quads) is staged in a per-wave LDS slot and regathered.  grid.y = sequence.
//
// A wave's first page is requested before the tables are built, and each next page while the
// current one is transcoded, so loads, table set-up and stores overlap.
constexpr int kWsWaves = 16;   // 1024 threads: two table entries each
#ifndef NVKV_WS_WORKGROUPS
#define NVKV_WS_WORKGROUPS 256
#endif

struct WsUnit {
  uint4 kd, vd;        // this lane's 16 bytes of K and V data
  uint32_t ks;         // its two K scale bytes
  uint32_t vs_a, vs_b; // the V scale bytes of its token for its two blocks
};

// Raw buffer over one (page, head) block of `records` bytes (0: every read returns zeros without
// touching memory, which is how a wave skips a unit past the end without a branch).
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const uint8_t* base, size_t blk, int bytes, int records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + blk * bytes, 0, records, 0x00020000);
}

__device__ __forceinline__ void ws_load(WsUnit& w, const uint8_t* __restrict__ k_data,
                                        const uint8_t* __restrict__ k_scale, const uint8_t* __restrict__ v_data,
                                        const uint8_t* __restrict__ v_scale, size_t blk, bool valid, int lane) {
  const int o = lane & 15, grp = lane >> 4;
  const int nd = valid ? kNvfp4DataBytes : 0, ns = valid ? kNvfp4ScaleBytes : 0;
  if (!valid) blk = 0;
  u4v t = __builtin_amdgcn_raw_buffer_load_b128(ws_rsrc(k_data, blk, kNvfp4DataBytes, nd), lane * 16, 0, 0);
  w.kd = make_uint4(t[0], t[1], t[2], t[3]);
  w.ks = __builtin_amdgcn_raw_buffer_load_b16(ws_rsrc(k_scale, blk, kNvfp4ScaleBytes, ns), lane * 2, 0, 0);
  t = __builtin_amdgcn_raw_buffer_load_b128(ws_rsrc(v_data, blk, kNvfp4DataBytes, nd), lane * 16, 0, 0);
  w.vd = make_uint4(t[0], t[1], t[2], t[3]);
  // V scales of token o for blocks 2 grp, 2 grp + 1: bytes ((o/4)*8 + n)*4 + o%4
  const __amdgpu_buffer_rsrc_t rvs = ws_rsrc(v_scale, blk, kNvfp4ScaleBytes, ns);
  const int vso = ((o >> 2) * 8 + 2 * grp) * 4 + (o & 3);
  w.vs_a = __builtin_amdgcn_raw_buffer_load_b8(rvs, vso, 0, 0);
  w.vs_b = __builtin_amdgcn_raw_buffer_load_b8(rvs, vso + 4, 0, 0);
}

__global__ __launch_bounds__(64 * kWsWaves) void nvfp4_to_fp8_ws_kernel(
    const uint8_t* __restrict__ k_data, const uint8_t* __restrict__ k_scale, const uint8_t* __restrict__ v_data,
    const uint8_t* __restrict__ v_scale, float gk, float gv, const int32_t* __restrict__ page_table, int max_pages,
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ ws_offsets, int hkv, int max_prefix,
    float sk_ws, float sv_ws, uint8_t* __restrict__ k_ws, uint8_t* __restrict__ v_ws) {
  // The workspace byte of every E2M1 magnitude under every non-negative E4M3 block scale (128 x 8),
  // for K and V: each workgroup transcodes these 2048 cases once instead of dividing per value.
  __shared__ uint2 lut[2][128];
  // per-wave V slot: row (q, r) of the page at q * kStageQ + r (uint4 units); the pad of one uint4 per
  // token quad puts the four quads a regather instruction reads in different LDS banks
  constexpr int kStageQ = 17;
  __shared__ uint4 stage[kWsWaves][4 * kStageQ];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // page ids then load as scalars
  const int b = blockIdx.y;
  const int stride = (int)gridDim.x * kWsWaves;
  const int32_t* pt = page_table + (size_t)b * max_pages;
  // The page id of a unit is read without waiting for the prefix length: every sequence's page
  // table row has at least ceil(max_prefix / 16) entries, and a unit past the sequence's own pages
  // reads nothing (empty buffer) and writes nothing.
  const int row_pages = (max_prefix + 15) >> 4;
  auto page_id = [&](int u) { return pt[min(u / hkv, row_pages - 1)]; };
  const int u0 = (int)blockIdx.x * kWsWaves + wave;
  const int id0 = page_id(u0), id1 = page_id(u0 + stride);
  asm volatile("" ::: "memory");   // issue the page-id reads before the length read, not after its wait
  const int len = min(prefix_lens[b], max_prefix);
  const int units = ((len + 15) >> 4) * hkv;
  auto load = [&](WsUnit& w, int u, int pid) {
    ws_load(w, k_data, k_scale, v_data, v_scale, (size_t)pid * hkv + (u % hkv), u < units, lane);
  };
  // two pages in flight per wave
  WsUnit c0, c1;
  load(c0, u0, id0);
  load(c1, u0 + stride, id1);
  for (int e = threadIdx.x; e < 2048; e += blockDim.x) {
    const bool v = e >= 1024;
    reinterpret_cast<uint8_t*>(lut)[e] = (uint8_t)transcode_e2m1((uint32_t)(e & 7), e4m3_value((uint32_t)((e >> 3) & 127)),
                                                                 v ? gv : gk, v ? sv_ws : sk_ws);
  }
  __syncthreads();
  const size_t off = (size_t)ws_offsets[b];
  const size_t row_bytes = (size_t)hkv * kHeadDim;
  const int o = lane & 15, grp = lane >> 4;                // token and 32-channel group of this lane
  const int q = o >> 2, k = o & 3;
  const uint8_t* vst = reinterpret_cast<const uint8_t*>(stage[wave]);
  auto emit = [&](const WsUnit& w, int u) {
    const int p = u / hkv, h = u - p * hkv;
    const int nv = min(16, len - 16 * p);
    // K: already token-major
    const uint2 r0 = lut[0][w.ks & 0x7Fu], r1 = lut[0][(w.ks >> 8) & 0x7Fu];
    const uint2 ka = ws_bytes8(r0, w.kd.x), kb = ws_bytes8(r0, w.kd.y), kc = ws_bytes8(r1, w.kd.z),
                ke = ws_bytes8(r1, w.kd.w);
    // V: byte ((o/4)*16 + r)*16 + 4 grp + i of the page holds channel 32 grp + 16 (i/2) + r for tokens
    // 4q + 2(i%2) + {0, 1}; the 32-bit word at 4 grp therefore has token k's nibble of channel
    // 32 grp + r in bits 4k and of channel 32 grp + 16 + r in bits 16 + 4k.  acc[r / 4] collects the
    // nibbles of rows r: the first block's in bits 4 (r % 4), the second's in bits 16 + 4 (r % 4).
    stage[wave][(lane >> 4) * kStageQ + (lane & 15)] = w.vd;   // LDS operations of one wave complete in order
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(vst + (q * kStageQ + r) * 16 + 4 * grp);
      acc[r >> 2] |= ((x >> (4 * k)) & 0x000F000Fu) << (4 * (r & 3));
    }
    const uint32_t va0 = __builtin_amdgcn_perm(acc[1], acc[0], 0x05040100u);
    const uint32_t va1 = __builtin_amdgcn_perm(acc[3], acc[2], 0x05040100u);
    const uint32_t vb0 = __builtin_amdgcn_perm(acc[1], acc[0], 0x07060302u);
    const uint32_t vb1 = __builtin_amdgcn_perm(acc[3], acc[2], 0x07060302u);
    const uint2 s0 = lut[1][w.vs_a & 0x7Fu], s1 = lut[1][w.vs_b & 0x7Fu];
    const uint2 va = ws_bytes8(s0, va0), vb = ws_bytes8(s0, va1), vc = ws_bytes8(s1, vb0), ve = ws_bytes8(s1, vb1);
    if (o < nv) {
      // plain stores: the two halves of each 128-byte row meet in L2 and leave it as whole lines
      // (streaming stores of 64-byte halves raised the HBM write bytes by a third)
      const size_t row = (off + 16 * p + o) * row_bytes + (size_t)h * kHeadDim + 32 * grp;
      *reinterpret_cast<uint4*>(k_ws + row) = make_uint4(ka.x, ka.y, kb.x, kb.y);
      *reinterpret_cast<uint4*>(k_ws + row + 16) = make_uint4(kc.x, kc.y, ke.x, ke.y);
      *reinterpret_cast<uint4*>(v_ws + row) = make_uint4(va.x, va.y, vb.x, vb.y);
      *reinterpret_cast<uint4*>(v_ws + row + 16) = make_uint4(vc.x, vc.y, ve.x, ve.y);
    }
  };
  for (int u = u0; u < units; u += 2 * stride) {
    emit(c0, u);
    load(c0, u + 2 * stride, page_id(u + 2 * stride));
    if (u + stride >= units) break;
    emit(c1, u + stride);
    load(c1, u + 3 * stride, page_id(u + 3 * stride));
  }
}

// ---------------------------------------------------------------------------------------------
// launchers (validated arguments only; called from the C ABI layer)
// ---------------------------------------------------------------------------------------------
constexpr int kAmaxBlocks = 2048;   // eight 256-thread workgroups per CU: the streaming-read probe's shape

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
  dim3 grid((unsigned)(((size_t)n_tok + kQWin - 1) / kQWin), hkv);
  hipLaunchKernelGGL(nvfp4_quantize_kernel<false>, grid, dim3(kQThreads), 0, stream, (const uint8_t*)k_in,
                     (const uint8_t*)v_in, in_dtype, k_in_scale, v_in_scale, slots, n_tok, hkv, gk, gv, k_data, k_scale,
                     v_data, v_scale, 1.0f, 1.0f, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_nvfp4_prefill_write(const void* k_in, const void* v_in, int in_dtype, float k_in_scale,
                                      float v_in_scale, const int32_t* slots, int n_tok, int hkv, float gk, float gv,
                                      uint8_t* k_data, uint8_t* k_scale, uint8_t* v_data, uint8_t* v_scale, float sk_ws,
                                      float sv_ws, uint8_t* k_ws, uint8_t* v_ws, hipStream_t stream) {
  dim3 grid((unsigned)(((size_t)n_tok + kQWin - 1) / kQWin), hkv);
  hipLaunchKernelGGL(nvfp4_quantize_kernel<true>, grid, dim3(kQThreads), 0, stream, (const uint8_t*)k_in,
                     (const uint8_t*)v_in, in_dtype, k_in_scale, v_in_scale, slots, n_tok, hkv, gk, gv, k_data, k_scale,
                     v_data, v_scale, sk_ws, sv_ws, k_ws, v_ws);
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
  // one wave per (page, head) at a time; about one workgroup per CU in all, so that each wave
  // transcodes several pages (its next page loads while the current one is written) and each
  // workgroup's tables serve many
  const size_t units = (((size_t)max_prefix + 15) / 16) * hkv;
  const size_t want = (units + kWsWaves - 1) / kWsWaves;
  const size_t cap = std::max<size_t>(1, (size_t)NVKV_WS_WORKGROUPS / (size_t)batch);
  dim3 grid((unsigned)std::max<size_t>(1, std::min(want, cap)), batch);
  hipLaunchKernelGGL(nvfp4_to_fp8_ws_kernel, grid, dim3(64 * kWsWaves), 0, stream, k_data, k_scale, v_data, v_scale,
                     gk, gv, page_table, max_pages, prefix_lens, ws_offsets, hkv, max_prefix, sk_ws, sv_ws, k_ws,
                     v_ws);
  return hipGetLastError();
}

}  // namespace nvkv

// C ABI of libnvkv.so (declared in include/nvkv.h): argument validation, split planning and
// dispatch to the HIP launchers.  Nothing here allocates device memory or synchronizes.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/nvkv.h"
#include "nvkv_launch.h"

namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxDevices = 64;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A scale usable as a multiplier and divisor: finite, normal, positive.
bool good_scale(float s) { return isfinite(s) && s >= 1.17549435e-38f && s <= 1e30f; }

int shape_status(int head_dim, int page_size) {
  if (head_dim <= 0 || page_size <= 0) return NVKV_E_INVAL;
  if (head_dim != kD || page_size != kPage) return NVKV_E_UNSUPPORTED;
  return NVKV_OK;
}

int heads_status(int num_q_heads, int num_kv_heads) {
  if (num_q_heads < 1 || num_kv_heads < 1) return NVKV_E_INVAL;
  if (num_q_heads % num_kv_heads) return NVKV_E_INVAL;
  if (num_q_heads / num_kv_heads > kMaxGroup) return NVKV_E_UNSUPPORTED;
  if (num_kv_heads > 65535) return NVKV_E_UNSUPPORTED;
  return NVKV_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? NVKV_OK : NVKV_E_LAUNCH; }

// Compute units of the current device, cached per device; 256 (MI355X) when no device answers,
// which only affects split planning.
int device_cus() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Decode arguments other than the pools and the workspace.
int decode_args_status(const void* q, const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                       int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size, float sm_scale,
                       int pages_per_split, int num_splits, const float* out) {
  int st = shape_status(head_dim, page_size);
  if (st) return st;
  st = heads_status(num_q_heads, num_kv_heads);
  if (st) return st;
  if (batch < 1 || batch > 65535 || max_pages_per_seq < 1) return NVKV_E_INVAL;
  if (!q || !page_table || !seq_lens || !out) return NVKV_E_INVAL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4)) return NVKV_E_INVAL;
  if (!isfinite(sm_scale) || !(sm_scale > 0.0f)) return NVKV_E_INVAL;
  if (pages_per_split < 1 || num_splits < 1) return NVKV_E_INVAL;
  // unit counts (pages x kv heads) and piece offsets are 32-bit in the kernels
  if ((long long)batch * (max_pages_per_seq + nvkv::kStreamCostPages) * num_kv_heads + 2LL * num_splits >
          0x7FFFFFFFLL ||
      (long long)num_splits * pages_per_split > 0x7FFFFFFFLL)
    return NVKV_E_UNSUPPORTED;
  // the kernels address the workspace with 32-bit byte offsets
  if (nvkv::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, num_splits) > 0x7FFFFFFFull)
    return NVKV_E_UNSUPPORTED;
  return NVKV_OK;
}

int decode_common_status(const void* q, const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                         int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size, float sm_scale,
                         int pages_per_split, int num_splits, const float* out, const void* workspace,
                         size_t workspace_bytes) {
  int st = decode_args_status(q, page_table, max_pages_per_seq, seq_lens, batch, num_q_heads, num_kv_heads, head_dim,
                              page_size, sm_scale, pages_per_split, num_splits, out);
  if (st) return st;
  const size_t need = nvkv::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NVKV_E_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return NVKV_E_INVAL;
  return NVKV_OK;
}

// The NVFP4 pools, global scales and fused-append inputs of a decode call.
int nvfp4_pool_status(const uint8_t* k_data, const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                      float k_global_scale, float v_global_scale, const void* new_k, const void* new_v) {
  if (!k_data || !k_scale || !v_data || !v_scale) return NVKV_E_INVAL;
  if (!aligned(k_data, 16) || !aligned(k_scale, 16) || !aligned(v_data, 16) || !aligned(v_scale, 16))
    return NVKV_E_INVAL;
  if (!good_scale(k_global_scale) || !good_scale(v_global_scale)) return NVKV_E_INVAL;
  if ((new_k == nullptr) != (new_v == nullptr)) return NVKV_E_INVAL;
  if (new_k && (!aligned(new_k, 16) || !aligned(new_v, 16))) return NVKV_E_INVAL;
  return NVKV_OK;
}

}  // namespace

namespace nvkv {

// Split partials of a multi-split decode: per (query row, split) 128 unnormalised output floats,
// then per (query row, split) the (max, sum) pair -- the layout the decode kernels use.
// Partial slots: one per (piece, stream) pair along the unit order, at most pieces + streams - 1;
// then one 64-bit arrival word per stream, 16-byte aligned.
size_t decode_workspace_bytes(int batch, int hq, int hkv, int num_splits) {
  if (num_splits <= 1) return 0;
  const size_t streams = (size_t)batch * hkv;
  const size_t partials = ((size_t)num_splits + streams) * (size_t)(hq / hkv) * (kD + 2) * sizeof(float);
  return ((partials + 15) & ~size_t(15)) + streams * sizeof(unsigned long long);
}

// Generation numbers tag the arrival words of each decode launch, so a word written by any earlier
// launch reads as zero arrivals.  They start from a per-process value and skip 0.
unsigned next_decode_gen() {
  static std::atomic<unsigned> counter{static_cast<unsigned>(reinterpret_cast<uintptr_t>(&counter) >> 4) * 2654435761u};
  unsigned g;
  do {
    g = counter.fetch_add(1, std::memory_order_relaxed) + 1u;
  } while (g == 0);
  return g;
}

}  // namespace nvkv

extern "C" {

const char* nvkv_status_string(int status) {
  switch (status) {
    case NVKV_OK: return "ok";
    case NVKV_E_INVAL: return "invalid argument";
    case NVKV_E_UNSUPPORTED: return "unsupported shape (head_dim must be 128, page_size 16, GQA group 1..16)";
    case NVKV_E_LAUNCH: return "HIP launch or device query failed";
    case NVKV_E_WORKSPACE: return "workspace missing or too small";
    case NVKV_E_SCRATCH: return "split partials exceed the library-held scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

int nvkv_version(void) { return 100; }

size_t nvkv_global_scale_workspace_size(void) { return nvkv::global_scale_workspace_bytes(); }

int nvkv_global_scale(const void* x, int in_dtype, float in_scale, size_t n, float divisor, float* out_scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!x || !out_scale || n == 0) return NVKV_E_INVAL;
  if (in_dtype != NVKV_IN_BF16 && in_dtype != NVKV_IN_FP8_E4M3) return NVKV_E_INVAL;
  if (!aligned(x, 16) || !aligned(out_scale, 4)) return NVKV_E_INVAL;
  if (!good_scale(divisor)) return NVKV_E_INVAL;
  if (in_dtype == NVKV_IN_FP8_E4M3 && !good_scale(in_scale)) return NVKV_E_INVAL;
  if (!workspace || workspace_bytes < nvkv::global_scale_workspace_bytes()) return NVKV_E_WORKSPACE;
  if (!aligned(workspace, 16)) return NVKV_E_INVAL;
  return launch_status(nvkv::launch_global_scale(x, in_dtype, in_scale, n, divisor, out_scale, workspace, stream));
}

int nvfp4_kv_quantize_append(const void* k_in, const void* v_in, int in_dtype, float k_in_scale, float v_in_scale,
                             const int32_t* slots, int n_tok, int num_kv_heads, int head_dim, int page_size,
                             float k_global_scale, float v_global_scale, uint8_t* k_data, uint8_t* k_scale,
                             uint8_t* v_data, uint8_t* v_scale, hipStream_t stream) {
  int st = shape_status(head_dim, page_size);
  if (st) return st;
  if (n_tok < 0 || num_kv_heads < 1) return NVKV_E_INVAL;
  if (in_dtype != NVKV_IN_BF16 && in_dtype != NVKV_IN_FP8_E4M3) return NVKV_E_INVAL;
  if (!good_scale(k_global_scale) || !good_scale(v_global_scale)) return NVKV_E_INVAL;
  if (in_dtype == NVKV_IN_FP8_E4M3 && (!good_scale(k_in_scale) || !good_scale(v_in_scale))) return NVKV_E_INVAL;
  if (n_tok == 0) return NVKV_OK;
  if (!k_in || !v_in || !slots || !k_data || !k_scale || !v_data || !v_scale) return NVKV_E_INVAL;
  if (!aligned(k_in, 16) || !aligned(v_in, 16) || !aligned(slots, 4)) return NVKV_E_INVAL;
  if (!aligned(k_data, 16) || !aligned(k_scale, 16) || !aligned(v_data, 16) || !aligned(v_scale, 16))
    return NVKV_E_INVAL;
  if (num_kv_heads > 65535) return NVKV_E_UNSUPPORTED;      // one grid row per kv head
  return launch_status(nvkv::launch_nvfp4_quantize(k_in, v_in, in_dtype, k_in_scale, v_in_scale, slots, n_tok,
                                                   num_kv_heads, k_global_scale, v_global_scale, k_data, k_scale,
                                                   v_data, v_scale, stream));
}

int fp8_kv_quantize_append(const void* k_in, const void* v_in, const int32_t* slots, int n_tok, int num_kv_heads,
                           int head_dim, int page_size, float k_scale, float v_scale, uint8_t* k_cache,
                           uint8_t* v_cache, hipStream_t stream) {
  int st = shape_status(head_dim, page_size);
  if (st) return st;
  if (n_tok < 0 || num_kv_heads < 1) return NVKV_E_INVAL;
  if (!good_scale(k_scale) || !good_scale(v_scale)) return NVKV_E_INVAL;
  if (n_tok == 0) return NVKV_OK;
  if (!k_in || !v_in || !slots || !k_cache || !v_cache) return NVKV_E_INVAL;
  if (!aligned(k_in, 16) || !aligned(v_in, 16) || !aligned(slots, 4) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16))
    return NVKV_E_INVAL;
  return launch_status(
      nvkv::launch_fp8_quantize(k_in, v_in, slots, n_tok, num_kv_heads, k_scale, v_scale, k_cache, v_cache, stream));
}

int nvkv_plan_decode(int batch, int num_kv_heads, int max_seq_len, long long total_tokens, int force_pages_per_split,
                     int* pages_per_split, int* num_splits) {
  if (batch < 1 || num_kv_heads < 1 || max_seq_len < 1 || total_tokens < 0 || force_pages_per_split < 0 ||
      !pages_per_split || !num_splits)
    return NVKV_E_INVAL;
  const long long max_pages = ((long long)max_seq_len + kPage - 1) / kPage;
  // the step's units (pages x kv heads): from the total when given (each sequence rounds up to
  // whole pages), else every sequence as long as the longest
  long long seq_pages = (long long)batch * max_pages;
  if (total_tokens > 0) seq_pages = std::min(seq_pages, (total_tokens + (long long)batch * (kPage - 1)) / kPage);
  const long long units = std::max(1LL, seq_pages * num_kv_heads);
  long long pps, pieces;
  if (force_pages_per_split > 0) {
    // pieces of the forced size, rounded up to even (whole pairs of pages) and at most the step
    pps = std::min<long long>((force_pages_per_split + 1LL) & ~1LL, std::max(2LL, (units + 1) & ~1LL));
    pieces = (units + pps - 1) / pps;
  } else {
    // Two workgroups per compute unit, each with an equal piece of the step, all resident at once:
    // on equal lengths this is the fastest shape measured (long contexts: 16 pieces per stream,
    // 116-118 us against 119-120 us at three per unit; 32 x 4096: 34.5 against 36 us), and on a
    // ragged batch it leaves no workgroup waiting for a slot and no tail of short splits.  Small
    // steps keep pieces of at least kMinPiecePages pages.
    constexpr long long kMinPiecePages = 16;
    pps = 2;
    pieces = std::min<long long>(2 * device_cus(), (units + kMinPiecePages - 1) / kMinPiecePages);
  }
  pieces = std::max(1LL, pieces);
  if (pieces > 0x3FFFFFFFLL || pieces * pps > 0x7FFFFFFFLL) return NVKV_E_UNSUPPORTED;
  *pages_per_split = (int)pps;
  *num_splits = (int)pieces;
  return NVKV_OK;
}

size_t nvkv_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim, int num_splits) {
  if (batch < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim != kD || num_splits < 1) return 0;
  return nvkv::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, num_splits);
}

int nvfp4_paged_decode_attn(const void* q, const uint8_t* k_data, const uint8_t* k_scale, const uint8_t* v_data,
                            const uint8_t* v_scale, float k_global_scale, float v_global_scale,
                            const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                            int num_q_heads, int num_kv_heads, int head_dim, int page_size, float sm_scale,
                            int pages_per_split, int num_splits, const void* new_k, const void* new_v, float* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return nvfp4_paged_decode_attn_timed(q, k_data, k_scale, v_data, v_scale, k_global_scale, v_global_scale,
                                       page_table, max_pages_per_seq, seq_lens, batch, num_q_heads, num_kv_heads,
                                       head_dim, page_size, sm_scale, pages_per_split, num_splits, new_k, new_v, out,
                                       workspace, workspace_bytes, stream, nullptr, nullptr);
}

int nvfp4_paged_decode_attn_timed(const void* q, const uint8_t* k_data, const uint8_t* k_scale,
                                  const uint8_t* v_data, const uint8_t* v_scale, float k_global_scale,
                                  float v_global_scale, const int32_t* page_table, int max_pages_per_seq,
                                  const int32_t* seq_lens, int batch, int num_q_heads, int num_kv_heads,
                                  int head_dim, int page_size, float sm_scale, int pages_per_split, int num_splits,
                                  const void* new_k, const void* new_v, float* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream, hipEvent_t split_start,
                                  hipEvent_t split_stop) {
  int st = decode_common_status(q, page_table, max_pages_per_seq, seq_lens, batch, num_q_heads, num_kv_heads,
                                head_dim, page_size, sm_scale, pages_per_split, num_splits, out, workspace,
                                workspace_bytes);
  if (st) return st;
  st = nvfp4_pool_status(k_data, k_scale, v_data, v_scale, k_global_scale, v_global_scale, new_k, new_v);
  if (st) return st;
  nvkv::DecodeArgs a{};
  a.format = nvkv::kFmtNvfp4;
  a.q = q;
  a.k_data = k_data;
  a.k_scale = k_scale;
  a.v_data = v_data;
  a.v_scale = v_scale;
  a.k_gscale = k_global_scale;
  a.v_gscale = v_global_scale;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.sm_scale = sm_scale;
  a.pages_per_split = pages_per_split;
  a.num_splits = num_splits;
  a.gen = nvkv::next_decode_gen();
  a.new_k = new_k;
  a.new_v = new_v;
  a.out = out;
  a.workspace = workspace;
  return launch_status(nvkv::launch_decode(a, stream, split_start, split_stop));
}

int nvfp4_paged_decode_attn_noalloc(const void* q, const uint8_t* k_data, const uint8_t* k_scale,
                                    const uint8_t* v_data, const uint8_t* v_scale, float k_global_scale,
                                    float v_global_scale, const int32_t* page_table, int max_pages_per_seq,
                                    const int32_t* seq_lens, int batch, int num_q_heads, int num_kv_heads,
                                    int head_dim, int page_size, float sm_scale, int pages_per_split, int num_splits,
                                    const void* new_k, const void* new_v, float* out, hipStream_t stream) {
  // every argument is checked before the scratch array is resolved (the first device call)
  int st = decode_args_status(q, page_table, max_pages_per_seq, seq_lens, batch, num_q_heads, num_kv_heads, head_dim,
                              page_size, sm_scale, pages_per_split, num_splits, out);
  if (st) return st;
  st = nvfp4_pool_status(k_data, k_scale, v_data, v_scale, k_global_scale, v_global_scale, new_k, new_v);
  if (st) return st;
  const size_t need = nvkv::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, num_splits);
  if (need > nvkv::kDecodeScratchBytes) return NVKV_E_SCRATCH;
  void* scratch = nullptr;
  if (need > 0 && nvkv::decode_scratch(&scratch) != hipSuccess) {
    (void)hipGetLastError();
    return NVKV_E_LAUNCH;
  }
  return nvfp4_paged_decode_attn_timed(q, k_data, k_scale, v_data, v_scale, k_global_scale, v_global_scale,
                                       page_table, max_pages_per_seq, seq_lens, batch, num_q_heads, num_kv_heads,
                                       head_dim, page_size, sm_scale, pages_per_split, num_splits, new_k, new_v, out,
                                       scratch, need > 0 ? nvkv::kDecodeScratchBytes : 0, stream, nullptr, nullptr);
}

size_t nvkv_decode_noalloc_max_bytes(void) { return nvkv::kDecodeScratchBytes; }

int fp8_paged_decode_attn(const void* q, const uint8_t* k_cache, const uint8_t* v_cache, float k_scale, float v_scale,
                          const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                          int num_q_heads, int num_kv_heads, int head_dim, int page_size, float sm_scale,
                          int pages_per_split, int num_splits, float* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  int st = decode_common_status(q, page_table, max_pages_per_seq, seq_lens, batch, num_q_heads, num_kv_heads,
                                head_dim, page_size, sm_scale, pages_per_split, num_splits, out, workspace,
                                workspace_bytes);
  if (st) return st;
  if (!k_cache || !v_cache || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return NVKV_E_INVAL;
  if (!good_scale(k_scale) || !good_scale(v_scale)) return NVKV_E_INVAL;
  nvkv::DecodeArgs a{};
  a.format = nvkv::kFmtFp8;
  a.q = q;
  a.k_data = k_cache;
  a.v_data = v_cache;
  a.k_gscale = k_scale;
  a.v_gscale = v_scale;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.sm_scale = sm_scale;
  a.pages_per_split = pages_per_split;
  a.num_splits = num_splits;
  a.gen = nvkv::next_decode_gen();
  a.out = out;
  a.workspace = workspace;
  return launch_status(nvkv::launch_decode(a, stream));
}

int nvkv_decode_layers(const nvkv_layer* layers, int num_layers, const int32_t* page_table, int max_pages_per_seq,
                       const int32_t* seq_lens, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                       int page_size, float sm_scale, int pages_per_split, int num_splits, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!layers || num_layers < 1) return NVKV_E_INVAL;
  // validate every layer before launching anything, so a bad entry launches nothing
  for (int i = 0; i < num_layers; ++i) {
    const nvkv_layer& L = layers[i];
    int st = decode_common_status(L.q, page_table, max_pages_per_seq, seq_lens, batch, num_q_heads, num_kv_heads,
                                  head_dim, page_size, sm_scale, pages_per_split, num_splits, L.out, workspace,
                                  workspace_bytes);
    if (st) return st;
    if (L.precision != NVKV_PREC_NVFP4 && L.precision != NVKV_PREC_FP8) return NVKV_E_INVAL;
    if (!L.k_data || !L.v_data || !aligned(L.k_data, 16) || !aligned(L.v_data, 16)) return NVKV_E_INVAL;
    if (L.precision == NVKV_PREC_NVFP4 &&
        (!L.k_scale || !L.v_scale || !aligned(L.k_scale, 16) || !aligned(L.v_scale, 16)))
      return NVKV_E_INVAL;
    if (!good_scale(L.k_gscale) || !good_scale(L.v_gscale)) return NVKV_E_INVAL;
  }
  for (int i = 0; i < num_layers; ++i) {
    const nvkv_layer& L = layers[i];
    nvkv::DecodeArgs a{};
    a.format = L.precision == NVKV_PREC_NVFP4 ? nvkv::kFmtNvfp4 : nvkv::kFmtFp8;
    a.q = L.q;
    a.k_data = L.k_data;
    a.k_scale = L.k_scale;
    a.v_data = L.v_data;
    a.v_scale = L.v_scale;
    a.k_gscale = L.k_gscale;
    a.v_gscale = L.v_gscale;
    a.page_table = page_table;
    a.max_pages = max_pages_per_seq;
    a.seq_lens = seq_lens;
    a.batch = batch;
    a.hq = num_q_heads;
    a.hkv = num_kv_heads;
    a.sm_scale = sm_scale;
    a.pages_per_split = pages_per_split;
    a.num_splits = num_splits;
    a.gen = nvkv::next_decode_gen();
    a.out = L.out;
    a.workspace = workspace;
    int st = launch_status(nvkv::launch_decode(a, stream));
    if (st) return st;
  }
  return NVKV_OK;
}

int nvfp4_dequant_to_workspace(const uint8_t* k_data, const uint8_t* k_scale, const uint8_t* v_data,
                               const uint8_t* v_scale, float k_global_scale, float v_global_scale,
                               const int32_t* page_table, int max_pages_per_seq, const int32_t* prefix_lens,
                               const int32_t* ws_offsets, int batch, int num_kv_heads, int head_dim, int page_size,
                               int max_prefix_len, float k_ws_scale, float v_ws_scale, uint8_t* k_ws, uint8_t* v_ws,
                               hipStream_t stream) {
  int st = shape_status(head_dim, page_size);
  if (st) return st;
  if (batch < 1 || batch > 65535 || num_kv_heads < 1 || max_pages_per_seq < 1 || max_prefix_len < 0)
    return NVKV_E_INVAL;
  if (!good_scale(k_global_scale) || !good_scale(v_global_scale) || !good_scale(k_ws_scale) ||
      !good_scale(v_ws_scale))
    return NVKV_E_INVAL;
  if (!k_data || !k_scale || !v_data || !v_scale || !page_table || !prefix_lens || !ws_offsets || !k_ws || !v_ws)
    return NVKV_E_INVAL;
  if (!aligned(k_data, 16) || !aligned(k_scale, 16) || !aligned(v_data, 16) || !aligned(v_scale, 16) ||
      !aligned(k_ws, 16) || !aligned(v_ws, 16) || !aligned(page_table, 4) || !aligned(prefix_lens, 4) ||
      !aligned(ws_offsets, 4))
    return NVKV_E_INVAL;
  if ((long long)max_prefix_len > (long long)max_pages_per_seq * kPage) return NVKV_E_INVAL;
  if (max_prefix_len == 0) return NVKV_OK;
  return launch_status(nvkv::launch_dequant_to_ws(k_data, k_scale, v_data, v_scale, k_global_scale, v_global_scale,
                                                  page_table, max_pages_per_seq, prefix_lens, ws_offsets, batch,
                                                  num_kv_heads, max_prefix_len, k_ws_scale, v_ws_scale, k_ws, v_ws,
                                                  stream));
}

int nvfp4_prefill_write(const void* k_in, const void* v_in, int in_dtype, float k_in_scale, float v_in_scale,
                        const int32_t* slots, int n_tok, int num_kv_heads, int head_dim, int page_size,
                        float k_global_scale, float v_global_scale, uint8_t* k_data, uint8_t* k_scale,
                        uint8_t* v_data, uint8_t* v_scale, float k_ws_scale, float v_ws_scale, uint8_t* k_ws,
                        uint8_t* v_ws, hipStream_t stream) {
  int st = shape_status(head_dim, page_size);
  if (st) return st;
  if (n_tok < 0 || num_kv_heads < 1) return NVKV_E_INVAL;
  if (in_dtype != NVKV_IN_BF16 && in_dtype != NVKV_IN_FP8_E4M3) return NVKV_E_INVAL;
  if (!good_scale(k_global_scale) || !good_scale(v_global_scale) || !good_scale(k_ws_scale) ||
      !good_scale(v_ws_scale))
    return NVKV_E_INVAL;
  if (in_dtype == NVKV_IN_FP8_E4M3 && (!good_scale(k_in_scale) || !good_scale(v_in_scale))) return NVKV_E_INVAL;
  if (n_tok == 0) return NVKV_OK;
  if (!k_in || !v_in || !slots || !k_data || !k_scale || !v_data || !v_scale || !k_ws || !v_ws) return NVKV_E_INVAL;
  if (!aligned(k_in, 16) || !aligned(v_in, 16) || !aligned(slots, 4) || !aligned(k_ws, 16) || !aligned(v_ws, 16))
    return NVKV_E_INVAL;
  if (!aligned(k_data, 16) || !aligned(k_scale, 16) || !aligned(v_data, 16) || !aligned(v_scale, 16))
    return NVKV_E_INVAL;
  if (num_kv_heads > 65535) return NVKV_E_UNSUPPORTED;
  return launch_status(nvkv::launch_nvfp4_prefill_write(k_in, v_in, in_dtype, k_in_scale, v_in_scale, slots, n_tok,
                                                        num_kv_heads, k_global_scale, v_global_scale, k_data,
                                                        k_scale, v_data, v_scale, k_ws_scale, v_ws_scale, k_ws, v_ws,
                                                        stream));
}

static int extend_common_status(int batch, int num_kv_heads, int head_dim, int max_chunk_len, int max_prefix_len,
                                float k_ws_scale, float v_ws_scale) {
  if (head_dim <= 0) return NVKV_E_INVAL;
  if (head_dim != kD) return NVKV_E_UNSUPPORTED;
  if (batch < 1 || batch > 65535 || num_kv_heads < 1 || num_kv_heads > 65535) return NVKV_E_INVAL;
  if (max_chunk_len < 0 || max_prefix_len < 0) return NVKV_E_INVAL;
  if (!good_scale(k_ws_scale) || !good_scale(v_ws_scale)) return NVKV_E_INVAL;
  // workspace rows of one sequence are addressed with 32-bit byte offsets
  if (((long long)max_prefix_len + max_chunk_len) * num_kv_heads * kD >= (1LL << 31)) return NVKV_E_INVAL;
  return NVKV_OK;
}

int fp8_workspace_append(const void* k, const void* v, const int32_t* chunk_offsets, const int32_t* ws_offsets,
                         const int32_t* prefix_lens, int batch, int num_kv_heads, int head_dim, int max_chunk_len,
                         int max_prefix_len, float k_ws_scale, float v_ws_scale, uint8_t* k_ws, uint8_t* v_ws,
                         hipStream_t stream) {
  int st = extend_common_status(batch, num_kv_heads, head_dim, max_chunk_len, max_prefix_len, k_ws_scale, v_ws_scale);
  if (st) return st;
  if (!k || !v || !chunk_offsets || !ws_offsets || !prefix_lens || !k_ws || !v_ws) return NVKV_E_INVAL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_ws, 16) || !aligned(v_ws, 16) || !aligned(chunk_offsets, 4) ||
      !aligned(ws_offsets, 4) || !aligned(prefix_lens, 4))
    return NVKV_E_INVAL;
  if (max_chunk_len == 0) return NVKV_OK;
  return launch_status(nvkv::launch_fp8_ws_append(k, v, chunk_offsets, ws_offsets, prefix_lens, batch, num_kv_heads,
                                                  max_chunk_len, k_ws_scale, v_ws_scale, k_ws, v_ws, stream));
}

int fp8_extend_attn(const void* q, const int32_t* chunk_offsets, const uint8_t* k_ws, const uint8_t* v_ws,
                    const int32_t* ws_offsets, const int32_t* prefix_lens, float k_ws_scale, float v_ws_scale,
                    float sm_scale, int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_chunk_len,
                    int max_prefix_len, float* out, hipStream_t stream) {
  int st = extend_common_status(batch, num_kv_heads, head_dim, max_chunk_len, max_prefix_len, k_ws_scale, v_ws_scale);
  if (st) return st;
  st = heads_status(num_q_heads, num_kv_heads);
  if (st) return st;
  if (!(isfinite(sm_scale) && sm_scale > 0.0f)) return NVKV_E_INVAL;
  if (!q || !chunk_offsets || !k_ws || !v_ws || !ws_offsets || !prefix_lens || !out) return NVKV_E_INVAL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_ws, 16) || !aligned(v_ws, 16) || !aligned(chunk_offsets, 4) ||
      !aligned(ws_offsets, 4) || !aligned(prefix_lens, 4))
    return NVKV_E_INVAL;
  if (max_chunk_len == 0) return NVKV_OK;
  return launch_status(nvkv::launch_extend_attn(q, chunk_offsets, k_ws, v_ws, ws_offsets, prefix_lens, k_ws_scale,
                                                v_ws_scale, sm_scale, batch, num_q_heads, num_kv_heads,
                                                max_chunk_len, device_cus(), out, stream));
}

int nvkv_read_probe(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return NVKV_E_INVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return NVKV_E_INVAL;
  const int cus = device_cus();
  if (cus < 1) return NVKV_E_LAUNCH;
  // eight workgroups of 256 threads per compute unit: the fastest grid-stride shape measured
  return launch_status(nvkv::launch_read_probe(buf, bytes, sink, 8 * cus, stream));
}

}  // extern "C"

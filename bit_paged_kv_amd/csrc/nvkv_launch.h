// Internal launchers behind the C ABI (arguments already validated by nvkv_api.cpp).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace nvkv {

size_t global_scale_workspace_bytes();
hipError_t launch_global_scale(const void* x, int in_dtype, float in_scale, size_t n, float divisor, float* out,
                               void* workspace, hipStream_t stream);
hipError_t launch_nvfp4_quantize(const void* k_in, const void* v_in, int in_dtype, float k_in_scale, float v_in_scale,
                                 const int32_t* slots, int n_tok, int hkv, float gk, float gv, uint8_t* k_data,
                                 uint8_t* k_scale, uint8_t* v_data, uint8_t* v_scale, hipStream_t stream);
hipError_t launch_nvfp4_prefill_write(const void* k_in, const void* v_in, int in_dtype, float k_in_scale,
                                      float v_in_scale, const int32_t* slots, int n_tok, int hkv, float gk, float gv,
                                      uint8_t* k_data, uint8_t* k_scale, uint8_t* v_data, uint8_t* v_scale, float sk_ws,
                                      float sv_ws, uint8_t* k_ws, uint8_t* v_ws, hipStream_t stream);
hipError_t launch_fp8_quantize(const void* k_in, const void* v_in, const int32_t* slots, int n_tok, int hkv, float sk,
                               float sv, uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream);
hipError_t launch_dequant_to_ws(const uint8_t* k_data, const uint8_t* k_scale, const uint8_t* v_data,
                                const uint8_t* v_scale, float gk, float gv, const int32_t* page_table, int max_pages,
                                const int32_t* prefix_lens, const int32_t* ws_offsets, int batch, int hkv,
                                int max_prefix, float sk_ws, float sv_ws, uint8_t* k_ws, uint8_t* v_ws,
                                hipStream_t stream);

hipError_t launch_fp8_ws_append(const void* k, const void* v, const int32_t* chunk_offsets, const int32_t* ws_offsets,
                                const int32_t* prefix_lens, int batch, int hkv, int max_chunk, float sk, float sv,
                                uint8_t* k_ws, uint8_t* v_ws, hipStream_t stream);
hipError_t launch_extend_attn(const void* q, const int32_t* chunk_offsets, const uint8_t* k_ws, const uint8_t* v_ws,
                              const int32_t* ws_offsets, const int32_t* prefix_lens, float k_ws_scale,
                              float v_ws_scale, float sm_scale, int batch, int hq, int hkv, int max_chunk,
                              int cus, float* out, hipStream_t stream);

// Decode: the step's pages are cut into num_splits pieces of equal cost, one workgroup of four
// wavefronts each; a stream split over several pieces leaves partial softmax states that the last
// of its pieces to finish merges.
enum CacheFormat { kFmtNvfp4 = 0, kFmtFp8 = 1 };

struct DecodeArgs {
  int format;                 // CacheFormat
  const void* q;              // bf16 [B][Hq][128]
  const uint8_t* k_data;
  const uint8_t* k_scale;     // NVFP4 only
  const uint8_t* v_data;
  const uint8_t* v_scale;     // NVFP4 only
  float k_gscale, v_gscale;   // NVFP4 global scales, or FP8 per-tensor scales
  const int32_t* page_table;
  int max_pages;
  const int32_t* seq_lens;
  int batch, hq, hkv;
  float sm_scale;
  int pages_per_split, num_splits;   // minimum piece size (pages), pieces = workgroups
  const void* new_k;          // NVFP4 fused append, or null
  const void* new_v;
  float* out;                 // fp32 [B][Hq][128]
  void* workspace;            // partials and arrival words when num_splits > 1
  unsigned gen;               // this launch's generation number (nonzero, distinct per launch)
};

size_t decode_workspace_bytes(int batch, int hq, int hkv, int num_splits);
// A fresh generation number for one decode launch (never 0).
unsigned next_decode_gen();

// Cost, in pages, that the decode partition charges for each stream of a batch whose lengths
// differ: the start-up of a segment (two memory round trips and the combine) against the time a
// workgroup takes per page.  Swept on a 64-sequence ragged batch: 16 pages 134.2-134.7 us per
// step, 32 126.3-126.7, 48 124.7-125.2, 64 125.1-125.9.
constexpr int kStreamCostPages = 48;

// Split partials held by the library for the no-allocation decode entry point: a 32 MiB array per
// device, room for 64,527 partial rows of 130 floats (e.g. 7553 pieces + 512 streams of 8 query
// heads); its device address is resolved once per device.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
constexpr int kMaxScratchDevices = 64;
// Device address of the current device's array (hipGetSymbolAddress, cached per device).
hipError_t decode_scratch(void** ptr);
// start / stop (may be null) are recorded by the split kernel's own dispatch.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);

// Streaming-read probe over `bytes` (a multiple of 16) with `workgroups` workgroups of 256 threads.
hipError_t launch_read_probe(const void* buf, size_t bytes, unsigned* sink, int workgroups, hipStream_t stream);

}  // namespace nvkv

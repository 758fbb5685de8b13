/*
 * nvkv.h -- C ABI of libnvkv.so: NVFP4 / FP8 paged KV cache for decode attention on MI355X (gfx950).
 *
 * The operations follow the NVFP4 KV-cache design described in
 *   [S] "SGLang x Qwen x NVIDIA Collaboration: NVFP4 KV Cache Breaks Long-Context and Agentic
 *       Inference Bottlenecks" (ai.synthepulse.app story), sections "The Ledger of 4-bit KV Cache",
 *       "The Core of the Ledger: 4-bit Does Not Equal 2x" and "Three Paths", and
 *   [O] "SOAR Weekly Champion Notes 05: NVFP4 KV Cache and Mixed-Precision Practice" (openbmb.cn),
 *       sections "02 NVFP4 KV Cache" and "03 Mixed-precision KV Cache".
 *
 * FORMAT ([S] "The Core of the Ledger" paragraphs 1-2, [O] "02 NVFP4 KV Cache").  Every value is a
 * 4-bit E2M1 code (sign, 2 exponent bits, 1 mantissa bit: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6),
 * two codes per byte; each block of 16 consecutive channels of one (token, head) has one OCP E4M3
 * scale byte; each tensor (one layer's K, or its V) has one fp32 global scale g.  A value reads
 * back as e2m1 * e4m3_scale * g.  16 values take 9 bytes, 56.25% of FP8.
 *   Quantization (bit-exact contract):  a = max|x| over the block;  s = E4M3_rne_sat(a / fp32(6 g));
 *   code = E2M1_rne_sat(x / fp32(s g)) with the sign of x (signed zeros kept); s == 0 gives signed zeros.
 *   All arithmetic is fp32 with correctly rounded division.  Input x is bf16, or FP8 E4M3 times a
 *   per-tensor fp32 scale (then x = fp32(e4m3 * in_scale)).
 *
 * PAGED POOLS.  Page size 16 tokens, head_dim 128 (the only supported shape).  A token of sequence b
 * at position t lives in page page_table[b * max_pages_per_seq + t / 16] at offset o = t % 16
 * ("slot" = page * 16 + o).  Every pool is [num_pages][num_kv_heads][block]; inside a block
 * (d = channel, j = d / 16) the bytes are laid out for the decode kernel's 16-byte lane loads:
 *   NVFP4 K data  1024 B: byte ((d/32)*16 + o)*16 + (d%32)/2,  nibble d%2 (0 = low)
 *   NVFP4 K scale  128 B: byte ((j/2)*16 + o)*2 + j%2
 *   NVFP4 V data  1024 B: byte ((o/4)*16 + d%16)*16 + 2*(d/16) + (o%4)/2,  nibble o%2
 *   NVFP4 V scale  128 B: byte ((o/4)*8 + j)*4 + o%4
 *   FP8   K       2048 B: byte ((d/32)*16 + o)*32 + d%32
 *   FP8   V       2048 B: byte ((o/4)*16 + d%16)*32 + (d/16)*4 + o%4
 * In NVFP4 V data two tokens (o even and o+1) share each byte; writers update single nibbles.
 *
 * CONVENTIONS.  All pointers are device pointers unless stated; the caller owns all memory; the
 * library allocates and frees nothing and keeps no state besides a per-device CU-count cache and,
 * for nvfp4_paged_decode_attn_noalloc only, one library-held scratch array per device.
 * Every call enqueues work on `stream` and returns without synchronizing.  Calls return an
 * NVKV_* status; nothing is thrown.  Host-side validation covers null pointers, alignment (16 B
 * for pools, q, out and workspace; 4 B for int arrays), shapes, group size and scalar scales.
 * Device-resident contents (page ids, slots, sequence lengths) are NOT validated: an out-of-range
 * value is undefined behaviour.  Concurrent calls on different streams that write the same pool
 * bytes race.
 */
#ifndef NVKV_H
#define NVKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifndef NVKV_API
#define NVKV_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
enum {
  NVKV_OK = 0,
  NVKV_E_INVAL = -1,        /* bad argument (null pointer, misalignment, negative size, bad scale) */
  NVKV_E_UNSUPPORTED = -2,  /* shape outside what the kernels implement (head_dim != 128, page != 16, group > 16) */
  NVKV_E_LAUNCH = -3,       /* a HIP launch or device query failed */
  NVKV_E_WORKSPACE = -4,    /* workspace missing or smaller than the size query returns */
  NVKV_E_SCRATCH = -5       /* the no-allocation decode needs more than the library-held scratch */
};

/* ---- input element types ---- */
enum { NVKV_IN_BF16 = 0, NVKV_IN_FP8_E4M3 = 1 };

/* ---- per-layer cache precision ---- */
enum { NVKV_PREC_NVFP4 = 0, NVKV_PREC_FP8 = 1 };

/* Static string for a status code (never NULL). */
NVKV_API const char* nvkv_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
NVKV_API int nvkv_version(void);

/*
 * nvkv_global_scale -- per-tensor fp32 scale: *out_scale = fp32(max|x| / divisor).
 * [S] "The Core of the Ledger" paragraph 1 (one FP32 scale for the whole tensor); the NVFP4
 * global scale uses divisor 2688 = 6 * 448 (E2M1 max times E4M3 max), the per-tensor FP8 scale of
 * a sensitive layer ([O] "03 Mixed-precision KV Cache") uses 448.
 *   x          : n elements of `in_dtype` (bf16, or E4M3 bytes meaning e4m3 * in_scale), device.
 *   out_scale  : one float, device.  Written by the second of two kernels.
 *   workspace  : >= nvkv_global_scale_workspace_size() bytes, device, 16-B aligned.
 * Returns NVKV_E_INVAL for n == 0, a non-positive divisor or in_scale, or null pointers.
 */
NVKV_API size_t nvkv_global_scale_workspace_size(void);
NVKV_API int nvkv_global_scale(const void* x, int in_dtype, float in_scale, size_t n, float divisor,
                      float* out_scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_kv_quantize_append -- quantize-on-write of n_tok tokens of K and V into the NVFP4 pools.
 * [S] "Three Paths" paragraphs 1-2 (prefill and extend quantize K/V into the persistent NVFP4
 * cache), [O] "02 NVFP4 KV Cache" (the quantized write path).
 *   k_in, v_in   : [n_tok][num_kv_heads][128] of in_dtype (bf16 or E4M3 bytes), device, 16-B aligned.
 *   k_in_scale, v_in_scale : fp32 scale of E4M3 input (x = e4m3 * scale); ignored for bf16.
 *   slots        : [n_tok] int32, device: destination slot of each token (page * 16 + offset).
 *                  Slots must be distinct and < num_pages * 16 (not checked).
 *   k_global_scale, v_global_scale : g of each tensor, finite and > 0 (from nvkv_global_scale).
 *   k_data, k_scale, v_data, v_scale : the NVFP4 pools (layout above), modified in place.
 * Only the bytes (and, in V data, the nibbles) of the given slots are written.
 */
NVKV_API int nvfp4_kv_quantize_append(const void* k_in, const void* v_in, int in_dtype,
                             float k_in_scale, float v_in_scale,
                             const int32_t* slots, int n_tok, int num_kv_heads, int head_dim, int page_size,
                             float k_global_scale, float v_global_scale,
                             uint8_t* k_data, uint8_t* k_scale, uint8_t* v_data, uint8_t* v_scale,
                             hipStream_t stream);

/*
 * fp8_kv_quantize_append -- per-tensor-scaled FP8 E4M3 write for the sensitive layers
 * ([O] "03 Mixed-precision KV Cache").  byte = E4M3_rne_sat(fp32(x / scale)), sign kept.
 *   k_in, v_in : [n_tok][num_kv_heads][128] bf16, device.  slots as above.
 *   k_cache, v_cache : FP8 pools (layout above).
 */
NVKV_API int fp8_kv_quantize_append(const void* k_in, const void* v_in, const int32_t* slots, int n_tok,
                           int num_kv_heads, int head_dim, int page_size, float k_scale, float v_scale,
                           uint8_t* k_cache, uint8_t* v_cache, hipStream_t stream);

/*
 * Split planning for decode.  The step's work -- the pages of every (sequence b, kv head h) stream,
 * in that order -- is cut into num_splits pieces of equal cost, one workgroup of four wavefronts
 * each.  When the sequence lengths differ, each stream is also charged a fixed cost of 48 pages (the
 * start-up of a segment), so a piece that holds many short streams gets fewer pages.  A piece
 * takes max(pages_per_split, the even ceiling of the step's cost / num_splits) units.  When the
 * lengths are equal and num_splits is even, pieces 2k and 2k + 1 (the two workgroups that share a
 * compute unit) split their two pieces' units 9 : 7, the larger part going to the workgroup the
 * hardware dispatches first.
 * A workgroup walks the streams its piece holds: the four wavefronts split each stream's part
 * and combine in LDS.  A stream that lies in one piece is written out directly.  A stream split
 * over several pieces leaves one partial softmax state per piece.  The last of those pieces to
 * finish merges them (log-sum-exp), found by an arrival count per stream.  A decode is one
 * kernel launch.
 * nvkv_plan_decode picks num_splits from host-side hints: two pieces per compute unit (all
 * resident at once), or fewer for a small step so that pieces keep at least 16 pages.
 *   max_seq_len  : the longest sequence (tokens, including an appended token), > 0.
 *   total_tokens : sum of sequence lengths if known, else 0 (then batch * max_seq_len is assumed).
 *   force_pages_per_split : > 0 asks for pieces of that many pages (rounded up to even, at most the
 *                  step); num_splits then covers the hinted step.  0 = automatic.
 * Outputs *pages_per_split (>= 2, the minimum piece size) and *num_splits (>= 1).  Any plan
 * computes the same attention (up to the order of the fp32 sums).  A step larger than the hints
 * only makes the pieces larger.
 */
NVKV_API int nvkv_plan_decode(int batch, int num_kv_heads, int max_seq_len, long long total_tokens,
                     int force_pages_per_split, int* pages_per_split, int* num_splits);

/*
 * Workspace bytes for decode with the given plan: partial states for (num_splits + batch *
 * num_kv_heads) pieces-by-streams of (num_q_heads / num_kv_heads) rows of 130 floats, then one
 * 64-bit arrival word per stream.  The size is 0 when num_splits == 1, because one piece holds
 * every stream whole.  The contents need no initialisation: partials are written before they are
 * read, and every launch tags the arrival words with its own generation number, so a word left by
 * another call or plan, or any byte pattern in a fresh allocation, reads as no arrivals.  One
 * workspace may serve calls of any plan and shape in turn; calls that overlap in time on one
 * workspace race.
 */
NVKV_API size_t nvkv_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                           int num_splits);

/*
 * nvfp4_paged_decode_attn -- one decode step of attention reading the NVFP4 cache directly.
 * [S] "Three Paths" paragraph 3: decode reads NVFP4 K/V and the E4M3 block scales from memory and
 * dequantizes on the fly; paragraph 4: decode is memory-bound and must read only what it uses.
 * Computes, for every sequence b and query head h (kv head h / (num_q_heads / num_kv_heads)):
 *     out[b][h] = sum_t softmax_t(sm_scale * <q[b][h], K_hat_t>) * V_hat_t,  t < seq_lens[b]
 * with K_hat, V_hat the dequantized cache.  Arithmetic: E2M1 x E4M3 products are exact in fp16,
 * q is rounded to fp16 after a per-row power-of-two rescale, QK^T and PV accumulate in fp32 on the
 * matrix cores, P enters PV as an fp16 hi + lo pair, output is fp32.
 *   q          : [batch][num_q_heads][128] bf16, device.
 *   page_table : [batch][max_pages_per_seq] int32, device.
 *   seq_lens   : [batch] int32, device, each >= 1 and <= max_pages_per_seq * 16 (includes the
 *                appended token when new_k != NULL).  NVKV_E_UNSUPPORTED when
 *                batch * (max_pages_per_seq + 48) * num_kv_heads + 2 * num_splits or
 *                num_splits * pages_per_split exceeds 2^31 - 1 (32-bit unit offsets).
 *   num_q_heads / num_kv_heads must be an integer in 1..16.
 *   pages_per_split, num_splits : from nvkv_plan_decode.
 *   new_k, new_v : NULL, or [batch][num_kv_heads][128] bf16: fused quantize-append of one token
 *                  per sequence at position seq_lens[b] - 1 (its page must be in the page table)
 *                  before attending; uses k_global_scale / v_global_scale.  Both or neither.  The
 *                  bytes written equal nvfp4_kv_quantize_append's for every input without NaN
 *                  (+-inf saturates to a 448 block scale and code +-6); NaN input is outside the
 *                  contract of both writers.
 *   out        : [batch][num_q_heads][128] fp32, device.
 *   workspace  : >= nvkv_decode_workspace_size(...) bytes, device (may be NULL if that is 0).
 */
NVKV_API int nvfp4_paged_decode_attn(const void* q,
                            const uint8_t* k_data, const uint8_t* k_scale,
                            const uint8_t* v_data, const uint8_t* v_scale,
                            float k_global_scale, float v_global_scale,
                            const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                            int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            float sm_scale, int pages_per_split, int num_splits,
                            const void* new_k, const void* new_v,
                            float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_paged_decode_attn_timed -- nvfp4_paged_decode_attn with a measurement hook: split_start and
 * split_stop (hipEvent_t created by the caller, or NULL) are recorded by the dispatch of the decode
 * kernel itself (an extended launch), so hipEventElapsedTime(split_start, split_stop) is that
 * kernel's execution time -- the whole decode, merge included -- and no command is added to the
 * stream.  Arguments, results and errors as above.
 */
NVKV_API int nvfp4_paged_decode_attn_timed(const void* q,
                            const uint8_t* k_data, const uint8_t* k_scale,
                            const uint8_t* v_data, const uint8_t* v_scale,
                            float k_global_scale, float v_global_scale,
                            const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                            int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            float sm_scale, int pages_per_split, int num_splits,
                            const void* new_k, const void* new_v,
                            float* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                            hipEvent_t split_start, hipEvent_t split_stop);

/*
 * nvfp4_paged_decode_attn_noalloc -- nvfp4_paged_decode_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc): the
 * split partials live in a library-held array of nvkv_decode_noalloc_max_bytes() bytes (32 MiB) per
 * device instead of a caller workspace, so nothing is allocated.  The caller still passes q, the
 * pools, the tables and out.  Arguments, results and the other errors as nvfp4_paged_decode_attn.
 *   Returns NVKV_E_SCRATCH when nvkv_decode_workspace_size(batch, num_q_heads, num_kv_heads, 128,
 *   num_splits) exceeds nvkv_decode_noalloc_max_bytes(); NVKV_E_LAUNCH if the array's device address
 *   cannot be resolved (done once per device, on the first call with that device current).
 *   Every call on a device shares that device's array (it keeps the last call's partials, which the
 *   kernels overwrite before reading): calls that overlap on one device -- concurrent streams or
 *   threads -- race and must be serialised by the caller.  The array stays allocated on each device
 *   the library ran on until the process ends.
 */
NVKV_API size_t nvkv_decode_noalloc_max_bytes(void);
NVKV_API int nvfp4_paged_decode_attn_noalloc(const void* q,
                            const uint8_t* k_data, const uint8_t* k_scale,
                            const uint8_t* v_data, const uint8_t* v_scale,
                            float k_global_scale, float v_global_scale,
                            const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                            int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                            float sm_scale, int pages_per_split, int num_splits,
                            const void* new_k, const void* new_v,
                            float* out, hipStream_t stream);

/*
 * fp8_paged_decode_attn -- the same decode step over a per-tensor-scaled FP8 E4M3 cache (the
 * sensitive layers of a mixed-precision stack, [O] "03 Mixed-precision KV Cache").
 * K_hat = e4m3 * k_scale, V_hat = e4m3 * v_scale.  Arguments as above.
 */
NVKV_API int fp8_paged_decode_attn(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                          float k_scale, float v_scale,
                          const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                          int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                          float sm_scale, int pages_per_split, int num_splits,
                          float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvkv_decode_layers -- one decode step across a stack of layers with a per-layer precision map
 * ([O] "03 Mixed-precision KV Cache": FP8 for the sensitive first and last layers, NVFP4 for the
 * rest).  Layers share the page table, sequence lengths, shapes, split plan and workspace and run
 * in order on `stream`.  For an FP8 layer k_data / v_data are the FP8 pools and k_scale / v_scale
 * are ignored; k_gscale / v_gscale are the NVFP4 global scales or the FP8 per-tensor scales.
 */
typedef struct nvkv_layer {
  int precision;              /* NVKV_PREC_NVFP4 or NVKV_PREC_FP8 */
  const void* q;              /* [batch][num_q_heads][128] bf16 */
  const uint8_t* k_data;
  const uint8_t* k_scale;     /* NVFP4 only */
  const uint8_t* v_data;
  const uint8_t* v_scale;     /* NVFP4 only */
  float k_gscale;
  float v_gscale;
  float* out;                 /* [batch][num_q_heads][128] fp32 */
} nvkv_layer;

NVKV_API int nvkv_decode_layers(const nvkv_layer* layers, int num_layers,
                       const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                       int batch, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                       float sm_scale, int pages_per_split, int num_splits,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_dequant_to_workspace -- chunked-extend prefix gather ([S] "Three Paths" paragraph 2): the
 * cached NVFP4 prefix of each sequence is gathered through the page table and dequantized into a
 * dense FP8 E4M3 workspace shared across layers, using the FP8 scale the extend attention uses:
 *     w = E4M3_rne_sat(fp32(fp32(fp32(e2m1 * s_blk) * g) / ws_scale)), sign of the E2M1 code.
 *   prefix_lens : [batch] int32, device: tokens 0..prefix_lens[b]-1 are gathered.
 *   ws_offsets  : [batch + 1] int32, device: sequence b goes to workspace rows
 *                 ws_offsets[b] .. ws_offsets[b] + prefix_lens[b] - 1.
 *   max_prefix_len : host upper bound of prefix_lens (sizes the grid); longer prefixes are cut.
 *   k_ws, v_ws  : [rows][num_kv_heads][128] E4M3, device.
 */
NVKV_API int nvfp4_dequant_to_workspace(const uint8_t* k_data, const uint8_t* k_scale,
                               const uint8_t* v_data, const uint8_t* v_scale,
                               float k_global_scale, float v_global_scale,
                               const int32_t* page_table, int max_pages_per_seq,
                               const int32_t* prefix_lens, const int32_t* ws_offsets,
                               int batch, int num_kv_heads, int head_dim, int page_size, int max_prefix_len,
                               float k_ws_scale, float v_ws_scale,
                               uint8_t* k_ws, uint8_t* v_ws, hipStream_t stream);

/*
 * nvfp4_prefill_write -- the prefill path's single-pass write ([S] "Three Paths" paragraph 1 and
 * summary bullet 2: prefill quantizes K/V into the persistent NVFP4 cache and attends with BF16 Q
 * against FP8 K/V, without reading the cache): nvfp4_kv_quantize_append, plus every token's K and V
 * as E4M3_rne_sat(fp32(x / ws_scale)) in row t (input order) of a dense FP8 copy that
 * fp8_extend_attn reads with prefix_lens = 0 and ws_offsets = the token offsets of each sequence.
 *   k_ws, v_ws : [n_tok][num_kv_heads][128] E4M3, device, 16-byte aligned.
 * Other arguments, errors and the no-op at n_tok == 0 as nvfp4_kv_quantize_append, plus bad
 * ws scales (NVKV_E_INVAL).
 */
NVKV_API int nvfp4_prefill_write(const void* k_in, const void* v_in, int in_dtype,
                        float k_in_scale, float v_in_scale, const int32_t* slots, int n_tok,
                        int num_kv_heads, int head_dim, int page_size,
                        float k_global_scale, float v_global_scale,
                        uint8_t* k_data, uint8_t* k_scale, uint8_t* v_data, uint8_t* v_scale,
                        float k_ws_scale, float v_ws_scale, uint8_t* k_ws, uint8_t* v_ws, hipStream_t stream);

/*
 * fp8_workspace_append -- the extend chunk's own K/V join its prefix in the FP8 workspace ([S]
 * "Three Paths" paragraph 2: the extend attention runs over prefix || chunk in FP8):
 *     w = E4M3_rne_sat(fp32(x / ws_scale)), x the bf16 value (the FP8 encoding of the mixed-precision
 *     layers, [O] "03 Mixed-precision KV Cache").
 *   k, v          : [total_chunk][num_kv_heads][128] bf16, device: the chunks of all sequences,
 *                   concatenated; sequence b's rows are chunk_offsets[b] .. chunk_offsets[b+1]-1.
 *   chunk_offsets : [batch + 1] int32, device, non-decreasing; chunk lengths <= max_chunk_len.
 *   ws_offsets, prefix_lens : as for nvfp4_dequant_to_workspace; chunk row i of sequence b goes to
 *                   workspace row ws_offsets[b] + prefix_lens[b] + i.
 *   max_chunk_len, max_prefix_len : host upper bounds (grid size, offset range checks).
 * Bytes are written only to those rows.  Errors: NVKV_E_INVAL for null / misaligned pointers (16
 * bytes for k, v, k_ws, v_ws; 4 for the int32 arrays), batch outside [1, 65535], negative bounds,
 * bad scales, or a workspace span (max_prefix_len + max_chunk_len) * num_kv_heads * 128 of 2^31
 * bytes or more; NVKV_E_UNSUPPORTED for head_dim != 128.  max_chunk_len == 0 is a no-op.
 */
NVKV_API int fp8_workspace_append(const void* k, const void* v, const int32_t* chunk_offsets,
                         const int32_t* ws_offsets, const int32_t* prefix_lens,
                         int batch, int num_kv_heads, int head_dim, int max_chunk_len, int max_prefix_len,
                         float k_ws_scale, float v_ws_scale, uint8_t* k_ws, uint8_t* v_ws, hipStream_t stream);

/*
 * fp8_extend_attn -- chunked-extend attention ([S] "Three Paths" paragraph 2; summary bullet 2:
 * BF16 Q against FP8 KV): the chunk's queries attend over their sequence's prefix || chunk in the
 * FP8 workspace, causally.  For chunk row i of sequence b and query head hq (kv head hq / G):
 *     z_j = sm_scale * <q, k_ws_scale * e4m3(K_j)>,  j = 0 .. prefix_lens[b] + i,
 *     out = v_ws_scale * sum_j softmax(z)_j e4m3(V_j),
 * with key j at workspace row ws_offsets[b] + j (the prefix rows, then the chunk rows).
 *   q             : [total_chunk][num_q_heads][128] bf16, device, rows as chunk_offsets.
 *   k_ws, v_ws    : [rows][num_kv_heads][128] E4M3, device (written by nvfp4_dequant_to_workspace
 *                   and fp8_workspace_append).
 *   out           : [total_chunk][num_q_heads][128] fp32, device; every row of every chunk is written.
 *   max_chunk_len, max_prefix_len : host upper bounds of the chunk lengths and prefix_lens.
 * Computed with bf16 q x bf16 K (exact from E4M3) on the matrix cores, fp32 scores, softmax weights
 * as an fp16 hi + lo pair x fp16 V (exact from E4M3), fp32 accumulation.  The workspace rows a call
 * reads must hold no E4M3 NaN byte (0x7F, 0xFF; the library's writers produce none from finite
 * inputs), and q must be finite.  Errors as fp8_workspace_append, plus NVKV_E_INVAL /
 * NVKV_E_UNSUPPORTED for the head counts (as the decode calls) and a bad sm_scale.
 */
NVKV_API int fp8_extend_attn(const void* q, const int32_t* chunk_offsets,
                    const uint8_t* k_ws, const uint8_t* v_ws,
                    const int32_t* ws_offsets, const int32_t* prefix_lens,
                    float k_ws_scale, float v_ws_scale, float sm_scale,
                    int batch, int num_q_heads, int num_kv_heads, int head_dim,
                    int max_chunk_len, int max_prefix_len, float* out, hipStream_t stream);

/*
 * nvkv_read_probe -- measurement helper, not part of the attention path: reads `bytes` bytes at
 * `buf` once with coalesced 16-byte loads spread over the whole device (eight 256-thread
 * workgroups per compute unit, grid-stride).  Each thread folds its words by xor and writes the
 * fold to *sink only if it equals 0x9E3779B9, so the loads cannot be elided and normally nothing
 * is written.  Timing it gives the streaming-read rate of the device, the practical ceiling for
 * the decode's reads (the quoted HBM peak is not reached by any read pattern).
 *   buf   : device, 16-byte aligned; bytes >= 16 and a multiple of 16.
 *   sink  : device, 4 bytes, 4-byte aligned.
 * Errors: NVKV_E_INVAL for a null pointer, misalignment or a bad size; NVKV_E_LAUNCH.
 */
NVKV_API int nvkv_read_probe(const void* buf, size_t bytes, unsigned* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVKV_H */

// Host-only driver of the C ABI layer (bit_paged_kv_amd/csrc/nvkv_api.cpp), built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitize.py.
//
// The HIP launchers and the three HIP runtime calls the layer makes are replaced by stubs that only
// record what they were given, so every path of the layer -- argument validation, split planning,
// workspace sizing, per-layer dispatch -- runs to its end on the CPU, including the calls that
// would launch kernels.  Pointers are fake, aligned addresses that nothing dereferences.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <vector>

#include "../../include/nvkv.h"
#include "../../bit_paged_kv_amd/csrc/nvkv_launch.h"

// ---- stubs -----------------------------------------------------------------------------------
static int g_launches = 0;            // launcher calls since the last reset
static nvkv::DecodeArgs g_last_decode{};
static char g_scratch_anchor alignas(256)[256];

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
}

namespace nvkv {
size_t global_scale_workspace_bytes() { return 4096; }
hipError_t launch_global_scale(const void*, int, float, size_t, float, float*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_nvfp4_quantize(const void*, const void*, int, float, float, const int32_t*, int, int, float, float,
                                 uint8_t*, uint8_t*, uint8_t*, uint8_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_nvfp4_prefill_write(const void*, const void*, int, float, float, const int32_t*, int, int, float,
                                      float, uint8_t*, uint8_t*, uint8_t*, uint8_t*, float, float, uint8_t*, uint8_t*,
                                      hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fp8_quantize(const void*, const void*, const int32_t*, int, int, float, float, uint8_t*, uint8_t*,
                               hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dequant_to_ws(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, float, float,
                                const int32_t*, int, const int32_t*, const int32_t*, int, int, int, float, float,
                                uint8_t*, uint8_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fp8_ws_append(const void*, const void*, const int32_t*, const int32_t*, const int32_t*, int, int,
                                int, float, float, uint8_t*, uint8_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_extend_attn(const void*, const int32_t*, const uint8_t*, const uint8_t*, const int32_t*,
                              const int32_t*, float, float, float, int, int, int, int, int, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t, hipEvent_t, hipEvent_t) {
  ++g_launches;
  g_last_decode = a;
  return hipSuccess;
}
hipError_t decode_scratch(void** p) {
  *p = g_scratch_anchor;
  return hipSuccess;
}
hipError_t launch_read_probe(const void*, size_t, unsigned*, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace nvkv

// ---- checks ----------------------------------------------------------------------------------
static int g_failed = 0, g_checks = 0;
#define CHECK(cond)                                                                   \
  do {                                                                                \
    ++g_checks;                                                                       \
    if (!(cond)) {                                                                    \
      ++g_failed;                                                                     \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond);      \
    }                                                                                 \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t A = 1u << 20;      // 16-byte aligned
static const uintptr_t MIS = A + 4;

template <class T>
static T* P(uintptr_t a) {
  return static_cast<T*>(fake(a));
}

struct Dec {
  uintptr_t q = A, kd = A, ks = A, vd = A, vs = A, pt = A, sl = A, out = A, ws = A, nk = 0, nv = 0;
  float gk = 1.f, gv = 1.f, sm = 0.1f;
  int maxp = 4, b = 1, hq = 8, hkv = 2, d = 128, page = 16, pps = 2, ns = 1;
  size_t wsb = 1 << 20;
  int run() const {
    return nvfp4_paged_decode_attn(P<void>(q), P<uint8_t>(kd), P<uint8_t>(ks), P<uint8_t>(vd), P<uint8_t>(vs), gk, gv,
                                   P<int32_t>(pt), maxp, P<int32_t>(sl), b, hq, hkv, d, page, sm, pps, ns,
                                   nk ? P<void>(nk) : nullptr, nv ? P<void>(nv) : nullptr, P<float>(out),
                                   ws ? P<void>(ws) : nullptr, wsb, nullptr);
  }
  int run_noalloc() const {
    return nvfp4_paged_decode_attn_noalloc(P<void>(q), P<uint8_t>(kd), P<uint8_t>(ks), P<uint8_t>(vd),
                                           P<uint8_t>(vs), gk, gv, P<int32_t>(pt), maxp, P<int32_t>(sl), b, hq, hkv, d,
                                           page, sm, pps, ns, nk ? P<void>(nk) : nullptr, nv ? P<void>(nv) : nullptr,
                                           P<float>(out), nullptr);
  }
  int run_fp8() const {
    return fp8_paged_decode_attn(P<void>(q), P<uint8_t>(kd), P<uint8_t>(vd), gk, gv, P<int32_t>(pt), maxp,
                                 P<int32_t>(sl), b, hq, hkv, d, page, sm, pps, ns, P<float>(out),
                                 ws ? P<void>(ws) : nullptr, wsb, nullptr);
  }
};

static void check_plans() {
  const int batches[] = {1, 3, 4, 32, 44, 64, 1000, 65535};
  const int heads[] = {1, 2, 8, 64};
  const int lens[] = {1, 15, 16, 17, 256, 4096, 8192, 131072, 1 << 24, INT_MAX};
  for (int b : batches)
    for (int h : heads)
      for (int L : lens)
        for (long long tot : {0LL, (long long)b * L / 3 + 1, (long long)b * L})
          for (int force : {0, 1, 2, 7, 512, INT_MAX}) {
            int pps = -1, ns = -1;
            const int st = nvkv_plan_decode(b, h, L, tot, force, &pps, &ns);
            CHECK(st == NVKV_OK || st == NVKV_E_UNSUPPORTED);
            if (st != NVKV_OK) continue;
            long long pages = (long long)b * (((long long)L + 15) / 16);
            if (tot > 0) pages = std::min(pages, (tot + 15LL * b) / 16);
            const long long units = std::max(1LL, pages * h);
            CHECK(pps >= 2 && pps % 2 == 0 && ns >= 1);
            CHECK((long long)ns * pps <= 0x7FFFFFFFLL);
            if (force == 0) CHECK(pps == 2 && ns == std::min(512LL, (units + 15) / 16));
            else CHECK((long long)ns * pps >= units && (long long)(ns - 1) * pps < units);
          }
  int pps, ns;
  CHECK(nvkv_plan_decode(0, 8, 10, 0, 0, &pps, &ns) == NVKV_E_INVAL);
  CHECK(nvkv_plan_decode(1, 8, 0, 0, 0, &pps, &ns) == NVKV_E_INVAL);
  CHECK(nvkv_plan_decode(1, 8, 10, -1, 0, &pps, &ns) == NVKV_E_INVAL);
  CHECK(nvkv_plan_decode(1, 8, 10, 0, -1, &pps, &ns) == NVKV_E_INVAL);
  CHECK(nvkv_plan_decode(1, 8, 10, 0, 0, nullptr, &ns) == NVKV_E_INVAL);
  // the long-context plan: two pieces per compute unit
  CHECK(nvkv_plan_decode(4, 8, 131072, 4LL * 131072, 0, &pps, &ns) == NVKV_OK && pps == 2 && ns == 512);
}

static void check_decode() {
  Dec ok;
  g_launches = 0;
  CHECK(ok.run() == NVKV_OK && g_launches == 1);
  CHECK(g_last_decode.format == nvkv::kFmtNvfp4 && g_last_decode.num_splits == 1 && g_last_decode.hq == 8);
  Dec d;
  struct {
    void (*set)(Dec&);
    int want;
  } cases[] = {
      {[](Dec& x) { x.q = 0; }, NVKV_E_INVAL},           {[](Dec& x) { x.kd = 0; }, NVKV_E_INVAL},
      {[](Dec& x) { x.out = MIS; }, NVKV_E_INVAL},       {[](Dec& x) { x.sl = A + 2; }, NVKV_E_INVAL},
      {[](Dec& x) { x.d = 64; }, NVKV_E_UNSUPPORTED},    {[](Dec& x) { x.page = 32; }, NVKV_E_UNSUPPORTED},
      {[](Dec& x) { x.hq = 7; }, NVKV_E_INVAL},          {[](Dec& x) { x.hq = 64; }, NVKV_E_UNSUPPORTED},
      {[](Dec& x) { x.gk = NAN; }, NVKV_E_INVAL},        {[](Dec& x) { x.gv = INFINITY; }, NVKV_E_INVAL},
      {[](Dec& x) { x.gk = 1e-40f; }, NVKV_E_INVAL},     {[](Dec& x) { x.sm = -1.f; }, NVKV_E_INVAL},
      {[](Dec& x) { x.b = 0; }, NVKV_E_INVAL},           {[](Dec& x) { x.b = 70000; }, NVKV_E_INVAL},
      {[](Dec& x) { x.nk = A; }, NVKV_E_INVAL},          {[](Dec& x) { x.ns = 4, x.ws = 0; }, NVKV_E_WORKSPACE},
      {[](Dec& x) { x.ns = 4, x.wsb = 100; }, NVKV_E_WORKSPACE},
      {[](Dec& x) { x.ns = 4, x.ws = MIS; }, NVKV_E_INVAL},
      {[](Dec& x) { x.ns = INT_MAX, x.b = 2, x.hkv = 2, x.hq = 2; }, NVKV_E_UNSUPPORTED},
      {[](Dec& x) { x.maxp = 1 << 30; }, NVKV_E_UNSUPPORTED},   // page-heads past 32 bits
      {[](Dec& x) { x.ns = 1 << 28, x.pps = 8; }, NVKV_E_UNSUPPORTED},
  };
  for (auto& c : cases) {
    Dec x;
    c.set(x);
    g_launches = 0;
    CHECK(x.run() == c.want);
    CHECK(g_launches == 0);
  }
  // several splits: the workspace pointer reaches the launcher
  d.ns = 4;
  g_launches = 0;
  CHECK(d.run() == NVKV_OK && g_launches == 1 && g_last_decode.workspace == fake(A));
  // fused append arguments pass through
  d.nk = A + 16, d.nv = A + 32;
  CHECK(d.run() == NVKV_OK && g_last_decode.new_k == fake(A + 16) && g_last_decode.new_v == fake(A + 32));
  // the FP8 call
  Dec f;
  g_launches = 0;
  CHECK(f.run_fp8() == NVKV_OK && g_launches == 1 && g_last_decode.format == nvkv::kFmtFp8);
  f.vd = 0;
  CHECK(f.run_fp8() == NVKV_E_INVAL);
  // the no-allocation call: the library's array replaces the workspace
  Dec n;
  n.ns = 4;
  g_launches = 0;
  CHECK(n.run_noalloc() == NVKV_OK && g_launches == 1 && g_last_decode.workspace == g_scratch_anchor);
  n.b = 64, n.hq = 64, n.hkv = 8, n.ns = 7553;     // (7553 + 512) x 8 x 520 B of partials + arrival words > 32 MiB
  g_launches = 0;
  CHECK(n.run_noalloc() == NVKV_E_SCRATCH && g_launches == 0);
  n.ns = 7552;
  CHECK(n.run_noalloc() == NVKV_OK && g_launches == 1);
  n.q = 0;
  CHECK(n.run_noalloc() == NVKV_E_INVAL);
  CHECK(nvkv_decode_noalloc_max_bytes() == (size_t)32 << 20);
  // workspace sizes
  CHECK(nvkv_decode_workspace_size(4, 64, 8, 128, 1) == 0);
  CHECK(nvkv_decode_workspace_size(4, 64, 8, 128, 16) == (size_t)(16 + 32) * 8 * 130 * 4 + 32 * 8);
  // every launch carries its own nonzero generation number
  {
    Dec g1, g2;
    g1.ns = g2.ns = 4;
    CHECK(g1.run() == NVKV_OK);
    const unsigned first = g_last_decode.gen;
    CHECK(g2.run() == NVKV_OK);
    CHECK(first != 0 && g_last_decode.gen != 0 && g_last_decode.gen != first);
  }
  CHECK(nvkv_decode_workspace_size(4, 64, 8, 64, 16) == 0);
  CHECK(nvkv_decode_workspace_size(0, 64, 8, 128, 16) == 0);
}

static void check_layers() {
  nvkv_layer L[3];
  for (auto& l : L) {
    memset(&l, 0, sizeof l);
    l.precision = NVKV_PREC_NVFP4;
    l.q = fake(A);
    l.k_data = P<uint8_t>(A);
    l.k_scale = P<uint8_t>(A);
    l.v_data = P<uint8_t>(A);
    l.v_scale = P<uint8_t>(A);
    l.k_gscale = l.v_gscale = 1.f;
    l.out = P<float>(A);
  }
  L[1].precision = NVKV_PREC_FP8;
  L[1].k_scale = L[1].v_scale = nullptr;
  g_launches = 0;
  CHECK(nvkv_decode_layers(L, 3, P<int32_t>(A), 4, P<int32_t>(A), 1, 8, 2, 128, 16, 0.1f, 2, 4, fake(A), 1 << 20,
                           nullptr) == NVKV_OK);
  CHECK(g_launches == 3);
  L[2].v_gscale = 0.f;                      // one bad layer: nothing is launched
  g_launches = 0;
  CHECK(nvkv_decode_layers(L, 3, P<int32_t>(A), 4, P<int32_t>(A), 1, 8, 2, 128, 16, 0.1f, 2, 4, fake(A), 1 << 20,
                           nullptr) == NVKV_E_INVAL);
  CHECK(g_launches == 0);
  L[2].v_gscale = 1.f;
  L[0].precision = 7;
  CHECK(nvkv_decode_layers(L, 3, P<int32_t>(A), 4, P<int32_t>(A), 1, 8, 2, 128, 16, 0.1f, 2, 4, fake(A), 1 << 20,
                           nullptr) == NVKV_E_INVAL);
  CHECK(nvkv_decode_layers(nullptr, 3, P<int32_t>(A), 4, P<int32_t>(A), 1, 8, 2, 128, 16, 0.1f, 2, 4, fake(A),
                           1 << 20, nullptr) == NVKV_E_INVAL);
  CHECK(g_launches == 0);
}

static void check_writers() {
  uint8_t* u = P<uint8_t>(A);
  const int32_t* sl = P<int32_t>(A);
  g_launches = 0;
  CHECK(nvfp4_kv_quantize_append(u, u, NVKV_IN_BF16, 1.f, 1.f, sl, 5, 8, 128, 16, 0.5f, 0.5f, u, u, u, u, nullptr) ==
        NVKV_OK);
  CHECK(nvfp4_kv_quantize_append(u, u, NVKV_IN_FP8_E4M3, 2.f, 2.f, sl, 5, 8, 128, 16, 0.5f, 0.5f, u, u, u, u,
                                 nullptr) == NVKV_OK);
  CHECK(g_launches == 2);
  CHECK(nvfp4_kv_quantize_append(u, u, NVKV_IN_BF16, 1.f, 1.f, sl, 0, 8, 128, 16, 0.5f, 0.5f, nullptr, nullptr,
                                 nullptr, nullptr, nullptr) == NVKV_OK);   // n_tok 0: nothing to do
  CHECK(g_launches == 2);
  CHECK(nvfp4_kv_quantize_append(u, u, 5, 1.f, 1.f, sl, 5, 8, 128, 16, 0.5f, 0.5f, u, u, u, u, nullptr) ==
        NVKV_E_INVAL);
  CHECK(nvfp4_kv_quantize_append(u, u, NVKV_IN_FP8_E4M3, 0.f, 1.f, sl, 5, 8, 128, 16, 0.5f, 0.5f, u, u, u, u,
                                 nullptr) == NVKV_E_INVAL);
  CHECK(nvfp4_kv_quantize_append(P<uint8_t>(MIS), u, NVKV_IN_BF16, 1.f, 1.f, sl, 5, 8, 128, 16, 0.5f, 0.5f, u, u, u,
                                 u, nullptr) == NVKV_E_INVAL);
  CHECK(nvfp4_kv_quantize_append(u, u, NVKV_IN_BF16, 1.f, 1.f, sl, 5, 70000, 128, 16, 0.5f, 0.5f, u, u, u, u,
                                 nullptr) == NVKV_E_UNSUPPORTED);
  CHECK(nvfp4_kv_quantize_append(u, u, NVKV_IN_BF16, 1.f, 1.f, sl, 5, 8, 96, 16, 0.5f, 0.5f, u, u, u, u, nullptr) ==
        NVKV_E_UNSUPPORTED);
  CHECK(fp8_kv_quantize_append(u, u, sl, 3, 8, 128, 16, 1.f, 1.f, u, u, nullptr) == NVKV_OK);
  CHECK(fp8_kv_quantize_append(u, u, sl, 3, 8, 128, 16, NAN, 1.f, u, u, nullptr) == NVKV_E_INVAL);
  CHECK(nvfp4_prefill_write(u, u, NVKV_IN_BF16, 1.f, 1.f, sl, 9, 8, 128, 16, 1.f, 1.f, u, u, u, u, 6.f, 6.f, u, u,
                            nullptr) == NVKV_OK);
  CHECK(nvfp4_prefill_write(u, u, NVKV_IN_BF16, 1.f, 1.f, sl, 9, 8, 128, 16, 1.f, 1.f, u, u, u, u, -6.f, 6.f, u, u,
                            nullptr) == NVKV_E_INVAL);
  const size_t gws = nvkv_global_scale_workspace_size();
  CHECK(nvkv_global_scale(u, NVKV_IN_BF16, 1.f, 100, 2688.f, P<float>(A), u, gws, nullptr) == NVKV_OK);
  CHECK(nvkv_global_scale(u, NVKV_IN_BF16, 1.f, 100, 2688.f, P<float>(A), u, gws - 1, nullptr) == NVKV_E_WORKSPACE);
  CHECK(nvkv_global_scale(u, NVKV_IN_BF16, 1.f, 0, 2688.f, P<float>(A), u, gws, nullptr) == NVKV_E_INVAL);
  CHECK(nvkv_global_scale(u, NVKV_IN_FP8_E4M3, -1.f, 10, 448.f, P<float>(A), u, gws, nullptr) == NVKV_E_INVAL);
  CHECK(nvfp4_dequant_to_workspace(u, u, u, u, 1.f, 1.f, sl, 4, sl, sl, 2, 8, 128, 16, 64, 6.f, 6.f, u, u,
                                   nullptr) == NVKV_OK);
  CHECK(nvfp4_dequant_to_workspace(u, u, u, u, 1.f, 1.f, sl, 4, sl, sl, 2, 8, 128, 16, 65, 6.f, 6.f, u, u,
                                   nullptr) == NVKV_E_INVAL);       // prefix beyond the page table
  CHECK(fp8_workspace_append(u, u, sl, sl, sl, 2, 8, 128, 2048, 16384, 6.f, 6.f, u, u, nullptr) == NVKV_OK);
  CHECK(fp8_workspace_append(u, u, sl, sl, sl, 2, 8, 128, 1 << 20, 1 << 20, 6.f, 6.f, u, u, nullptr) ==
        NVKV_E_INVAL);                                             // 2^31 workspace bytes
  CHECK(fp8_extend_attn(u, sl, u, u, sl, sl, 6.f, 6.f, 0.1f, 1, 32, 8, 128, 2048, 16384, P<float>(A), nullptr) ==
        NVKV_OK);
  CHECK(fp8_extend_attn(u, sl, u, u, sl, sl, 6.f, 6.f, 0.1f, 1, 33, 8, 128, 2048, 16384, P<float>(A), nullptr) ==
        NVKV_E_INVAL);
  CHECK(nvkv_read_probe(u, 1 << 20, P<unsigned>(A), nullptr) == NVKV_OK);
  CHECK(nvkv_read_probe(u, 17, P<unsigned>(A), nullptr) == NVKV_E_INVAL);
}

int main() {
  for (int st : {0, -1, -2, -3, -4, -5, 12345}) CHECK(nvkv_status_string(st) && strlen(nvkv_status_string(st)) > 0);
  CHECK(nvkv_version() >= 100);
  check_plans();
  check_decode();
  check_layers();
  check_writers();
  printf("%d checks, %d failed\n", g_checks, g_failed);
  return g_failed ? 1 : 0;
}

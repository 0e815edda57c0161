// dg_api.hip -- C ABI of the FP8 block-scaled GEMM library (declared in include/dg.h):
// host-side argument checks, the shape-keyed tile-configuration table, and the
// launches on the caller's stream.
//
// The configuration table plays the role of the pages' per-shape kernel selection
// (the DeepGEMM library news page, youleyou.com, "main features": kernels generated
// per hardware and input shape at run time; the project page, aiproducthub.cn,
// "quick start": DG_PRINT_CONFIGS shows the choice). Here every configuration is
// compiled ahead of time and chosen from the shape on the host.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "../../include/dg.h"
#include "gemm_kernel.hpp"

namespace dg {
namespace {

thread_local char g_detail[512] = "";

dg_status fail(dg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return s;
}

// ---------------------------------------------------------------- config table

enum CfgId : int { kCfg128x128 = 0, kCfg64x64 = 1, kNumCfg };

struct CfgInfo {
  const char* name;
  int bm, bn;
};
const CfgInfo kCfgInfo[kNumCfg] = {
    {"tile128x128_w2x2", 128, 128},
    {"tile64x64_w2x2", 64, 64},
};

using Cfg128 = TileCfg<128, 128, 2, 2>;
using Cfg64 = TileCfg<64, 64, 2, 2>;

// Shape key -> configuration. kind: dense / contiguous / masked; m is the rows per
// problem that matter for tiling (dense M, contiguous average segment, masked
// expected_m).
CfgId select_config(int kind, int64_t m, int64_t n, int64_t k, int32_t g) {
  (void)n;
  (void)k;
  (void)g;
  (void)kind;
  if (m <= 64) return kCfg64x64;
  return kCfg128x128;
}

bool print_configs() {
  static const bool on = [] {
    const char* e = getenv("DG_PRINT_CONFIGS");
    return e && *e && strcmp(e, "0") != 0;
  }();
  return on;
}

void maybe_print(int kind, int64_t M, int64_t N, int64_t K, int32_t G, CfgId id) {
  if (!print_configs()) return;
  static std::mutex mu;
  static std::set<std::tuple<int, int64_t, int64_t, int64_t, int32_t>> seen;
  std::lock_guard<std::mutex> lock(mu);
  if (!seen.insert(std::make_tuple(kind, M, N, K, G)).second) return;
  static const char* kinds[] = {"dense", "contiguous", "masked"};
  fprintf(stderr, "[dg] %s M=%lld N=%lld K=%lld G=%d -> %s\n", kinds[kind], (long long)M,
          (long long)N, (long long)K, G, kCfgInfo[id].name);
}

// ---------------------------------------------------------------- launching

template <class Cfg, int KIND>
dg_status launch_cfg(const Problem& p0, int64_t blocks, hipStream_t stream) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute((const void*)gemm_kernel<Cfg, KIND>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS_BYTES);
  });
  if (attr_err != hipSuccess)
    return fail(DG_ERR_LAUNCH, "hipFuncSetAttribute: %s", hipGetErrorString(attr_err));
  Problem p = p0;
  p.tiles_m = (int32_t)((p.M + Cfg::BM - 1) / Cfg::BM);
  p.tiles_n = (int32_t)((p.N + Cfg::BN - 1) / Cfg::BN);
  const int64_t grid = blocks * p.tiles_m * p.tiles_n;
  if (grid <= 0) return DG_OK;
  if (grid > 0x7FFFFFFF) return fail(DG_ERR_UNSUPPORTED_SHAPE, "grid of %lld tiles", (long long)grid);
  hipLaunchKernelGGL((gemm_kernel<Cfg, KIND>), dim3((unsigned)grid), dim3(Cfg::NT),
                     Cfg::LDS_BYTES, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(DG_ERR_LAUNCH, "launch: %s", hipGetErrorString(err));
  return DG_OK;
}

template <int KIND>
dg_status launch(CfgId id, const Problem& p, int64_t blocks, hipStream_t stream) {
  switch (id) {
    case kCfg128x128:
      return launch_cfg<Cfg128, KIND>(p, blocks, stream);
    case kCfg64x64:
      return launch_cfg<Cfg64, KIND>(p, blocks, stream);
    default:
      return fail(DG_ERR_UNSUPPORTED_SHAPE, "no configuration %d", (int)id);
  }
}

// ---------------------------------------------------------------- validation

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

dg_status check_common(const void* A, const void* B, const void* C, const float* sfA,
                       const float* sfB, int64_t N, int64_t K, bool any_output) {
  if (N < 0 || K < 0) return fail(DG_ERR_BAD_SHAPE, "negative size (N=%lld, K=%lld)",
                                  (long long)N, (long long)K);
  if (K % kKBlock != 0) return fail(DG_ERR_BAD_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
  if (N % 16 != 0) return fail(DG_ERR_BAD_SHAPE, "N=%lld is not a multiple of 16", (long long)N);
  if (!any_output) return DG_OK;
  if (K == 0) return fail(DG_ERR_BAD_SHAPE, "K=0 with outputs to produce");
  if (!A || !B || !C || !sfA || !sfB) return fail(DG_ERR_NULL_POINTER, "NULL operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16))
    return fail(DG_ERR_MISALIGNED, "A, B and C must be 16-byte aligned");
  if (!aligned(sfA, 4) || !aligned(sfB, 4))
    return fail(DG_ERR_MISALIGNED, "sfA and sfB must be 4-byte aligned");
  if (K > (int64_t)1 << 30 || N > (int64_t)1 << 30)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "N or K beyond 2^30");
  return DG_OK;
}

}  // namespace
}  // namespace dg

using namespace dg;

extern "C" {

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "DG_OK";
    case DG_ERR_NULL_POINTER: return "DG_ERR_NULL_POINTER";
    case DG_ERR_BAD_SHAPE: return "DG_ERR_BAD_SHAPE";
    case DG_ERR_UNSUPPORTED_SHAPE: return "DG_ERR_UNSUPPORTED_SHAPE";
    case DG_ERR_MISALIGNED: return "DG_ERR_MISALIGNED";
    case DG_ERR_NO_DEVICE: return "DG_ERR_NO_DEVICE";
    case DG_ERR_LAUNCH: return "DG_ERR_LAUNCH";
  }
  return "DG_ERR_UNKNOWN";
}

const char* dg_last_error_detail(void) { return g_detail; }

dg_status dg_fp8_gemm_nt(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* stream) {
  g_detail[0] = 0;
  if (M < 0) return fail(DG_ERR_BAD_SHAPE, "negative M=%lld", (long long)M);
  dg_status s = check_common(A, B, C, sfA, sfB, N, K, M > 0 && N > 0);
  if (s != DG_OK || M == 0 || N == 0) return s;
  if (M > (int64_t)1 << 30) return fail(DG_ERR_UNSUPPORTED_SHAPE, "M beyond 2^30");
  Problem p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.C = (uint16_t*)C;
  p.sfA = sfA;
  p.sfB = sfB;
  p.M = M;
  p.N = N;
  p.K = K;
  p.G = 1;
  const CfgId id = select_config(kDense, M, N, K, 1);
  maybe_print(kDense, M, N, K, 1, id);
  return launch<kDense>(id, p, 1, (hipStream_t)stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* A, const void* B, void* C,
                                              const float* sfA, const float* sfB,
                                              const int32_t* m_indices, int64_t M_total,
                                              int64_t N, int64_t K, int32_t G, void* stream) {
  g_detail[0] = 0;
  if (M_total < 0) return fail(DG_ERR_BAD_SHAPE, "negative M_total=%lld", (long long)M_total);
  if (G < 1) return fail(DG_ERR_BAD_SHAPE, "G=%d, need at least one expert", G);
  dg_status s = check_common(A, B, C, sfA, sfB, N, K, M_total > 0 && N > 0);
  if (s != DG_OK || M_total == 0 || N == 0) return s;
  if (!m_indices) return fail(DG_ERR_NULL_POINTER, "NULL m_indices");
  if (!aligned(m_indices, 4)) return fail(DG_ERR_MISALIGNED, "m_indices must be 4-byte aligned");
  if (M_total > (int64_t)1 << 30) return fail(DG_ERR_UNSUPPORTED_SHAPE, "M_total beyond 2^30");
  Problem p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.C = (uint16_t*)C;
  p.sfA = sfA;
  p.sfB = sfB;
  p.m_indices = m_indices;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.G = G;
  const CfgId id = select_config(kContiguous, M_total / G, N, K, G);
  maybe_print(kContiguous, M_total, N, K, G, id);
  return launch<kContiguous>(id, p, 1, (hipStream_t)stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* A, const void* B, void* C,
                                          const float* sfA, const float* sfB,
                                          const int32_t* masked_m, int32_t G, int64_t M_max,
                                          int64_t N, int64_t K, int64_t expected_m,
                                          void* stream) {
  g_detail[0] = 0;
  if (M_max < 0) return fail(DG_ERR_BAD_SHAPE, "negative M_max=%lld", (long long)M_max);
  if (G < 1) return fail(DG_ERR_BAD_SHAPE, "G=%d, need at least one expert", G);
  dg_status s = check_common(A, B, C, sfA, sfB, N, K, M_max > 0 && N > 0);
  if (s != DG_OK || M_max == 0 || N == 0) return s;
  if (!masked_m) return fail(DG_ERR_NULL_POINTER, "NULL masked_m");
  if (!aligned(masked_m, 4)) return fail(DG_ERR_MISALIGNED, "masked_m must be 4-byte aligned");
  if (M_max > (int64_t)1 << 30 || (int64_t)G * M_max > (int64_t)1 << 34)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "G*M_max too large");
  Problem p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.C = (uint16_t*)C;
  p.sfA = sfA;
  p.sfB = sfB;
  p.masked_m = masked_m;
  p.M = M_max;
  p.N = N;
  p.K = K;
  p.G = G;
  const int64_t em = expected_m > 0 && expected_m < M_max ? expected_m : M_max;
  const CfgId id = select_config(kMasked, em, N, K, G);
  maybe_print(kMasked, M_max, N, K, G, id);
  return launch<kMasked>(id, p, G, (hipStream_t)stream);
}

dg_status dg_describe_config(int32_t kind, int64_t M, int64_t N, int64_t K, int32_t G,
                             int64_t expected_m, char* buf, int64_t len) {
  if (kind < 0 || kind > 2 || !buf || len <= 0) return DG_ERR_BAD_SHAPE;
  int64_t m = M;
  if (kind == kContiguous) m = G > 0 ? M / G : M;
  if (kind == kMasked) m = expected_m > 0 && expected_m < M ? expected_m : M;
  const CfgId id = select_config(kind, m, N, K, G);
  snprintf(buf, (size_t)len, "%s", kCfgInfo[id].name);
  return DG_OK;
}

}  // extern "C"

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
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/dg.h"
#include "gemm_kernel.hpp"
#include "pipe_kernel.hpp"
#include "quant_kernel.hpp"
#include "skinny_kernel.hpp"
#include "stream_kernel.hpp"
#include "transpose_kernel.hpp"

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

constexpr int64_t kCUs = 256;  // MI355X compute units (8 XCDs x 32)

using Cfg128 = TileCfg<128, 128, 2, 2>;
using Cfg64 = TileCfg<64, 64, 2, 2>;

template <class Cfg, int KIND>
dg_status launch_tile(const Problem& p0, int64_t blocks, hipStream_t stream) {
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

dg_status get_workspace(hipStream_t stream, size_t partial_bytes, size_t counters,
                        float** partials, uint32_t** counter_ptr);

// Dense tail balancing: with T tiles on kCUs CUs (one workgroup each), the last
// r = T mod kCUs tiles would run in a partial round. Each of them is split into
// `parts` K ranges (at least 8 K-blocks each) so that the last round fills the GPU.
struct TailSplit {
  int64_t full, parts;
};

TailSplit pipe_tail_split(int64_t tiles, int64_t KB) {
  TailSplit t{tiles, 1};
  const int64_t r = tiles % kCUs;
  if (r == 0) return t;
  int64_t parts = kCUs / r;
  if (parts > 8) parts = 8;
  if (parts > KB / 8) parts = KB / 8;
  if (parts < 2) return t;
  t.full = tiles - r;
  t.parts = parts;
  return t;
}

template <class Cfg, int KIND, int LAY = 0>
dg_status launch_pipe(const Problem& p0, int64_t blocks, hipStream_t stream) {
  PipeArgs a{};
  a.p = p0;
  Problem& p = a.p;
  p.tiles_m = (int32_t)((p.M + Cfg::BM - 1) / Cfg::BM);
  p.tiles_n = (int32_t)((p.N + Cfg::BN - 1) / Cfg::BN);
  int64_t grid = blocks * p.tiles_m * p.tiles_n;
  if (grid <= 0) return DG_OK;
  if (grid > 0x7FFFFFFF) return fail(DG_ERR_UNSUPPORTED_SHAPE, "grid of %lld tiles", (long long)grid);
  a.full_tiles = (int32_t)grid;
  a.parts = 1;
  if (KIND == kDense) {
    const TailSplit ts = pipe_tail_split(grid, p.K / kKBlock);
    if (ts.parts > 1) {
      const int64_t split = grid - ts.full;
      const size_t bytes = (size_t)(split * ts.parts) * Cfg::BM * Cfg::BN * sizeof(float);
      dg_status st = get_workspace(stream, bytes, (size_t)split, &a.ws, &a.counters);
      if (st != DG_OK) return st;
      a.full_tiles = (int32_t)ts.full;
      a.parts = (int32_t)ts.parts;
      grid = ts.full + split * ts.parts;
    }
  }
  a.items = (int32_t)grid;
  const int64_t wgs = grid < kCUs ? grid : kCUs;  // persistent, one workgroup per CU
  hipLaunchKernelGGL((pipe_kernel<Cfg, KIND, false, LAY>), dim3((unsigned)wgs), dim3(Cfg::NT), 0,
                     stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(DG_ERR_LAUNCH, "launch: %s", hipGetErrorString(err));
  return DG_OK;
}

using Pipe256x128 = PipeCfg<256, 128>;
using Pipe128x256 = PipeCfg<128, 256>;
using Pipe128x256L = PipeCfg<128, 256, 12>;  // long K: scales loaded per 12 K-blocks
constexpr int kLongKB = 32;                  // K-blocks from which the 128x256 tiles use it

// The 128x256-tile kernel, with the scale loads of its K length.
template <int KIND, int LAY = 0>
dg_status launch_pipe128(const Problem& p, int64_t blocks, hipStream_t stream) {
  return p.K / kKBlock >= kLongKB ? launch_pipe<Pipe128x256L, KIND, LAY>(p, blocks, stream)
                                  : launch_pipe<Pipe128x256, KIND, LAY>(p, blocks, stream);
}

// Grouped GEMM with the fused SwiGLU epilogue: p.N = 2 * I rows of B per expert
// ([gate; up]); one 128x256 tile per 128 columns of h.
template <class Cfg, int KIND>
dg_status launch_pipe_swiglu_as(const Problem& p0, int64_t blocks, int64_t I, uint8_t* codes,
                                float* sf, hipStream_t stream) {
  PipeArgs a{};
  a.p = p0;
  a.p.tiles_m = (int32_t)((p0.M + Cfg::BM - 1) / Cfg::BM);
  a.p.tiles_n = (int32_t)(I / 128);
  const int64_t grid = blocks * a.p.tiles_m * a.p.tiles_n;
  if (grid <= 0) return DG_OK;
  if (grid > 0x7FFFFFFF) return fail(DG_ERR_UNSUPPORTED_SHAPE, "grid of %lld tiles", (long long)grid);
  a.full_tiles = (int32_t)grid;
  a.parts = 1;
  a.sw.codes = codes;
  a.sw.sf = sf;
  a.sw.I = (int32_t)I;
  a.items = (int32_t)grid;
  const int64_t wgs = grid < kCUs ? grid : kCUs;  // persistent, one workgroup per CU
  hipLaunchKernelGGL((pipe_kernel<Cfg, KIND, true>), dim3((unsigned)wgs), dim3(Cfg::NT), 0, stream,
                     a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(DG_ERR_LAUNCH, "launch: %s", hipGetErrorString(err));
  return DG_OK;
}

template <int KIND>
dg_status launch_pipe_swiglu(const Problem& p, int64_t blocks, int64_t I, uint8_t* codes,
                             float* sf, hipStream_t stream) {
  return p.K / kKBlock >= kLongKB
             ? launch_pipe_swiglu_as<Pipe128x256L, KIND>(p, blocks, I, codes, sf, stream)
             : launch_pipe_swiglu_as<Pipe128x256, KIND>(p, blocks, I, codes, sf, stream);
}

// ---------------------------------------------------------------- split-K workspace
//
// Launches that split K across workgroups (the M <= 64 kernels, the dense tail
// split of the compute-bound kernel) keep fp32 partials and per-tile arrival
// counters in library-owned device buffers, one set per (device, stream):
// calls on one stream run in order and reuse them; calls on different streams never
// share them. Every counter is zero between calls (zeroed when allocated, reset by
// the kernel after use), so the counter buffer stays valid when a later call uses
// more of it. Buffers only grow. An outgrown buffer is not freed but retired: a HIP
// graph captured earlier may still point at it, so it stays allocated until
// dg_release_workspaces() or the end of the process. A call that would have to
// grow a buffer while its stream is being captured returns DG_ERR_CAPTURE instead
// of allocating (and zeroing) inside the capture.
struct Workspace {
  void* partials = nullptr;
  size_t partial_bytes = 0;
  uint32_t* counters = nullptr;
  size_t counter_count = 0;
  void* a_t = nullptr;  // K-contiguous copies of operands given in another layout
  size_t a_t_bytes = 0;
  void* b_t = nullptr;
  size_t b_t_bytes = 0;
  std::vector<void*> retired;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

dg_status grow(Workspace& w, void** buf, size_t* have, size_t need, size_t elem,
               hipStream_t stream, bool zero) {
  if (*have >= need) return DG_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess)
    return fail(DG_ERR_LAUNCH, "hipStreamIsCapturing: %s", hipGetErrorString(e));
  if (cap != hipStreamCaptureStatusNone)
    return fail(DG_ERR_CAPTURE,
                "the stream is being captured and this shape needs a larger library "
                "workspace (%zu bytes); run the call once on this stream outside capture first",
                need * elem);
  void* fresh = nullptr;
  e = hipMalloc(&fresh, need * elem);
  if (e != hipSuccess)
    return fail(DG_ERR_LAUNCH, "workspace hipMalloc(%zu): %s", need * elem, hipGetErrorString(e));
  if (zero) {
    e = hipMemsetAsync(fresh, 0, need * elem, stream);
    if (e != hipSuccess) {
      (void)hipFree(fresh);
      return fail(DG_ERR_LAUNCH, "workspace clear: %s", hipGetErrorString(e));
    }
  }
  if (*buf) w.retired.push_back(*buf);
  *buf = fresh;
  *have = need;
  return DG_OK;
}

// ---------------------------------------------------------------- allocation-free scratch
//
// dg_fp8_gemm_nt_noalloc runs the dense GEMM without any allocation: the split-K
// partials and arrival counters live in this fixed array, one copy per GPU the
// library runs on (zero-filled when the code object is loaded, held until the
// process ends). Host code never passes `scratch` itself to a kernel -- on the host
// it only names the symbol -- but the device address hipGetSymbolAddress gives for
// the current device, looked up once per device. Every allocation-free call on a GPU
// shares its array: the counters are zero between calls because each kernel resets
// the ones it used, and two such calls that overlap on one GPU race.
constexpr size_t kScratchPartialBytes = size_t(32) << 20;  // fp32 partial tiles
constexpr size_t kScratchCounters = 4096;                   // per-tile arrival counters
static __device__ __align__(256) uint8_t
    scratch[kScratchPartialBytes + kScratchCounters * sizeof(uint32_t)];

thread_local bool g_noalloc = false;  // set for the duration of an allocation-free call
std::mutex g_scratch_mu;
std::map<int, uint8_t*> g_scratch_ptr;  // device -> device address of its `scratch`

struct NoAllocCall {
  NoAllocCall() { g_noalloc = true; }
  ~NoAllocCall() { g_noalloc = false; }
};

dg_status scratch_workspace(size_t partial_bytes, size_t counters, float** partials,
                            uint32_t** counter_ptr) {
  if (partial_bytes > kScratchPartialBytes || counters > kScratchCounters)
    return fail(DG_ERR_UNSUPPORTED_SHAPE,
                "this shape needs %zu bytes of split-K partials and %zu counters; the "
                "allocation-free call holds at most %zu bytes and %zu counters",
                partial_bytes, counters, kScratchPartialBytes, kScratchCounters);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    uint8_t* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DG_ERR_LAUNCH, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *partials = (float*)it->second;
  *counter_ptr = (uint32_t*)(it->second + kScratchPartialBytes);
  return DG_OK;
}

dg_status get_workspace(hipStream_t stream, size_t partial_bytes, size_t counters,
                        float** partials, uint32_t** counter_ptr) {
  if (g_noalloc) return scratch_workspace(partial_bytes, counters, partials, counter_ptr);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& w = g_ws[std::make_pair(dev, stream)];
  dg_status st = grow(w, &w.partials, &w.partial_bytes, partial_bytes, 1, stream, false);
  if (st != DG_OK) return st;
  st = grow(w, (void**)&w.counters, &w.counter_count, counters, sizeof(uint32_t), stream, true);
  if (st != DG_OK) return st;
  *partials = (float*)w.partials;
  *counter_ptr = w.counters;
  return DG_OK;
}

// The per-(device, stream) buffers for K-contiguous copies of A (a_bytes) and B.
dg_status get_transpose_workspace(hipStream_t stream, size_t a_bytes, size_t b_bytes,
                                  uint8_t** a, uint8_t** b) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace& w = g_ws[std::make_pair(dev, stream)];
  dg_status st = grow(w, &w.a_t, &w.a_t_bytes, a_bytes, 1, stream, false);
  if (st != DG_OK) return st;
  st = grow(w, &w.b_t, &w.b_t_bytes, b_bytes, 1, stream, false);
  if (st != DG_OK) return st;
  *a = (uint8_t*)w.a_t;
  *b = (uint8_t*)w.b_t;
  return DG_OK;
}

// dst [C][R] = src [R][C]^T (bytes), R a multiple of 128.
dg_status launch_transpose(const uint8_t* src, uint8_t* dst, int64_t R, int64_t C,
                           hipStream_t stream) {
  const int64_t tiles_c = (C + kTrTile - 1) / kTrTile, tiles = (R / kTrTile) * tiles_c;
  if (tiles > 0x7FFFFFFF) return fail(DG_ERR_UNSUPPORTED_SHAPE, "transpose of %lld tiles", (long long)tiles);
  hipLaunchKernelGGL(transpose_bytes_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, src, dst,
                     R, C, tiles_c);
  const hipError_t err = hipGetLastError();
  return err == hipSuccess ? DG_OK : fail(DG_ERR_LAUNCH, "transpose: %s", hipGetErrorString(err));
}

// Most column tiles one XCD holds when groups of G consecutive tiles go to the XCDs
// round robin (group q on XCD q % 8; the last group may be short); the kernel gives an
// XCD's tiles the slots 0, 1, ... in group order. G = 1: ceil(tiles / 8).
int64_t tiles_per_xcd(int64_t tiles, int G) {
  int64_t most = 0;
  for (int64_t x = 0; x < 8; ++x) {
    int64_t n = 0;
    for (int64_t q = x; q * G < tiles; q += 8) n += tiles - q * G < G ? tiles - q * G : G;
    most = n > most ? n : most;
  }
  return most;
}

// LAY with kLayBN (B stored [K][N]): column tiles go to the XCDs in groups of 4 or 2
// consecutive ones (the kernel's mapping explains why), the largest group that leaves
// the most tiles per XCD, and so the split, as they are with single tiles.
// B stored [K][N] on the M <= 64 kernels: a 64-column tile's k-row piece is half a
// 128-byte line shared with a neighbouring tile, so column tiles go to the XCDs in
// groups of consecutive ones: the largest group of 4 or 2 that leaves the most tiles
// per XCD as with single tiles (so the split is unchanged), else 1.
int tile_group(int64_t tiles) {
  const int64_t one = tiles_per_xcd(tiles, 1);
  for (int G : {4, 2})
    if (tiles_per_xcd(tiles, G) == one) return G;
  return 1;
}

template <class Cfg, int LAY = 0>
dg_status launch_skinny(const Problem& p0, int64_t blocks, hipStream_t stream) {
  (void)blocks;
  if (LAY != 0 && p0.sfa_packed) return fail(DG_ERR_UNSUPPORTED_SHAPE, "packed sfA with MN-contiguous operands");
  constexpr int lds_bytes = (LAY & kLayBN) ? Cfg::LDS_BYTES_BN : Cfg::LDS_BYTES;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute((const void*)skinny_kernel<Cfg, false, LAY>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (attr_err == hipSuccess && LAY == 0)
      attr_err = hipFuncSetAttribute((const void*)skinny_kernel<Cfg, true>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  });
  if (attr_err != hipSuccess)
    return fail(DG_ERR_LAUNCH, "hipFuncSetAttribute: %s", hipGetErrorString(attr_err));
  SkinnyArgs a{};
  a.p = p0;
  const int KB = (int)(p0.K / kKBlock);
  const int64_t tiles = (p0.N + Cfg::BN - 1) / Cfg::BN;
  // K splits: as many as keep the grid within one workgroup per CU (a grid slightly
  // above the CU count would double up a few CUs and stretch the tail), at most SMAX
  // and at most one per K-block; then evened out so that no split is empty.
  int64_t S = kCUs / tiles;
  if (S > Cfg::SMAX) S = Cfg::SMAX;
  if (S > KB) S = KB;
  if (S < 1) S = 1;
  const int KS = (int)((KB + S - 1) / S);
  S = (KB + KS - 1) / KS;
  a.S = (int32_t)S;
  a.KS = KS;
  a.p.tiles_m = 1;
  a.p.tiles_n = (int32_t)tiles;
  a.tiles = (int32_t)tiles;
  // B stored [K][N]: workgroups are dealt to the XCDs (workgroup b on XCD b % 8), so the
  // grid covers every XCD's most tiles; the kernel leaves idle slots at once
  a.group = (LAY & kLayBN) ? tile_group(tiles) : 1;
  const int64_t grid = (LAY & kLayBN) ? 8 * tiles_per_xcd(tiles, 1) * S : tiles * S;
  if (grid > 0x7FFFFFFF) return fail(DG_ERR_UNSUPPORTED_SHAPE, "grid of %lld", (long long)grid);
  if (S > 1) {
    const size_t part = (size_t)(tiles * S) * 64 * Cfg::BN * sizeof(float);
    dg_status st = get_workspace(stream, part, (size_t)tiles, &a.ws, &a.counters);
    if (st != DG_OK) return st;
  }
  if (LAY != 0)
    hipLaunchKernelGGL((skinny_kernel<Cfg, false, LAY>), dim3((unsigned)grid), dim3(Cfg::NT),
                       lds_bytes, stream, a);
  else if (p0.sfa_packed)
    hipLaunchKernelGGL((skinny_kernel<Cfg, true>), dim3((unsigned)grid), dim3(Cfg::NT),
                       lds_bytes, stream, a);
  else
    hipLaunchKernelGGL((skinny_kernel<Cfg, false>), dim3((unsigned)grid), dim3(Cfg::NT),
                       lds_bytes, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(DG_ERR_LAUNCH, "launch: %s", hipGetErrorString(err));
  return DG_OK;
}

// ---------------------------------------------------------------- stream kernel

// Split choice of the stream kernel: all splits of a column tile share an XCD, so an
// XCD holds ceil(tiles / 8) tiles times S splits and should not exceed its 32 CUs.
struct StreamPlan {
  int64_t tiles, S, KS, grid, group;
};

template <class Cfg, int LAY = 0>
StreamPlan stream_plan(int64_t N, int64_t K) {
  StreamPlan pl;
  const int64_t KB = K / kKBlock;
  pl.tiles = (N + Cfg::BN - 1) / Cfg::BN;
  const int64_t per_xcd = tiles_per_xcd(pl.tiles, 1);
  pl.group = (LAY & kLayBN) ? tile_group(pl.tiles) : 1;
  int64_t S = (kCUs / 8) / per_xcd;
  if (S > Cfg::SMAX) S = Cfg::SMAX;
  if (S > KB) S = KB;
  if (S < 1) S = 1;
  pl.KS = (KB + S - 1) / S;
  pl.S = (KB + pl.KS - 1) / pl.KS;
  pl.grid = 8 * per_xcd * pl.S;
  return pl;
}

template <class Cfg>
bool stream_fits(int64_t M, int64_t N, int64_t K) {
  if (M > 64 || K / kKBlock < 1) return false;
  return stream_plan<Cfg>(N, K).KS <= Cfg::D;
}

template <class Cfg, int LAY = 0>
dg_status launch_stream(const Problem& p0, int64_t blocks, hipStream_t stream) {
  (void)blocks;
  if (LAY != 0 && p0.sfa_packed) return fail(DG_ERR_UNSUPPORTED_SHAPE, "packed sfA with MN-contiguous operands");
  const StreamPlan pl = stream_plan<Cfg, LAY>(p0.N, p0.K);
  if (pl.KS > Cfg::D) return fail(DG_ERR_UNSUPPORTED_SHAPE, "K run %lld > %d", (long long)pl.KS, Cfg::D);
  StreamArgs a{};
  a.p = p0;
  a.S = (int32_t)pl.S;
  a.KS = (int32_t)pl.KS;
  a.tiles = (int32_t)pl.tiles;
  a.group = (int32_t)pl.group;
  if (pl.grid > 0x7FFFFFFF) return fail(DG_ERR_UNSUPPORTED_SHAPE, "grid of %lld", (long long)pl.grid);
  if (pl.S > 1) {
    const size_t part = (size_t)(pl.tiles * pl.S) * 64 * Cfg::BN * sizeof(float);
    dg_status st = get_workspace(stream, part, (size_t)pl.tiles, &a.ws, &a.counters);
    if (st != DG_OK) return st;
  }
  if (LAY != 0)
    hipLaunchKernelGGL((stream_kernel<Cfg, false, LAY>), dim3((unsigned)pl.grid), dim3(Cfg::NT), 0, stream, a);
  else if (p0.sfa_packed)
    hipLaunchKernelGGL((stream_kernel<Cfg, true>), dim3((unsigned)pl.grid), dim3(Cfg::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((stream_kernel<Cfg, false>), dim3((unsigned)pl.grid), dim3(Cfg::NT), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(DG_ERR_LAUNCH, "launch: %s", hipGetErrorString(err));
  return DG_OK;
}

using Stream1x10 = StreamCfg<4, 1, 10>;
using Stream2x4 = StreamCfg<4, 2, 4>;
using Stream1x4 = StreamCfg<4, 1, 4>;
using Stream8w10 = StreamCfg<8, 1, 10>;
using Stream8w4 = StreamCfg<8, 1, 4>;
using Stream2w4 = StreamCfg<2, 1, 4>;

typedef dg_status (*Launcher)(const Problem&, int64_t, hipStream_t);
typedef bool (*Fits)(int64_t M, int64_t N, int64_t K);

struct CfgEntry {
  const char* name;
  Launcher dense, contiguous, masked;  // NULL where the configuration does not apply
  int max_m;                            // skinny: rows it covers; 0 = any
  int max_kb;                           // K/128 it supports; 0 = any
  Fits fits;                            // further shape test (dense); NULL = none
};

// The pipelined kernel addresses a tile's rows with 32-bit offsets below 256 * K
// bytes; this bound keeps them under 2^31.
constexpr int kPipeMaxKB = (1 << 22) / kKBlock;

const CfgEntry kTable[] = {
    {"tile128x128_w2x2", launch_tile<Cfg128, kDense>, launch_tile<Cfg128, kContiguous>,
     launch_tile<Cfg128, kMasked>, 0, 0},
    {"tile64x64_w2x2", launch_tile<Cfg64, kDense>, launch_tile<Cfg64, kContiguous>,
     launch_tile<Cfg64, kMasked>, 0, 0},
    {"pipe256x128", launch_pipe<Pipe256x128, kDense>, launch_pipe<Pipe256x128, kContiguous>,
     launch_pipe<Pipe256x128, kMasked>, 0, kPipeMaxKB},
    {"pipe128x256", launch_pipe128<kDense>, launch_pipe128<kContiguous>,
     launch_pipe128<kMasked>, 0, kPipeMaxKB},
    {"skinny_w4_tn1_d3", launch_skinny<SkinnyCfg<4, 1, 3>>, nullptr, nullptr, 64, 0},
    {"skinny_w4_tn1_d2", launch_skinny<SkinnyCfg<4, 1, 2>>, nullptr, nullptr, 64, 0},
    {"skinny_w4_tn1_d5", launch_skinny<SkinnyCfg<4, 1, 5>>, nullptr, nullptr, 64, 0},
    {"skinny_w4_tn1_d8", launch_skinny<SkinnyCfg<4, 1, 8>>, nullptr, nullptr, 64, 0},
    {"skinny_w2_tn1_d3", launch_skinny<SkinnyCfg<2, 1, 3>>, nullptr, nullptr, 64, 0},
    {"skinny_w2_tn1_d5", launch_skinny<SkinnyCfg<2, 1, 5>>, nullptr, nullptr, 64, 0},
    {"skinny_w2_tn1_d8", launch_skinny<SkinnyCfg<2, 1, 8>>, nullptr, nullptr, 64, 0},
    {"skinny_w8_tn1_d4", launch_skinny<SkinnyCfg<8, 1, 4>>, nullptr, nullptr, 64, 0},
    {"skinny_w8_tn1_d2", launch_skinny<SkinnyCfg<8, 1, 2>>, nullptr, nullptr, 64, 0},
    {"skinny_w2_tn1_d2", launch_skinny<SkinnyCfg<2, 1, 2>>, nullptr, nullptr, 64, 0},
    {"stream_w4_tn1_d10", launch_stream<Stream1x10>, nullptr, nullptr, 64, 0,
     stream_fits<Stream1x10>},
    {"stream_w4_tn2_d4", launch_stream<Stream2x4>, nullptr, nullptr, 64, 0,
     stream_fits<Stream2x4>},
    {"stream_w4_tn1_d4", launch_stream<Stream1x4>, nullptr, nullptr, 64, 0,
     stream_fits<Stream1x4>},
    {"stream_w8_tn1_d10", launch_stream<Stream8w10>, nullptr, nullptr, 64, 0,
     stream_fits<Stream8w10>},
    {"stream_w8_tn1_d4", launch_stream<Stream8w4>, nullptr, nullptr, 64, 0,
     stream_fits<Stream8w4>},
    {"stream_w2_tn1_d4", launch_stream<Stream2w4>, nullptr, nullptr, 64, 0,
     stream_fits<Stream2w4>},
};
constexpr int kNumCfg = (int)(sizeof(kTable) / sizeof(kTable[0]));

int find_cfg(const char* name) {
  for (int i = 0; i < kNumCfg; ++i)
    if (strcmp(kTable[i].name, name) == 0) return i;
  return -1;
}

Launcher launcher_for(int id, int kind) {
  const CfgEntry& c = kTable[id];
  return kind == kDense ? c.dense : kind == kContiguous ? c.contiguous : c.masked;
}

bool cfg_applies(int id, int kind, int64_t M, int64_t N, int64_t K) {
  const CfgEntry& c = kTable[id];
  if (!launcher_for(id, kind)) return false;
  if (c.max_m && M > c.max_m) return false;
  if (c.max_kb && K / kKBlock > c.max_kb) return false;
  if (c.fits && !c.fits(M, N, K)) return false;
  return true;
}

// Shape key -> configuration. m: rows that matter for tiling (dense M, contiguous
// rows per expert, masked expected_m); M: rows the kernel must cover.
int select_config(int kind, int64_t m, int64_t M, int64_t n, int64_t k, int32_t g) {
  (void)g;
  const char* forced = getenv("DG_FORCE_CONFIG");
  if (forced && *forced) {
    const int id = find_cfg(forced);
    if (id >= 0 && cfg_applies(id, kind, M, n, k)) return id;
  }
  if (kind == kDense && M <= 64) {
    // long K: the stream kernel (every load of a K run issued at once, split-K
    // reduction) when its run fits; short K: the rolling skinny kernel (measured
    // faster when each workgroup holds only a few K-blocks)
    const int s1 = find_cfg("stream_w4_tn1_d10");
    if (k / kKBlock >= 16 && cfg_applies(s1, kind, M, n, k)) return s1;
    // otherwise the rolling skinny kernel; its split choice for 64-column tiles decides the pipeline depth:
    // long K runs per workgroup keep 8 blocks in flight, short ones 2
    const int64_t kb = k / kKBlock, tiles = (n + 63) / 64;
    int64_t s = kCUs / tiles;
    s = s > 8 ? 8 : (s < 1 ? 1 : s);
    if (s > kb) s = kb;
    const int64_t run = (kb + s - 1) / s;
    return find_cfg(run >= 6 ? "skinny_w4_tn1_d8" : "skinny_w4_tn1_d2");
  }
  if (k / kKBlock > kPipeMaxKB) return find_cfg("tile128x128_w2x2");
  // 64 < M <= 128 and fewer than 8 column tiles of 256: 256x128 tiles (the upper
  // half of each idle) give twice the workgroups, each with half the B operand
  // (measured 128x256x512: 9.3 against 12.0 us; 128x1024x4096: 18.1 against 19.2 us)
  if (kind == kDense && M <= 128 && (n + 255) / 256 < 8) return find_cfg("pipe256x128");
  return find_cfg("pipe128x256");
}

bool print_configs() {
  static const bool on = [] {
    const char* e = getenv("DG_PRINT_CONFIGS");
    return e && *e && strcmp(e, "0") != 0;
  }();
  return on;
}

// One line per distinct (call, shape): the configuration, and for the NN / TN / TT calls
// the operand layout and whether it is read in place or through a transposed copy.
void maybe_print(int kind, int64_t M, int64_t N, int64_t K, int32_t G, int id,
                 const char* note = "") {
  if (!print_configs()) return;
  static std::mutex mu;
  static std::set<std::tuple<int, int64_t, int64_t, int64_t, int32_t, std::string>> seen;
  std::lock_guard<std::mutex> lock(mu);
  if (!seen.insert(std::make_tuple(kind, M, N, K, G, std::string(note))).second) return;
  static const char* kinds[] = {"dense", "contiguous", "masked"};
  fprintf(stderr, "[dg] %s M=%lld N=%lld K=%lld G=%d -> %s%s\n", kinds[kind], (long long)M,
          (long long)N, (long long)K, G, kTable[id].name, note);
}

dg_status launch(int kind, int id, const Problem& p, int64_t blocks, hipStream_t stream) {
  Launcher l = launcher_for(id, kind);
  if (!l) return fail(DG_ERR_UNSUPPORTED_SHAPE, "configuration %s does not apply", kTable[id].name);
  return l(p, blocks, stream);
}

// ---------------------------------------------------------------- validation

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

dg_status check_common(const void* A, const void* B, const void* C, const void* sfA,
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
    case DG_ERR_CAPTURE: return "DG_ERR_CAPTURE";
  }
  return "DG_ERR_UNKNOWN";
}

const char* dg_last_error_detail(void) { return g_detail; }

#ifndef DG_BUILD_ID
#define DG_BUILD_ID "unknown"
#endif
const char* dg_build_id(void) { return DG_BUILD_ID; }

dg_status dg_release_workspaces(void) {
  g_detail[0] = 0;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(DG_ERR_NO_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  std::set<int> devs;
  for (auto& kv : g_ws) devs.insert(kv.first.first);
  // nothing may still run on the buffers: wait for every device that holds some
  for (int d : devs) {
    if ((e = hipSetDevice(d)) != hipSuccess || (e = hipDeviceSynchronize()) != hipSuccess) {
      (void)hipSetDevice(cur);
      return fail(DG_ERR_LAUNCH, "synchronizing device %d: %s", d, hipGetErrorString(e));
    }
  }
  for (auto& kv : g_ws) {
    Workspace& w = kv.second;
    (void)hipSetDevice(kv.first.first);
    for (void* p : {w.partials, (void*)w.counters, w.a_t, w.b_t})
      if (p) (void)hipFree(p);
    for (void* p : w.retired) (void)hipFree(p);
  }
  g_ws.clear();
  (void)hipSetDevice(cur);
  return DG_OK;
}

}  // extern "C"

namespace dg {
namespace {

// The three GEMM forms with sfA as raw bytes: fp32 values, or packed UE8M0 words.
dg_status gemm_dense(const void* A, const void* B, void* C, const void* sfA, int packed,
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
  p.sfA = (const uint8_t*)sfA;
  p.sfa_packed = packed;
  p.sfB = sfB;
  p.M = M;
  p.N = N;
  p.K = K;
  p.G = 1;
  const int id = select_config(kDense, M, M, N, K, 1);
  maybe_print(kDense, M, N, K, 1, id);
  return launch(kDense, id, p, 1, (hipStream_t)stream);
}

dg_status gemm_contiguous(const void* A, const void* B, void* C, const void* sfA, int packed,
                          const float* sfB, const int32_t* m_indices, int64_t M_total,
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
  p.sfA = (const uint8_t*)sfA;
  p.sfa_packed = packed;
  p.sfB = sfB;
  p.m_indices = m_indices;
  p.M = M_total;
  p.N = N;
  p.K = K;
  p.G = G;
  const int id = select_config(kContiguous, M_total / G, M_total, N, K, G);
  maybe_print(kContiguous, M_total, N, K, G, id);
  return launch(kContiguous, id, p, 1, (hipStream_t)stream);
}

dg_status gemm_masked(const void* A, const void* B, void* C, const void* sfA, int packed,
                      const float* sfB, const int32_t* masked_m, int32_t G, int64_t M_max,
                      int64_t N, int64_t K, int64_t expected_m, void* stream) {
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
  p.sfA = (const uint8_t*)sfA;
  p.sfa_packed = packed;
  p.sfB = sfB;
  p.masked_m = masked_m;
  p.M = M_max;
  p.N = N;
  p.K = K;
  p.G = G;
  const int64_t em = expected_m > 0 && expected_m < M_max ? expected_m : M_max;
  const int id = select_config(kMasked, em, M_max, N, K, G);
  maybe_print(kMasked, M_max, N, K, G, id);
  return launch(kMasked, id, p, G, (hipStream_t)stream);
}

}  // namespace
}  // namespace dg

extern "C" {

dg_status dg_fp8_gemm_nt(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_dense(A, B, C, sfA, 0, sfB, M, N, K, stream);
}

dg_status dg_fp8_gemm_nt_noalloc(const void* A, const void* B, void* C, const float* sfA,
                                 const float* sfB, int64_t M, int64_t N, int64_t K,
                                 void* stream) {
  NoAllocCall scope;
  return gemm_dense(A, B, C, sfA, 0, sfB, M, N, K, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* A, const void* B, void* C,
                                              const float* sfA, const float* sfB,
                                              const int32_t* m_indices, int64_t M_total,
                                              int64_t N, int64_t K, int32_t G, void* stream) {
  return gemm_contiguous(A, B, C, sfA, 0, sfB, m_indices, M_total, N, K, G, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* A, const void* B, void* C,
                                          const float* sfA, const float* sfB,
                                          const int32_t* masked_m, int32_t G, int64_t M_max,
                                          int64_t N, int64_t K, int64_t expected_m,
                                          void* stream) {
  return gemm_masked(A, B, C, sfA, 0, sfB, masked_m, G, M_max, N, K, expected_m, stream);
}

dg_status dg_fp8_gemm_nt_ue8m0(const void* A, const void* B, void* C, const uint32_t* sfA,
                               const float* sfB, int64_t M, int64_t N, int64_t K,
                               void* stream) {
  return gemm_dense(A, B, C, sfA, 1, sfB, M, N, K, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* A, const void* B, void* C,
                                                    const uint32_t* sfA, const float* sfB,
                                                    const int32_t* m_indices, int64_t M_total,
                                                    int64_t N, int64_t K, int32_t G,
                                                    void* stream) {
  return gemm_contiguous(A, B, C, sfA, 1, sfB, m_indices, M_total, N, K, G, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* A, const void* B, void* C,
                                                const uint32_t* sfA, const float* sfB,
                                                const int32_t* masked_m, int32_t G,
                                                int64_t M_max, int64_t N, int64_t K,
                                                int64_t expected_m, void* stream) {
  return gemm_masked(A, B, C, sfA, 1, sfB, masked_m, G, M_max, N, K, expected_m, stream);
}

}  // extern "C"

namespace dg {
namespace {

dg_status check_swiglu(const void* A, const void* B, const void* codes, const float* sf,
                       const float* sfA, const float* sfB, const int32_t* idx, int64_t rows,
                       int64_t I, int64_t K, int32_t G) {
  if (rows < 0 || I < 0 || K < 0) return fail(DG_ERR_BAD_SHAPE, "negative size");
  if (G < 1) return fail(DG_ERR_BAD_SHAPE, "G=%d, need at least one expert", G);
  if (I % 128 != 0) return fail(DG_ERR_BAD_SHAPE, "I=%lld is not a multiple of 128", (long long)I);
  if (K % kKBlock != 0) return fail(DG_ERR_BAD_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
  if (rows == 0 || I == 0) return DG_OK;
  if (K == 0) return fail(DG_ERR_BAD_SHAPE, "K=0 with outputs to produce");
  if (!A || !B || !codes || !sf || !sfA || !sfB || !idx)
    return fail(DG_ERR_NULL_POINTER, "NULL operand pointer");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(codes, 16))
    return fail(DG_ERR_MISALIGNED, "A, B and codes must be 16-byte aligned");
  if (!aligned(sf, 4) || !aligned(sfA, 4) || !aligned(sfB, 4) || !aligned(idx, 4))
    return fail(DG_ERR_MISALIGNED, "scales and index arrays must be 4-byte aligned");
  if (K / kKBlock > kPipeMaxKB || (I + 256) * K >= ((int64_t)1 << 31) || rows > ((int64_t)1 << 30))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "(I + 256) * K must stay below 2^31");
  return DG_OK;
}

}  // namespace
}  // namespace dg

extern "C" {

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(const void* A, const void* B, void* codes,
                                                     float* sf, const float* sfA,
                                                     const float* sfB, const int32_t* m_indices,
                                                     int64_t M_total, int64_t I, int64_t K,
                                                     int32_t G, void* stream) {
  g_detail[0] = 0;
  dg_status s = check_swiglu(A, B, codes, sf, sfA, sfB, m_indices, M_total, I, K, G);
  if (s != DG_OK || M_total == 0 || I == 0) return s;
  Problem p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.sfA = (const uint8_t*)sfA;
  p.sfB = sfB;
  p.m_indices = m_indices;
  p.M = M_total;
  p.N = 2 * I;
  p.K = K;
  p.G = G;
  return launch_pipe_swiglu<kContiguous>(p, 1, I, (uint8_t*)codes, sf, (hipStream_t)stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked_swiglu(const void* A, const void* B, void* codes,
                                                 float* sf, const float* sfA, const float* sfB,
                                                 const int32_t* masked_m, int32_t G,
                                                 int64_t M_max, int64_t I, int64_t K,
                                                 void* stream) {
  g_detail[0] = 0;
  dg_status s = check_swiglu(A, B, codes, sf, sfA, sfB, masked_m, M_max, I, K, G);
  if (s != DG_OK || M_max == 0 || I == 0) return s;
  if ((int64_t)G * M_max > (int64_t)1 << 34) return fail(DG_ERR_UNSUPPORTED_SHAPE, "G*M_max too large");
  Problem p{};
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.sfA = (const uint8_t*)sfA;
  p.sfB = sfB;
  p.masked_m = masked_m;
  p.M = M_max;
  p.N = 2 * I;
  p.K = K;
  p.G = G;
  return launch_pipe_swiglu<kMasked>(p, G, I, (uint8_t*)codes, sf, (hipStream_t)stream);
}

}  // extern "C"

namespace dg {
namespace {

// C = op(A) op(B) with A stored [K][M] (a_t) and/or B stored [K][N] (b_n). The
// compute-bound kernel and the M <= 64 kernels read such operands in place: their tiles
// are staged as k-rows and transposed on the way from LDS into the MFMA (kLayAT /
// kLayBN). The tiled kernel past the compute-bound kernel's K range, and A stored
// [K][M] with M % 16 != 0, take the other route: the operand is first transposed into
// the stream's workspace and the NT kernels run on the copy.
template <int LAY>
dg_status launch_layout(int id, const Problem& p, hipStream_t st) {
  const char* name = kTable[id].name;
  if (strcmp(name, "stream_w4_tn1_d10") == 0) return launch_stream<Stream1x10, LAY>(p, 1, st);
  if (strcmp(name, "stream_w4_tn1_d4") == 0) return launch_stream<Stream1x4, LAY>(p, 1, st);
  if (strcmp(name, "skinny_w4_tn1_d2") == 0) return launch_skinny<SkinnyCfg<4, 1, 2>, LAY>(p, 1, st);
  if (strcmp(name, "skinny_w4_tn1_d3") == 0) return launch_skinny<SkinnyCfg<4, 1, 3>, LAY>(p, 1, st);
  if (strcmp(name, "skinny_w4_tn1_d5") == 0) return launch_skinny<SkinnyCfg<4, 1, 5>, LAY>(p, 1, st);
  if (strcmp(name, "skinny_w4_tn1_d8") == 0) return launch_skinny<SkinnyCfg<4, 1, 8>, LAY>(p, 1, st);
  if (strcmp(name, "pipe256x128") == 0) return launch_pipe<Pipe256x128, kDense, LAY>(p, 1, st);
  return launch_pipe128<kDense, LAY>(p, 1, st);
}

// The configuration reads MN-contiguous operands in place: the compute-bound kernels
// and the 64-column, 4-wave M <= 64 kernels.
bool layout_in_place(int id) {
  const char* name = kTable[id].name;
  return strncmp(name, "pipe", 4) == 0 || strncmp(name, "stream_w4_tn1_", 14) == 0 ||
         strncmp(name, "skinny_w4_tn1_", 14) == 0;
}

dg_status gemm_layout(const void* A, const void* B, void* C, const float* sfA,
                      const float* sfB, int64_t M, int64_t N, int64_t K, bool a_t, bool b_n,
                      void* stream) {
  g_detail[0] = 0;
  if (M < 0) return fail(DG_ERR_BAD_SHAPE, "negative M=%lld", (long long)M);
  dg_status s = check_common(A, B, C, sfA, sfB, N, K, M > 0 && N > 0);
  if (s != DG_OK || M == 0 || N == 0) return s;
  if (M > (int64_t)1 << 30) return fail(DG_ERR_UNSUPPORTED_SHAPE, "M beyond 2^30");
  const hipStream_t st = (hipStream_t)stream;
  // the NT call's configuration: every M <= 64 kernel it picks reads these layouts in
  // place too (64x32768x512 NN on the rolling kernel: 9.5 us, against 12.9 us on the
  // 128x256-tile kernel and 16.5 us through a copy)
  const int id = select_config(kDense, M, M, N, K, 1);
  // in place: 32-bit buffer offsets reach every byte of an MN-contiguous operand (the
  // compute-bound kernel addresses all of K from one base, the stream kernel at most
  // 10 K-blocks, the rolling kernel uses 64-bit addresses), and its k-rows start
  // 16-byte aligned (N % 16 == 0 always; M % 16 for A stored [K][M])
  const char* name = kTable[id].name;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t kreach = strncmp(name, "pipe", 4) == 0 ? K
                         : strncmp(name, "stream", 6) == 0 ? 10 * kKBlock : 0;
  if (layout_in_place(id) && (!a_t || (kreach * M < lim && M % 16 == 0)) &&
      (!b_n || kreach * N < lim)) {
    maybe_print(kDense, M, N, K, 1, id, a_t ? (b_n ? " (TN, in place)" : " (TT, in place)")
                                             : " (NN, in place)");
    Problem p{};
    p.A = (const uint8_t*)A;
    p.B = (const uint8_t*)B;
    p.C = (uint16_t*)C;
    p.sfA = (const uint8_t*)sfA;
    p.sfB = sfB;
    p.M = M;
    p.N = N;
    p.K = K;
    p.G = 1;
    const int lay = (a_t ? kLayAT : 0) | (b_n ? kLayBN : 0);
    return lay == kLayBN ? launch_layout<kLayBN>(id, p, st)
         : lay == kLayAT ? launch_layout<kLayAT>(id, p, st)
                         : launch_layout<kLayAT | kLayBN>(id, p, st);
  }
  maybe_print(kDense, M, N, K, 1, id, a_t ? (b_n ? " (TN, transposed copy)" : " (TT, transposed copy)")
                                           : " (NN, transposed copy)");
  uint8_t *a2 = nullptr, *b2 = nullptr;
  s = get_transpose_workspace(st, a_t ? (size_t)(M * K) : 0, b_n ? (size_t)(N * K) : 0, &a2, &b2);
  if (s != DG_OK) return s;
  if (a_t && (s = launch_transpose((const uint8_t*)A, a2, K, M, st)) != DG_OK) return s;
  if (b_n && (s = launch_transpose((const uint8_t*)B, b2, K, N, st)) != DG_OK) return s;
  return gemm_dense(a_t ? (const void*)a2 : A, b_n ? (const void*)b2 : B, C, sfA, 0, sfB, M, N, K,
                    stream);
}

}  // namespace
}  // namespace dg

extern "C" {

dg_status dg_fp8_gemm_nn(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_layout(A, B, C, sfA, sfB, M, N, K, false, true, stream);
}

dg_status dg_fp8_gemm_tn(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_layout(A, B, C, sfA, sfB, M, N, K, true, true, stream);
}

dg_status dg_fp8_gemm_tt(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* stream) {
  return gemm_layout(A, B, C, sfA, sfB, M, N, K, true, false, stream);
}

dg_status dg_quantize_fp8_1x128(const void* x, int32_t x_dtype, void* codes, float* sf,
                                int64_t M, int64_t K, void* stream) {
  g_detail[0] = 0;
  if (x_dtype != DG_DTYPE_F32 && x_dtype != DG_DTYPE_BF16)
    return fail(DG_ERR_BAD_SHAPE, "x_dtype=%d is neither DG_DTYPE_F32 nor DG_DTYPE_BF16", x_dtype);
  if (M < 0 || K < 0)
    return fail(DG_ERR_BAD_SHAPE, "negative size (M=%lld, K=%lld)", (long long)M, (long long)K);
  if (K % kKBlock != 0) return fail(DG_ERR_BAD_SHAPE, "K=%lld is not a multiple of 128", (long long)K);
  if (M == 0 || K == 0) return DG_OK;
  if (!x || !codes || !sf) return fail(DG_ERR_NULL_POINTER, "NULL x, codes or sf");
  if (!aligned(x, 16) || !aligned(codes, 16))
    return fail(DG_ERR_MISALIGNED, "x and codes must be 16-byte aligned");
  if (!aligned(sf, 4)) return fail(DG_ERR_MISALIGNED, "sf must be 4-byte aligned");
  if (M > ((int64_t)1 << 40) / K) return fail(DG_ERR_UNSUPPORTED_SHAPE, "M*K beyond 2^40");
  const int64_t nblocks = M * (K / kKBlock);
  const int64_t per_wg = (int64_t)(kQuantThreads / 64) * kQuantBlocksPerWave * kQuantUnroll;
  int64_t grid = (nblocks + per_wg - 1) / per_wg;
  if (grid > 8 * kCUs) grid = 8 * kCUs;  // grid-stride beyond eight workgroups per CU
  if (x_dtype == DG_DTYPE_BF16)
    hipLaunchKernelGGL(quant_kernel<true>, dim3((unsigned)grid), dim3(kQuantThreads), 0,
                       (hipStream_t)stream, x, (uint8_t*)codes, sf, nblocks);
  else
    hipLaunchKernelGGL(quant_kernel<false>, dim3((unsigned)grid), dim3(kQuantThreads), 0,
                       (hipStream_t)stream, x, (uint8_t*)codes, sf, nblocks);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(DG_ERR_LAUNCH, "quant_kernel: %s", hipGetErrorString(err));
  return DG_OK;
}

int32_t dg_num_configs(void) { return kNumCfg; }

const char* dg_config_name(int32_t i) { return i >= 0 && i < kNumCfg ? kTable[i].name : nullptr; }

dg_status dg_describe_config(int32_t kind, int64_t M, int64_t N, int64_t K, int32_t G,
                             int64_t expected_m, char* buf, int64_t len) {
  if (kind < 0 || kind > 2 || !buf || len <= 0) return DG_ERR_BAD_SHAPE;
  int64_t m = M;
  if (kind == kContiguous) m = G > 0 ? M / G : M;
  if (kind == kMasked) m = expected_m > 0 && expected_m < M ? expected_m : M;
  const int id = select_config(kind, m, M, N, K, G);
  snprintf(buf, (size_t)len, "%s", kTable[id].name);
  return DG_OK;
}

}  // extern "C"

// hbm_probe.hip -- measurement companion of libdg.so (built as libdg_probe.so, loaded
// only by the benchmark), the calibrations the GEMM kernels are judged against:
//  - a plain streaming read of a byte range: it reads every 16-byte chunk of
//    [src, src + bytes) once and folds the data into one word per workgroup so that
//    the loads are not removed. Its duration for a given byte count is the achievable
//    time for that many bytes from HBM on this GPU: launch, ramp-up and the first
//    loads' latency included;
//  - the FP8 matrix instruction alone (v_mfma_f32_32x32x64_f8f6f4, the compute-bound
//    kernel's), on register operands of pseudo-random e4m3fn bytes, four independent
//    accumulator chains per wave and two waves per SIMD: the rate the matrix units
//    sustain on this chip when nothing else runs, at the clock its power limit allows
//    for random data.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane

template <bool NT>
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint8_t* src, int64_t chunks,
                                                                uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  const v4u* p = (const v4u*)src;
  // every lane issues up to kUnroll loads before it uses any (chunk indices past the
  // end are skipped), then moves kUnroll strides on
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < chunks;
       i += kUnroll * stride) {
    v4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + u * stride;
      v[u] = j < chunks ? (NT ? __builtin_nontemporal_load(p + j) : p[j]) : v4u{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per workgroup: lane 0 of wave 0 after a wave-wide fold
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ void empty_kernel() {}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// e4m3fn bytes from a counter hash (splitmix-style mixing), never the NaN code 0x7F.
__device__ __forceinline__ int rnd_codes(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (int)(x & 0xF7F7F7F7u);  // clears bit 3 of each byte's exponent: no 0x7F / 0xFF
}

__global__ void __launch_bounds__(512) mfma_rate_kernel(int iters, uint32_t seed, float* sink) {
  const uint32_t t = blockIdx.x * 512u + threadIdx.x;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = rnd_codes(seed ^ (t * 16u + i));
    b[i] = rnd_codes(seed ^ (t * 16u + 8 + i) ^ 0x9e3779b9u);
  }
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 0, 0, 0);
  }
  float x = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) x += c0[e] + c1[e] + c2[e] + c3[e];
  if (x == 1.2345f) sink[t] = x;  // keeps the chains; practically never stores
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16, src 16-byte aligned) by `blocks`
// workgroups of 256 threads, with non-temporal loads when nt != 0; sink (device)
// receives one uint32 per workgroup and must hold `blocks` of them. 0 on success,
// else the HIP error code.
int dg_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                         int32_t nt, void* stream) {
  if (!src || !sink || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15) || blocks < 1)
    return (int)hipErrorInvalidValue;
  if (nt)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (const uint8_t*)src, bytes / 16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (const uint8_t*)src, bytes / 16, sink);
  return (int)hipGetLastError();
}

// The matrix-instruction rate probe: `blocks` workgroups of 8 waves, each wave running
// 4 * iters FP8 32x32x64 MFMAs (131072 FLOP each). sink (device) must hold
// blocks * 512 floats; it is written only in the improbable case that a checksum
// hits its marker value. 0 on success, else the HIP error code.
int dg_probe_mfma_rate(int32_t iters, int32_t blocks, uint32_t seed, float* sink, void* stream) {
  if (iters < 1 || blocks < 1 || !sink) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream,
                     iters, seed, sink);
  return (int)hipGetLastError();
}

// An empty kernel: the launch and completion cost alone.
int dg_probe_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

}  // extern "C"

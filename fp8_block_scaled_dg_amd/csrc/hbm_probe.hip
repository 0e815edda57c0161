// hbm_probe.hip -- measurement companion of libdg.so (built as libdg_probe.so, loaded
// only by the benchmark): a plain streaming read of a byte range, the calibration
// against which the memory-bound GEMM kernels' HBM throughput is judged. It reads
// every 16-byte chunk of [src, src + bytes) once, with the same buffer-load path
// and the same one-workgroup-per-CU grid the decode kernels use, and folds the data
// into one word per workgroup so that the loads are not removed. Its duration for
// a given byte count is the achievable time for that many bytes from HBM on this
// GPU: launch, ramp-up and the first loads' latency included.
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

// An empty kernel: the launch and completion cost alone.
int dg_probe_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

}  // extern "C"

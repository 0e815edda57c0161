// transpose_kernel.hpp -- byte-matrix transpose for gfx950, the pre-pass of the GEMM
// calls whose operands are not K-contiguous (the NN / TN / TT memory layouts of one
// GEMM family: DeepGEMM project page, aiproducthub.cn, "core features").
//
// src [R][C] bytes (row-major) -> dst [C][R]; R is the contraction length K (a
// multiple of 128), so every destination row is a whole number of 16-byte chunks.
// A workgroup moves one 64 x 64 tile: each thread loads 16 bytes of a source row
// into a padded LDS tile, and after one barrier gathers 16 bytes of a source column
// and writes them as 16 contiguous bytes of a destination row. HBM-bound: one read
// and one write of the matrix.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dg {

constexpr int kTrTile = 64;
constexpr int kTrPitch = kTrTile + 4;  // LDS row pitch: column reads spread over banks

__global__ void __launch_bounds__(256) transpose_bytes_kernel(const uint8_t* __restrict__ src,
                                                              uint8_t* __restrict__ dst,
                                                              int64_t R, int64_t C,
                                                              int64_t tiles_c) {
  __shared__ __align__(16) uint8_t tile[kTrTile * kTrPitch];
  const int t = threadIdx.x;
  const int64_t tr = (int64_t)blockIdx.x / tiles_c, tc = (int64_t)blockIdx.x - tr * tiles_c;
  const int64_t r0 = tr * kTrTile, c0 = tc * kTrTile;
  {
    const int lr = t >> 2, lc = (t & 3) * 16;
    const int64_t r = r0 + lr, c = c0 + lc;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (r < R) {
      if ((C & 15) == 0 && c + 16 <= C) {
        const uint4 v = *(const uint4*)(src + r * C + c);
        w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (c + i < C) w[i >> 2] |= (uint32_t)src[r * C + c + i] << (8 * (i & 3));
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) *(uint32_t*)(tile + lr * kTrPitch + lc + 4 * q) = w[q];
  }
  __syncthreads();
  {
    const int lc = t >> 2, lr = (t & 3) * 16;
    const int64_t c = c0 + lc, r = r0 + lr;
    if (c < C && r < R) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i >> 2] |= (uint32_t)tile[(lr + i) * kTrPitch + lc] << (8 * (i & 3));
      *(uint4*)(dst + c * R + r) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace dg

// quant_kernel.hpp -- per-token 1x128 activation quantizer for gfx950: fp32 or bf16
// values -> e4m3fn codes plus one power-of-two fp32 scale per 1x128 block, which is
// the form the GEMM takes its A operand in (fine-grained scaling with one factor
// per small block, so that every block spans the FP8 range on its own: DeepGEMM
// launch article, deepseek.csdn.net, section 1.2 "precision safeguards").
//
// Per block of 128 consecutive values x (one row, one 128-wide K-block):
//   amax = max |x|;  e = the least integer with amax <= 448 * 2^e (e = 0 when
//   amax = 0);  scale = 2^e;  code = the e4m3fn value nearest to x / 2^e, ties to
//   the even code, a zero keeping the sign of x.
// Both steps are exact functions of the input bits (no rounded logarithm, no
// rounded division), so any implementation of the rule gives the same bytes.
//
// Memory-bound: one read of x, one write of codes and scales, both streamed with
// non-temporal accesses (nothing is reused). Blocks tile the row-major [M][K] array
// as consecutive runs of 128 values, so block b is values [128b, 128b + 128) and its
// scale is sf[b]. Eight lanes own a block (16 values and one 16-byte code store
// each) and a wave covers 8 consecutive blocks (1024 values) per pass, so its loads
// and stores are contiguous; each lane issues the loads of two passes before it
// converts either. The codes come from the packed hardware conversion, two values
// per instruction; the bit-level rounding it replaces cost about 10% of the time on
// bf16 [4096][18432] (2 bytes read and 1 written per value: 229 MB in about 42 us).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dg {

// e4m3fn codes nearest to a, b, c, d (|y| <= 448) in bytes 0..3, ties to the even
// code, the sign of a zero kept. Below 2^-6 the e4m3fn values are the multiples of
// 2^-9 (subnormals); in a binade [2^E, 2^(E+1)), E >= -6, their spacing is 2^(E-3).
// gfx950's v_cvt_pk_fp8_f32 converts two fp32 values to OCP e4m3fn with exactly this
// rounding (checked against the bit-level rule on every code, both neighbours of
// every code and every midpoint between codes, and two million random values).
__device__ __forceinline__ uint32_t quant_e4m3fn_x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// The least e with amax <= 448 * 2^e (0 when amax = 0). With amax = f * 2^x,
// f in [0.5, 1): 448 * 2^e = 0.875 * 2^(e + 9), so e = x - 9 when f <= 0.875 and
// x - 8 otherwise.
__device__ __forceinline__ int quant_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int x;
  const float f = frexpf(amax, &x);
  return x - 9 + (f > 0.875f ? 1 : 0);
}

typedef unsigned quant_v4u __attribute__((ext_vector_type(4)));

// 16 consecutive values starting at element idx, as fp32 (bf16 widens exactly).
template <bool BF16>
__device__ __forceinline__ void quant_load16(const void* src, int64_t idx, float (&v)[16]) {
  constexpr int Q = BF16 ? 2 : 4;  // 16-byte loads
  const quant_v4u* p = BF16 ? (const quant_v4u*)((const uint16_t*)src + idx)
                            : (const quant_v4u*)((const float*)src + idx);
  quant_v4u w[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) w[q] = __builtin_nontemporal_load(p + q);
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (BF16) {
        v[8 * q + 2 * j] = __uint_as_float(w[q][j] << 16);
        v[8 * q + 2 * j + 1] = __uint_as_float(w[q][j] & 0xFFFF0000u);
      } else {
        v[4 * q + j] = __uint_as_float(w[q][j]);
      }
    }
}

constexpr int kQuantThreads = 256;  // 4 waves
constexpr int kQuantLanes = 8;      // lanes per 1x128 block (16 values each)
constexpr int kQuantUnroll = 2;     // passes whose loads are in flight together
constexpr int kQuantBlocksPerWave = 64 / kQuantLanes;

// Wave w of the grid takes the 8-block chunks w, w + W, w + 2W, ... (W waves).
template <bool BF16>
__global__ void __launch_bounds__(kQuantThreads) quant_kernel(const void* __restrict__ x,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ sf,
                                                              int64_t nblocks) {
  constexpr int U = kQuantUnroll, L = kQuantLanes, BPW = kQuantBlocksPerWave;
  const int lane = threadIdx.x & 63, grp = lane / L, li = lane % L;
  const int64_t wave = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) >> 6;
  const int64_t W = (int64_t)gridDim.x * (kQuantThreads / 64);
  const int64_t nchunks = (nblocks + BPW - 1) / BPW;
  for (int64_t c0 = wave; c0 < nchunks; c0 += W * U) {
    float v[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = (c0 + u * W) * BPW + grp;
      if (b < nblocks) {
        quant_load16<BF16>(x, b * 128 + li * 16, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[u][i] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = (c0 + u * W) * BPW + grp;
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
#pragma unroll
      for (int d = 1; d < L; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, L));
      const int e = quant_scale_exp(amax);
      if (b < nblocks) {
        quant_v4u w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = quant_e4m3fn_x4(ldexpf(v[u][4 * q], -e), ldexpf(v[u][4 * q + 1], -e),
                                 ldexpf(v[u][4 * q + 2], -e), ldexpf(v[u][4 * q + 3], -e));
        __builtin_nontemporal_store(w, (quant_v4u*)(codes + b * 128 + li * 16));
        if (li == 0) sf[b] = ldexpf(1.f, e);
      }
    }
  }
}

}  // namespace dg

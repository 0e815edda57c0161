// stream_kernel.hpp -- block-scaled FP8 GEMM for M <= 64 (decode shapes), gfx950.
//
// Memory-bound regime: every byte of B meets at most 64 rows of A, so a workgroup's
// job is to pull its share of B from HBM with as many bytes in flight as possible
// and to keep everything else off the critical path. The work unit of a workgroup
// is (BN columns) x (a run of at most D consecutive K-blocks), all 64 rows:
//   1. Issue, at once and in block order, every load of the unit: per K-block the
//      A tile (64 x 128 bytes) by LDS DMA into that block's own __shared__ array,
//      and each wave's B fragments straight into MFMA operand registers; before
//      them the sfA column block (LDS DMA) and the wave's sfB values (registers).
//   2. For block t = 0..D-1 in order: wait until this wave's loads up to block t
//      have landed (vmcnt counts the later blocks' loads, all compile-time), one
//      barrier so that every wave's DMA share of the A tile is visible, then per
//      16x16 tile one v_mfma_f32_16x16x128_f8f6f4 gives the block partial and it is
//      promoted into the fp32 accumulators with sfA[m][kb] * sfB[n/128][kb] -- the
//      two-level accumulation of the DeepGEMM launch article (deepseek.csdn.net),
//      section 1.2 "precision safeguards".
//   3. One K split: round to bf16 and store through LDS. S > 1 splits: each writes
//      its fp32 partial to a workspace, and the last to arrive (atomic counter) sums
//      the S partials in split order -- deterministic -- then rounds and stores. All
//      splits of a column tile run on one XCD (workgroup b runs on XCD b % 8).
// The MFMA takes B as its first operand, so each lane of a 16x16 result holds one
// A row (lane % 16) and four columns: one sfA value per A tile and lane. Within a
// K-block both operands use the k order lane (g, r) <- [16g, 16g+16) and
// [64+16g, 80+16g); each B load then reads 64 contiguous bytes of 16 rows.
// Loads past the unit's last K-block re-read that block (uniform wait counts); the
// compute of such blocks is skipped. Rows past M or N clamp to the last row; such
// outputs are never stored.
#pragma once

#include "gemm_kernel.hpp"

namespace dg {

template <int W_, int TN_, int D_>
struct StreamCfg {
  static constexpr int W = W_, TN = TN_, D = D_, NT = W * 64;
  static constexpr int TM = 4;                   // 64 rows = 4 A tiles of 16
  static constexpr int BN = 16 * W * TN;         // columns per workgroup
  static constexpr int A_DMA = 8 / W;            // 1 KB A DMAs per wave and block
  static constexpr int SF4 = (D + 3) / 4;        // 16-byte groups of K-blocks
  static constexpr int PRO = SF4 + TN * SF4;     // per-wave scale loads before block 0
  static constexpr int OPB = A_DMA + 2 * TN;     // per-wave loads per block
  static constexpr int SMAX = TN == 1 ? 8 : 4;   // most K splits (partials held at once)
  static_assert(8 % W == 0, "A DMA split");
  static_assert(SF4 <= 3, "sfA staging holds 12 K-blocks");
  static_assert(BN <= 128, "output staging size");
  static_assert(PRO + D * OPB < 64, "vmcnt range");
};

template <int I>
__shared__ __align__(16) uint8_t stream_a[64 * kKBlock];  // A tile of block I
__shared__ __align__(16) uint8_t stream_sfa[3 * 1024];     // sfA: [group][row][4]
__shared__ __align__(16) uint16_t stream_out[64 * 128];    // bf16 output staging

struct StreamArgs {
  Problem p;
  float* ws;           // [tiles][S][64 * BN] fp32 partials (S > 1)
  uint32_t* counters;  // [tiles], zero between calls
  int32_t S;           // K splits
  int32_t KS;          // K-blocks per split (the last split may have fewer)
  int32_t tiles;
};

template <class Cfg>
struct StreamRegs {
  v8i b[Cfg::D][Cfg::TN];
  v4f sfb[Cfg::TN][Cfg::SF4];
};

// vmcnt = n, lgkmcnt = 0
template <int n>
__device__ __forceinline__ void stream_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

template <class Cfg, int T>
__device__ __forceinline__ void stream_issue_block(StreamRegs<Cfg>& r,
                                                   __amdgpu_buffer_rsrc_t a_rsrc,
                                                   const uint32_t (&a_off)[Cfg::A_DMA],
                                                   __amdgpu_buffer_rsrc_t b_rsrc,
                                                   const uint32_t (&b_off)[Cfg::TN], int tc,
                                                   int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int koff = tc * kKBlock;
#pragma unroll
  for (int q = 0; q < Cfg::A_DMA; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        a_rsrc, (__attribute__((address_space(3))) void*)(stream_a<T> + (wave * Cfg::A_DMA + q) * 1024),
        16, a_off[q], koff, 0, 0);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_off[j], koff, 0);
    const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_off[j] + 64, koff, 0);
    r.b[T][j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
#endif
}

template <class Cfg, int T>
__device__ __forceinline__ void stream_issue_all(StreamRegs<Cfg>& r, __amdgpu_buffer_rsrc_t a_rsrc,
                                                 const uint32_t (&a_off)[Cfg::A_DMA],
                                                 __amdgpu_buffer_rsrc_t b_rsrc,
                                                 const uint32_t (&b_off)[Cfg::TN], int ks,
                                                 int wave) {
  if constexpr (T < Cfg::D) {
    stream_issue_block<Cfg, T>(r, a_rsrc, a_off, b_rsrc, b_off, T < ks ? T : ks - 1, wave);
    stream_issue_all<Cfg, T + 1>(r, a_rsrc, a_off, b_rsrc, b_off, ks, wave);
  }
}

template <class Cfg, int T, bool PACKED>
__device__ __forceinline__ void stream_compute(v4f (&acc)[Cfg::TM][Cfg::TN], const StreamRegs<Cfg>& r,
                                               int ks, int g, int l16, int shift) {
  if constexpr (T < Cfg::D) {
    // this wave's loads of blocks 0..T have landed; every wave's A DMAs of block T
    // are visible after the barrier
    stream_wait<(Cfg::D - 1 - T) * Cfg::OPB>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (T < ks) {
      constexpr int TM = Cfg::TM, TN = Cfg::TN;
      v8i af[TM];
      float sa[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = i * 16 + l16;
        const uint8_t* rowp = stream_a<T> + row * kKBlock;
        const v4u lo = *(const v4u*)(rowp + ((g ^ swz(row)) << 4));
        const v4u hi = *(const v4u*)(rowp + (((g + 4) ^ swz(row)) << 4));
        af[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sa[i] = PACKED ? ue8m0_value(stream_sfa[row * 16 + shift + T])
                       : ((const float*)(stream_sfa + (T / 4) * 1024 + row * 16))[T % 4];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              r.b[T][j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          const float s = sa[i] * r.sfb[j][T / 4][T % 4];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(part[q], s, acc[i][j][q]);
        }
    }
    stream_compute<Cfg, T + 1, PACKED>(acc, r, ks, g, l16, shift);
  }
}

// PACKED: sfA in the packed UE8M0 layout (compile-time, as in the skinny kernel).
template <class Cfg, bool PACKED>
__global__ void __launch_bounds__(Cfg::NT) stream_kernel(StreamArgs args) {
  constexpr int TN = Cfg::TN, TM = Cfg::TM, NT = Cfg::NT, BN = Cfg::BN;
  const Problem& p = args.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int KB = (int)(K / kKBlock);
  const int S = args.S;

  // workgroup -> (tile, split): tile t's splits all run on XCD t % 8
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int tile = (local / S) * 8 + xcd, split = local - (local / S) * S;
  if (tile >= args.tiles) return;
  const int64_t n0 = (int64_t)tile * BN;
  const int kb0 = split * args.KS;
  const int ks = min(args.KS, KB - kb0);  // >= 1 (host guarantees)

  // ---- sources: buffer resources over the unit's rows, 32-bit per-lane offsets
  const int a_rows = (int)(M < 64 ? M : 64);
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.A + (int64_t)kb0 * kKBlock), 0, 0x7FFFFFFF, 0x00020000);
  uint32_t a_off[Cfg::A_DMA];
#pragma unroll
  for (int q = 0; q < Cfg::A_DMA; ++q) {
    const int R = (wave * Cfg::A_DMA + q) * 8 + (lane >> 3), c = lane & 7;
    const int row = R < a_rows ? R : a_rows - 1;
    a_off[q] = (uint32_t)row * (uint32_t)K + (uint32_t)((c ^ swz(R)) << 4);
  }
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.B + n0 * K + (int64_t)kb0 * kKBlock), 0, 0x7FFFFFFF, 0x00020000);
  uint32_t b_off[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int64_t r = (wave * TN + j) * 16 + l16;
    if (n0 + r >= N) r = N - 1 - n0;
    b_off[j] = (uint32_t)r * (uint32_t)K + (uint32_t)(g * 16);
  }
  // ---- issue every load of the unit
  StreamRegs<Cfg> r;
#if defined(__HIP_DEVICE_COMPILE__)
  {
    // scale resources end at the arrays' ends: reads past the last K-block give 0
    // fp32: the run's values start at sfA + kb0; packed: at the word holding K-block
    // kb0 (byte kb0 % 4 of the staged 16 bytes). Groups past the first hold nothing
    // the packed form uses; they keep the load count the same.
    const int64_t rb = sfa_row_bytes(KB, PACKED);
    const int64_t sa0 = PACKED ? (kb0 & ~3) : (int64_t)kb0 * 4;
    const __amdgpu_buffer_rsrc_t sa_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.sfA + sa0), 0, (int)(M * rb - sa0), 0x00020000);
    const int NB = (int)((N + kKBlock - 1) / kKBlock);
    const __amdgpu_buffer_rsrc_t sb_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.sfB + kb0), 0, (int)(((int64_t)NB * KB - kb0) * 4), 0x00020000);
    const int row = lane < a_rows ? lane : a_rows - 1;
#pragma unroll
    for (int c = 0; c < Cfg::SF4; ++c)  // identical bytes from every wave
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          sa_rsrc, (__attribute__((address_space(3))) void*)(stream_sfa + c * 1024), 16,
          (uint32_t)row * (uint32_t)rb, c * 16, 0, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int nb = (int)((n0 + (wave * TN + j) * 16) / kKBlock);
      if (nb >= NB) nb = NB - 1;
#pragma unroll
      for (int c = 0; c < Cfg::SF4; ++c)
        r.sfb[j][c] = __builtin_bit_cast(
            v4f, __builtin_amdgcn_raw_buffer_load_b128(sb_rsrc, (uint32_t)nb * (uint32_t)KB * 4u,
                                                       c * 16, 0));
    }
  }
#endif
  stream_issue_all<Cfg, 0>(r, a_rsrc, a_off, b_rsrc, b_off, ks, wave);

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  stream_compute<Cfg, 0, PACKED>(acc, r, ks, g, l16, kb0 & 3);

  // ---- split reduction. Partials are written and read with device-scope (sc1)
  // 16-byte accesses (measured faster here than L2-resident ones); splitk_arrive
  // orders them around the arrival count.
  if (S > 1) {
    constexpr int SMAX = Cfg::SMAX;
    constexpr int per_split = 64 * BN * 4;
    const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
        args.ws + (int64_t)tile * S * (64 * BN), 0, 0x7FFFFFFF, 0x00020000);
    constexpr int kSc1 = 16;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(v4u, acc[i][j]), ws,
            split * per_split + (((wave * TM + i) * TN + j) * 64 + lane) * 16, 0, kSc1);
    if (!splitk_arrive(&args.counters[tile], (uint32_t)S)) return;
    // the other splits' partials (this split's is in registers)
    v4u part[SMAX][TM][TN];
#pragma unroll
    for (int sp = 0; sp < SMAX; ++sp) {
      if (sp < S && sp != split) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            part[sp][i][j] = __builtin_amdgcn_raw_buffer_load_b128(
                ws, sp * per_split + (((wave * TM + i) * TN + j) * 64 + lane) * 16, 0, kSc1);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < SMAX; ++sp) {
          if (sp < S) {
            const v4f v = sp == split ? acc[i][j] : __builtin_bit_cast(v4f, part[sp][i][j]);
            sum[0] += v[0];
            sum[1] += v[1];
            sum[2] += v[2];
            sum[3] += v[3];
          }
        }
        acc[i][j] = sum;
      }
    if (tid == 0)
      __hip_atomic_store(&args.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- bf16 through LDS, 16-byte stores. Lane (g, l16) of tile (i, j) holds row
  // 16i + l16 and columns 16*(wave*TN + j) + 4g + q.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = i * 16 + l16, col = (wave * TN + j) * 16 + 4 * g;
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[i][j][0]) |
                          ((uint32_t)f32_to_bf16_rne(acc[i][j][1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[i][j][2]) |
                          ((uint32_t)f32_to_bf16_rne(acc[i][j][3]) << 16);
      *(uint2*)(stream_out + row * BN + col) = make_uint2(lo, hi);
    }
  __syncthreads();
  constexpr int CH = 64 * BN / 8;
  for (int c = tid; c < CH; c += NT) {
    const int row = c / (BN / 8), col0 = (c - row * (BN / 8)) * 8;
    if (row < M && n0 + col0 < N)
      __builtin_nontemporal_store(*(const v4u*)(stream_out + row * BN + col0),  // C is not read again
                                  (v4u*)(p.C + (int64_t)row * N + n0 + col0));
  }
}

}  // namespace dg

// gemm_kernel.hpp -- FP8 block-scaled GEMM tile kernel for CDNA4 (gfx950).
//
// One workgroup computes one BM x BN output tile. For every 128-wide K-block kb:
//   level 1: each wave runs v_mfma_f32_16x16x128_f8f6f4 on its 16x16 sub-tiles --
//            one instruction covers the whole K-block, so its fp32 result P is
//            exactly one block partial;
//   level 2: acc += P * (sfA[m][kb] * sfB[n/128][kb]) in fp32 VGPRs.
// This is the two-level accumulation of the DeepGEMM launch article
// (deepseek.csdn.net), section 1.2 "precision safeguards": scaled FP8 blocks whose
// products are promoted to FP32 for the accumulation across blocks. On gfx950 the
// promotion is needed too: the FP8 MFMA's internal 128-term sum is narrower than
// fp32 (measured error up to ~1e-4 of sum|a*b| per instruction), so partials must
// not be chained across K-blocks inside the MFMA accumulator.
//
// Operand movement: A and B tiles of one K-block are staged in LDS, double
// buffered: the global loads of block kb+1 are issued before the MFMAs of block kb
// and written to the other LDS buffer after them, with one barrier per block (the
// pages' Hopper design uses TMA for this; here plain coalesced 16-byte loads).
// LDS rows are 128 bytes; the 16-byte chunk c of row r sits at chunk
// c ^ swz(r) so that 16 lanes reading the same logical chunk of 16 rows hit
// disjoint banks.
//
// Out-of-range rows/columns: loads clamp the row index into the matrix, so every
// address is valid; the epilogue stores only produced rows and columns < N. An
// output (m, n) depends only on A row m and B row n, so clamped rows never reach
// a stored value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kKBlock = 128;

enum Kind : int { kDense = 0, kContiguous = 1, kMasked = 2 };

// Kernel arguments (plain data, passed by value).
struct Problem {
  const uint8_t* A;
  const uint8_t* B;
  uint16_t* C;
  const uint8_t* sfA;        // rows of KB fp32 values, or (sfa_packed) of ceil(KB/4)
                             // little-endian words of UE8M0 bytes, byte kb = K-block kb
  const float* sfB;
  const int32_t* m_indices;  // contiguous only
  const int32_t* masked_m;   // masked only
  int64_t M;                 // rows: dense M, contiguous M_total, masked M_max
  int64_t N;
  int64_t K;
  int32_t G;
  int32_t tiles_m;
  int32_t tiles_n;
  int32_t sfa_packed;        // 1: sfA in the packed UE8M0 layout
};

// Bytes of one sfA row: KB fp32 values, or ceil(KB/4) words of UE8M0 bytes.
__host__ __device__ inline int64_t sfa_row_bytes(int64_t KB, int packed) {
  return packed ? (KB + 3) / 4 * 4 : KB * 4;
}

// The scale a UE8M0 byte encodes: 2^(b - 127) (b = 255, NaN in the OCP MX format,
// is not a valid scale).
__device__ __forceinline__ float ue8m0_value(uint32_t b) { return ldexpf(1.f, (int)b - 127); }

// sfA of K-block kb from a row's bytes.
__device__ __forceinline__ float sfa_at(const uint8_t* row, int kb, int packed) {
  return packed ? ue8m0_value(row[kb]) : ((const float*)row)[kb];
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Arrival of one K part of a split-K tile at the tile's counter, called by every
// thread after the part has stored its fp32 partial with device-scope (sc1) buffer
// stores; returns true in every thread of the workgroup whose part arrived last, which
// then reads the other parts' partials with device-scope loads and resets the counter.
// The ordering is the one these accesses need on gfx950:
//  - release: the compiler fence keeps the partial stores above the wait, s_waitcnt 0
//    waits until each wave's stores have completed at the device coherence point, and
//    the barrier orders all waves' completed stores before thread 0's counter update;
//  - acquire: the partials are read with device-scope loads (served by the coherence
//    point, never by a stale cache line) that issue only after the counter value has
//    been seen: the workgroup barrier and the branch on it, held in place by the
//    compiler fence.
// The memory model's generic agent-scope release and acquire would instead write back
// and invalidate the whole L2 around the update; on the 64x2112x7168 decode kernel
// those measured 13.25 us (release and acquire) and 12.30 us (acquire alone) against
// 11.82 us for this protocol, with identical outputs.
__device__ __forceinline__ bool splitk_arrive(uint32_t* counter, uint32_t parts) {
  __shared__ uint32_t s_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             parts - 1;
  __syncthreads();
  const bool last = s_last != 0;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return last;
}

// Operand memory layouts of the dense GEMM (bit set: the operand is stored with M or
// N contiguous, i.e. as [K][M] or [K][N], instead of K-contiguous rows): the other
// layouts of one GEMM family, C = op(A) op(B) with A stored [K][M] (T) and B stored
// [K][N] (N) (DeepGEMM project page, aiproducthub.cn, "core features").
constexpr int kLayAT = 1, kLayBN = 2;

typedef int v2i __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b8: in each group of 16 lanes, lanes 2j and 2j+1 address the two
// 8-byte halves of 16 consecutive bytes of row j (j = 0..7), and lane i receives
// byte i of each of those 8 rows -- an 8 x 16 byte block read transposed.
__device__ __forceinline__ v2i tr8_at(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
}

// MN-contiguous staging of a 64-wide tile (the M <= 64 kernels): a K-block of an
// operand stored [K][M] or [K][N] is 128 k-rows of 64 bytes in LDS, chunk c of k-row
// kr at c ^ ((kr >> 4) & 3). mn_lds_off: byte offset of chunk c of k-row kr.
// mn_read_off: a lane's offset for the transposing reads of the 16 rows 16c..16c+15
// of the tile; with mn_frag, lane (g, p) receives row 16c + p at k in [16g, 16g + 16)
// and [64 + 16g, 80 + 16g), the k order of the K-contiguous operands. In one read the
// 32 k-rows 16g + 8h + j (g = 0..3, j = 0..7) fall on every 16-byte bank group exactly
// twice, since k mod 4 and the swizzle (k >> 4) & 3 = g both vary.
__device__ __forceinline__ uint32_t mn_lds_off(int kr, int c) {
  return (uint32_t)(kr * 64 + ((c ^ ((kr >> 4) & 3)) << 4));
}
__device__ __forceinline__ uint32_t mn_read_off(int lane, int c) {
  const int g = lane >> 4, p = lane & 15;
  return (uint32_t)((16 * g + (p >> 1)) * 64 + ((c ^ g) << 4) + 8 * (p & 1));
}
__device__ __forceinline__ v8i mn_frag(const uint8_t* tile, uint32_t off) {
  const uint8_t* q = tile + off;
  const v2i a = tr8_at(q), b = tr8_at(q + 8 * 64), c = tr8_at(q + 64 * 64),
            d = tr8_at(q + 72 * 64);
  return v8i{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Bank-spreading swizzle of 16-byte chunks within a 128-byte LDS row.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int NBT = BN >= 128 ? BN / 128 : 1;  // sfB blocks per tile
  static constexpr int A_CHUNKS = BM * 8 / NT;          // 16-byte loads per thread
  static constexpr int B_CHUNKS = BN * 8 / NT;
  static constexpr int LDS_A = BM * kKBlock, LDS_B = BN * kKBlock;
  static constexpr int LDS_STAGE = LDS_A + LDS_B + (BM + NBT) * 4;
  static constexpr int LDS_BYTES = 2 * LDS_STAGE;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be 16-aligned");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "loads must tile evenly");
  static_assert(BN % 128 == 0 || 128 % BN == 0, "tile N must nest with 128-blocks");
  static_assert(BM <= NT, "one thread per tile row for row metadata");
};

// Per-tile operand view: base pointers already offset to the tile's expert.
struct TileView {
  const uint8_t* A;    // [rows][K]
  const uint8_t* B;    // [N][K]
  const uint8_t* sfA;  // [rows] sfA rows (Problem::sfA layout)
  const float* sfB;    // [NB][KB]
  uint16_t* C;         // [rows][N]
  int64_t rows;        // rows addressable in A / sfA / C
  int64_t m0, n0;
};

template <class Cfg, int KIND>
__device__ __forceinline__ void run_tile(const Problem& p, const TileView& v, int expert,
                                         int valid_rows, uint8_t* lds) {
  constexpr int BM = Cfg::BM, NT = Cfg::NT;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, NBT = Cfg::NBT;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t K = p.K, N = p.N;
  const int KB = (int)(K / kKBlock);
  const int NB = (int)((N + kKBlock - 1) / kKBlock);
  const int nb0 = (int)(v.n0 / kKBlock);

  // ---- per-thread global source addresses (clamped rows), fixed across K
  const uint8_t* a_src[Cfg::A_CHUNKS];
  int a_dst[Cfg::A_CHUNKS];
#pragma unroll
  for (int i = 0; i < Cfg::A_CHUNKS; ++i) {
    const int idx = tid + i * NT, r = idx >> 3, c = idx & 7;
    int64_t row = v.m0 + r;
    if (row >= v.rows) row = v.rows - 1;
    a_src[i] = v.A + row * K + c * 16;
    a_dst[i] = r * kKBlock + ((c ^ swz(r)) << 4);
  }
  const uint8_t* b_src[Cfg::B_CHUNKS];
  int b_dst[Cfg::B_CHUNKS];
#pragma unroll
  for (int i = 0; i < Cfg::B_CHUNKS; ++i) {
    const int idx = tid + i * NT, r = idx >> 3, c = idx & 7;
    int64_t row = v.n0 + r;
    if (row >= N) row = N - 1;
    b_src[i] = v.B + row * K + c * 16;
    b_dst[i] = r * kKBlock + ((c ^ swz(r)) << 4);
  }
  const uint8_t* sa_src = nullptr;
  const int packed = p.sfa_packed;
  if (tid < BM) {
    int64_t row = v.m0 + tid;
    if (row >= v.rows) row = v.rows - 1;
    sa_src = v.sfA + row * sfa_row_bytes(KB, packed);
  }
  const float* sb_src = nullptr;
  if (tid < NBT) {
    int nb = nb0 + tid;
    if (nb >= NB) nb = NB - 1;
    sb_src = v.sfB + (int64_t)nb * KB;
  }

  uint4 ra[Cfg::A_CHUNKS], rb[Cfg::B_CHUNKS];
  float rsa = 0.f, rsb = 0.f;

  auto gload = [&](int kb) {
    const int64_t koff = (int64_t)kb * kKBlock;
#pragma unroll
    for (int i = 0; i < Cfg::A_CHUNKS; ++i) ra[i] = *(const uint4*)(a_src[i] + koff);
#pragma unroll
    for (int i = 0; i < Cfg::B_CHUNKS; ++i) rb[i] = *(const uint4*)(b_src[i] + koff);
    if (tid < BM) rsa = sfa_at(sa_src, kb, packed);
    if (tid < NBT) rsb = sb_src[kb];
  };
  auto lstore = [&](int buf) {
    uint8_t* st = lds + buf * Cfg::LDS_STAGE;
#pragma unroll
    for (int i = 0; i < Cfg::A_CHUNKS; ++i) *(uint4*)(st + a_dst[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < Cfg::B_CHUNKS; ++i) *(uint4*)(st + Cfg::LDS_A + b_dst[i]) = rb[i];
    float* ss = (float*)(st + Cfg::LDS_A + Cfg::LDS_B);
    if (tid < BM) ss[tid] = rsa;
    if (tid < NBT) ss[BM + tid] = rsb;
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) gload(kb + 1);

    const uint8_t* st = lds + buf * Cfg::LDS_STAGE;
    const float* ss = (const float*)(st + Cfg::LDS_A + Cfg::LDS_B);
    v8i af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * Cfg::WM + i * 16 + l16;
      const uint8_t* rowp = st + r * kKBlock;
      uint4 lo = *(const uint4*)(rowp + (((2 * g) ^ swz(r)) << 4));
      uint4 hi = *(const uint4*)(rowp + (((2 * g + 1) ^ swz(r)) << 4));
      af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * Cfg::WN + j * 16 + l16;
      const uint8_t* rowp = st + Cfg::LDS_A + r * kKBlock;
      uint4 lo = *(const uint4*)(rowp + (((2 * g) ^ swz(r)) << 4));
      uint4 hi = *(const uint4*)(rowp + (((2 * g + 1) ^ swz(r)) << 4));
      bfr[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    v4f sa[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = *(const v4f*)(ss + wm * Cfg::WM + i * 16 + 4 * g);
    float sb[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t ncol = v.n0 + wn * Cfg::WN + j * 16;
      sb[j] = ss[BM + (int)(ncol / kKBlock) - nb0];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[i], bfr[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i][j][r] = __builtin_fmaf(part[r], sa[i][r] * sb[j], acc[i][j][r]);
      }

    if (kb + 1 < KB) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bf16 RNE, produced rows and in-range columns only
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rloc = wm * Cfg::WM + i * 16 + 4 * g + r;
      const int64_t row = v.m0 + rloc;
      bool ok = row < (int64_t)valid_rows;
      if (KIND == kContiguous && ok) ok = p.m_indices[row] == expert;
      if (!ok) continue;
      uint16_t* crow = v.C + row * N;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = v.n0 + wn * Cfg::WN + j * 16 + l16;
        if (col < N) crow[col] = f32_to_bf16_rne(acc[i][j][r]);
      }
    }
  }
}

template <class Cfg, int KIND>
__global__ void __launch_bounds__(Cfg::NT) gemm_kernel(Problem p) {
  extern __shared__ __align__(16) uint8_t lds[];
  int tile = blockIdx.x;
  const int per_expert = p.tiles_m * p.tiles_n;
  const int NB = (int)((p.N + kKBlock - 1) / kKBlock);
  const int KB = (int)(p.K / kKBlock);
  TileView v;
  if (KIND == kMasked) {
    const int e = tile / per_expert;
    tile -= e * per_expert;
    const int tm = tile / p.tiles_n, tn = tile - (tile / p.tiles_n) * p.tiles_n;
    int valid = p.masked_m[e];
    valid = valid < 0 ? 0 : (valid > (int)p.M ? (int)p.M : valid);
    v.m0 = (int64_t)tm * Cfg::BM;
    v.n0 = (int64_t)tn * Cfg::BN;
    if (v.m0 >= valid) return;  // whole tile past the expert's valid rows
    v.A = p.A + (int64_t)e * p.M * p.K;
    v.sfA = p.sfA + (int64_t)e * p.M * sfa_row_bytes(KB, p.sfa_packed);
    v.C = p.C + (int64_t)e * p.M * p.N;
    v.B = p.B + (int64_t)e * p.N * p.K;
    v.sfB = p.sfB + (int64_t)e * NB * KB;
    v.rows = p.M;
    run_tile<Cfg, KIND>(p, v, e, valid, lds);
    return;
  }
  const int tm = tile / p.tiles_n, tn = tile - (tile / p.tiles_n) * p.tiles_n;
  v.m0 = (int64_t)tm * Cfg::BM;
  v.n0 = (int64_t)tn * Cfg::BN;
  v.A = p.A;
  v.sfA = p.sfA;
  v.C = p.C;
  v.rows = p.M;
  if (KIND == kDense) {
    v.B = p.B;
    v.sfB = p.sfB;
    run_tile<Cfg, KIND>(p, v, 0, (int)p.M, lds);
    return;
  }
  // contiguous: one pass per distinct expert id among the tile's rows, in
  // increasing id order (one pass when segments are 128-aligned).
  __shared__ int s_next;
  int prev = -1;
  for (;;) {
    if (threadIdx.x == 0) s_next = 0x7FFFFFFF;
    __syncthreads();
    if (threadIdx.x < Cfg::BM) {
      const int64_t row = v.m0 + threadIdx.x;
      if (row < p.M) {
        const int id = p.m_indices[row];
        if (id > prev && id < p.G) atomicMin(&s_next, id);
      }
    }
    __syncthreads();
    const int e = s_next;
    __syncthreads();
    if (e == 0x7FFFFFFF) break;
    v.B = p.B + (int64_t)e * p.N * p.K;
    v.sfB = p.sfB + (int64_t)e * NB * KB;
    run_tile<Cfg, KIND>(p, v, e, (int)p.M, lds);
    prev = e;
  }
}

}  // namespace dg

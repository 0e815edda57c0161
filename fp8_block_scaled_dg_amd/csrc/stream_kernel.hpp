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
//   2. For each group of three blocks in order: wait until this wave's loads up to
//      the group's last block have landed (vmcnt counts the later blocks' loads, all
//      compile-time), one barrier so that every wave's DMA share of the group's A
//      tiles is visible, then for each block of the group and each 16x16 tile one
//      v_mfma_f32_16x16x128_f8f6f4 gives the block partial and it is
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
//
// Operands stored MN-contiguous (LAY bits, 64-column workgroups: W = 4, TN = 1), the
// NN / TN / TT layouts of the DeepGEMM project page (aiproducthub.cn, "core
// features"), are read in place. A K-block's tile of such an operand is 128 k-rows of
// 64 bytes (the tile's 64 rows m or n), staged in LDS with chunk c of k-row k at
// c ^ ((k >> 4) & 3), and each MFMA operand is gathered from it by four transposing
// reads (ds_read_b64_tr_b8), each giving one row's 8 consecutive k:
//   - A stored [K][M]: the block's A tile arrives by LDS DMA in that layout;
//   - B stored [K][N]: each lane still loads two 16-byte k-row pieces per block into
//     registers (so every load of the unit is in flight at once, as for B stored
//     [N][K]). At the first block of each group of three, after the group's loads
//     have landed, the wave writes the group's pieces into one of two sets of three
//     LDS slots; the group's barrier makes them visible, and the transposing reads
//     follow it.
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
__shared__ __align__(16) uint8_t stream_bt[6][128 * 64];   // B stored [K][N]: two 3-block sets

struct StreamArgs {
  Problem p;
  float* ws;           // [tiles][S][64 * BN] fp32 partials (S > 1)
  uint32_t* counters;  // [tiles], zero between calls
  int32_t S;           // K splits
  int32_t KS;          // K-blocks per split (the last split may have fewer)
  int32_t tiles;
  int32_t group;       // consecutive column tiles per XCD group (workgroup mapping)
};

template <class Cfg>
struct StreamRegs {
  v8i b[Cfg::D][Cfg::TN];
  v4f sfb[Cfg::TN][Cfg::SF4];
};

// Operand sources of one lane: buffer resources at the unit's first K-block, per-lane
// offsets, and the bytes one K-block advances (128 for K-contiguous rows, 128 x the
// row length for an operand stored [K][M] or [K][N]); b_hi: from a lane's first B
// piece to its second.
template <class Cfg>
struct StreamSrc {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc;
  uint32_t a_off[Cfg::A_DMA];
  uint32_t b_off[Cfg::TN];
  uint32_t a_step, b_step, b_hi;
};

// A lane's LDS offsets for the MN-contiguous paths: where its two B pieces go
// (bw0, bw1), and its transposing-read offsets for B (b_rd) and the four A row groups.
struct StreamLane {
  uint32_t bw0, bw1, b_rd;
  uint32_t a_rd[4];
};

// A lane's two B pieces of one block (B stored [K][N]) into a ring slot.
__device__ __forceinline__ void stream_ring_write(uint8_t* slot, const StreamLane& L, const v8i& v) {
  *(v4u*)(slot + L.bw0) = v4u{(unsigned)v[0], (unsigned)v[1], (unsigned)v[2], (unsigned)v[3]};
  *(v4u*)(slot + L.bw1) = v4u{(unsigned)v[4], (unsigned)v[5], (unsigned)v[6], (unsigned)v[7]};
}

// vmcnt = n, lgkmcnt = 0
template <int n>
__device__ __forceinline__ void stream_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

template <class Cfg, int T>
__device__ __forceinline__ void stream_issue_block(StreamRegs<Cfg>& r, const StreamSrc<Cfg>& src,
                                                   int tc, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t koa = (uint32_t)tc * src.a_step, kob = (uint32_t)tc * src.b_step;
#pragma unroll
  for (int q = 0; q < Cfg::A_DMA; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src.a_rsrc, (__attribute__((address_space(3))) void*)(stream_a<T> + (wave * Cfg::A_DMA + q) * 1024),
        16, src.a_off[q], koa, 0, 0);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(src.b_rsrc, src.b_off[j], kob, 0);
    const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(src.b_rsrc, src.b_off[j] + src.b_hi, kob, 0);
    r.b[T][j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
#endif
}

template <class Cfg, int T>
__device__ __forceinline__ void stream_issue_all(StreamRegs<Cfg>& r, const StreamSrc<Cfg>& src,
                                                 int ks, int wave) {
  if constexpr (T < Cfg::D) {
    stream_issue_block<Cfg, T>(r, src, T < ks ? T : ks - 1, wave);
    stream_issue_all<Cfg, T + 1>(r, src, ks, wave);
  }
}

// K-blocks per wait and barrier. The blocks' data arrives in issue order over the whole
// stream, so the waves still compute a group as soon as its last block has landed; on
// 64x2112x7168 groups of 3 or 5 measured 2.4 % faster than a barrier per block (11.60
// against 11.89 us), one wait for all ten blocks 3 % slower; with B stored [K][N] the
// grouped ring measured 3.6 % faster than a per-block one.
constexpr int kSyncBlocks = 3;

template <class Cfg, int T, bool PACKED, int LAY>
__device__ __forceinline__ void stream_compute(v4f (&acc)[Cfg::TM][Cfg::TN], const StreamRegs<Cfg>& r,
                                               const StreamLane& L, int ks, int g, int l16,
                                               int shift) {
  if constexpr (T < Cfg::D) {
    // At the first block of each group of kSyncBlocks, this wave's loads of every block
    // of the group have landed, and every wave's A DMAs of those blocks are visible after
    // the barrier; the group's other blocks need neither. B stored [K][N]: before that
    // barrier each wave writes its pieces of the group's blocks into the group's set of
    // ring slots (sets alternate between groups) and waits for the writes (lgkmcnt 0).
    // A set is rewritten two groups later: every wave finished reading it before it
    // reached the barrier of the group in between, which this wave has passed.
    constexpr bool RING = (LAY & kLayBN) != 0;
    constexpr int G = kSyncBlocks;
    constexpr bool SYNC = T % G == 0;
    constexpr int LAST = T + G - 1 < Cfg::D ? T + G - 1 : Cfg::D - 1;
    constexpr int SET = ((T / G) % 2) * G;  // first ring slot of this group
    if constexpr (SYNC) stream_wait<(Cfg::D - 1 - LAST) * Cfg::OPB>();
    if constexpr (RING && SYNC) {
#pragma unroll
      for (int j = 0; j < G; ++j)
        if (T + j <= LAST && T + j < ks)
          stream_ring_write(stream_bt[SET + j], L, r.b[T + j < Cfg::D ? T + j : 0][0]);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0, vmcnt and expcnt untouched
    }
    if constexpr (SYNC) __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (T < ks) {
      constexpr int TM = Cfg::TM, TN = Cfg::TN;
      v8i af[TM];
      float sa[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = i * 16 + l16;
        if constexpr ((LAY & kLayAT) != 0) {
          af[i] = mn_frag(stream_a<T>, L.a_rd[i]);
        } else {
          const uint8_t* rowp = stream_a<T> + row * kKBlock;
          const v4u lo = *(const v4u*)(rowp + ((g ^ swz(row)) << 4));
          const v4u hi = *(const v4u*)(rowp + (((g + 4) ^ swz(row)) << 4));
          af[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
        sa[i] = PACKED ? ue8m0_value(stream_sfa[row * 16 + shift + T])
                       : ((const float*)(stream_sfa + (T / 4) * 1024 + row * 16))[T % 4];
      }
      v8i bf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr ((LAY & kLayBN) != 0)
          bf[j] = mn_frag(stream_bt[SET + T % G], L.b_rd);
        else
          bf[j] = r.b[T][j];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bf[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          const float s = sa[i] * r.sfb[j][T / 4][T % 4];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(part[q], s, acc[i][j][q]);
        }
    }
    stream_compute<Cfg, T + 1, PACKED, LAY>(acc, r, L, ks, g, l16, shift);
  }
}

// PACKED: sfA in the packed UE8M0 layout (compile-time, as in the skinny kernel).
// LAY: kLayAT / kLayBN bits, the operands stored MN-contiguous.
template <class Cfg, bool PACKED, int LAY = 0>
__global__ void __launch_bounds__(Cfg::NT) stream_kernel(StreamArgs args) {
  static_assert(LAY == 0 || (Cfg::W == 4 && Cfg::TN == 1),
                "MN-contiguous operands: 64-column workgroups of 4 waves");
  constexpr int TN = Cfg::TN, TM = Cfg::TM, NT = Cfg::NT, BN = Cfg::BN;
  const Problem& p = args.p;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int KB = (int)(K / kKBlock);
  const int S = args.S;

  // workgroup -> (tile, split): the column tiles are dealt to the XCDs in groups of G
  // consecutive ones, group q on XCD q % 8, and all splits of a tile run on its XCD.
  // G = 1 for B stored [N][K]. With B stored [K][N] a tile's k-row piece is 64 bytes,
  // half of a 128-byte cache line shared with a neighbouring tile (which one alternates
  // with the k-row when N % 128 == 64), so G up to 4 keeps both on one XCD, whose L2
  // then fetches the line once, except across the edges of a group.
  const int G = args.group;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int slot = local / S, split = local - slot * S;
  const int tile = ((slot / G) * 8 + xcd) * G + slot % G;
  if (tile >= args.tiles) return;
  const int64_t n0 = (int64_t)tile * BN;
  const int kb0 = split * args.KS;
  const int ks = min(args.KS, KB - kb0);  // >= 1 (host guarantees)

  // ---- sources: buffer resources over the unit's rows, 32-bit per-lane offsets
  const int a_rows = (int)(M < 64 ? M : 64);
  StreamSrc<Cfg> src;
  StreamLane L{};
  if constexpr ((LAY & kLayAT) != 0) {
    // A stored [K][M] (M % 16 == 0): the DMA's 1 KB fills 16 k-rows of 64 bytes in
    // order; lane l writes LDS chunk pc of its k-row, which holds chunk pc ^ swizzle;
    // chunks past the last row m re-read the last valid one (never stored)
    src.a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.A + (int64_t)kb0 * kKBlock * M), 0, 0x7FFFFFFF, 0x00020000);
    src.a_step = (uint32_t)(kKBlock * M);
    const int valid = (int)(M >> 4);
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA; ++q) {
      const int byte = (wave * Cfg::A_DMA + q) * 1024 + 16 * lane;
      const int kr = byte >> 6, pc = (byte & 63) >> 4;
      int lc = pc ^ ((kr >> 4) & 3);
      if (lc >= valid) lc = valid - 1;
      src.a_off[q] = (uint32_t)kr * (uint32_t)M + (uint32_t)(lc << 4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) L.a_rd[i] = mn_read_off(lane, i);
  } else {
    src.a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.A + (int64_t)kb0 * kKBlock), 0, 0x7FFFFFFF, 0x00020000);
    src.a_step = kKBlock;
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA; ++q) {
      const int R = (wave * Cfg::A_DMA + q) * 8 + (lane >> 3), c = lane & 7;
      const int row = R < a_rows ? R : a_rows - 1;
      src.a_off[q] = (uint32_t)row * (uint32_t)K + (uint32_t)((c ^ swz(R)) << 4);
    }
  }
  if constexpr ((LAY & kLayBN) != 0) {
    // B stored [K][N]: lane l loads 16 columns (chunk l % 4 of the tile, clamped to
    // the last valid chunk) of k-rows 32 wave + l / 4 and 16 further
    src.b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.B + (int64_t)kb0 * kKBlock * N + n0), 0, 0x7FFFFFFF, 0x00020000);
    src.b_step = (uint32_t)(kKBlock * N);
    src.b_hi = (uint32_t)(16 * N);
    const int kr = wave * 32 + (lane >> 2), c = lane & 3;
    const int valid = (int)((N - n0) >> 4);  // N % 16 == 0
    src.b_off[0] = (uint32_t)kr * (uint32_t)N + (uint32_t)((c < valid ? c : valid - 1) << 4);
    L.bw0 = mn_lds_off(kr, c);
    L.bw1 = mn_lds_off(kr + 16, c);
    L.b_rd = mn_read_off(lane, wave);
  } else {
    src.b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.B + n0 * K + (int64_t)kb0 * kKBlock), 0, 0x7FFFFFFF, 0x00020000);
    src.b_step = kKBlock;
    src.b_hi = 64;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int64_t r = (wave * TN + j) * 16 + l16;
      if (n0 + r >= N) r = N - 1 - n0;
      src.b_off[j] = (uint32_t)r * (uint32_t)K + (uint32_t)(g * 16);
    }
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
  stream_issue_all<Cfg, 0>(r, src, ks, wave);

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  stream_compute<Cfg, 0, PACKED, LAY>(acc, r, L, ks, g, l16, kb0 & 3);

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

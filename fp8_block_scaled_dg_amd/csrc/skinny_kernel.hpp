// skinny_kernel.hpp -- block-scaled FP8 GEMM for M <= 64 (decode shapes), gfx950.
//
// Memory-bound regime: each byte of B meets at most 64 rows of A, so the kernel is
// shaped to stream B from HBM once at full rate rather than to reuse it. The work
// unit of one workgroup is (BN columns) x (a run of consecutive K-blocks), all 64
// rows. Each K-block flows through a rolling pipeline D blocks deep:
//   1. loads: each wave's B fragments (16*TN columns) straight into MFMA operand
//      registers, and every thread's share of the block's A tile (64 x 128 bytes) and
//      sfA column into registers -- D blocks are always in flight;
//   2. when block t lands: its A share goes to LDS slot t%D (chunks swizzled so the
//      fragment reads are conflict-free), a barrier, then per 16x16 sub-tile one
//      v_mfma_f32_16x16x128_f8f6f4 gives the block partial, promoted into fp32
//      accumulators with sfA[m][kb] * sfB[n/128][kb] (sfB is one value per block: a
//      workgroup's columns lie in one 128-block) -- the two-level accumulation of the
//      DeepGEMM launch article, deepseek.csdn.net, section 1.2 "precision
//      safeguards"; then block t+D is issued into the freed registers;
//   3. with one K split (S = 1) the tile is rounded to bf16 and stored; with S > 1
//      each split writes its fp32 partial to a workspace, and the last split of a
//      column tile to arrive (an atomic counter) sums the S partials in split order
//      -- a fixed order, so the result is deterministic -- rounds and stores.
// Operand k order: within a K-block the MFMA sums over any order of k that A and B
// share, so lane (g, r) of a fragment holds k in [16g, 16g+16) and [64+16g, 80+16g)
// for both operands. Each B load instruction then reads 64 contiguous bytes of every
// row it touches (whole cache-line halves) rather than four scattered 16-byte pieces.
// Every load inside the loop is unconditional, its block index clamped into the unit's
// range, so the compiler's waits are exact: computing block t waits for block t only.
// The unit's last D blocks are computed after the loop with nothing more issued (a
// tail that re-read the last block instead was 13 % slower on 64x32768x512, whose
// units are 4 blocks: half again as many loads).
//
// Operands stored MN-contiguous (LAY bits; 64-column workgroups, W = 4, TN = 1), the
// NN / TN / TT layouts of the DeepGEMM project page (aiproducthub.cn, "core
// features"), are read in place. A block's tile of such an operand goes to its LDS slot
// as 128 k-rows of 64 bytes (mn_lds_off) and each MFMA operand is gathered from it by
// transposing reads (mn_frag):
//   - A stored [K][M] (M % 16 == 0): the threads' 16-byte chunks are k-row pieces;
//   - B stored [K][N]: each lane loads two 16-byte k-row pieces per block (4 lanes per
//     64-byte k-row segment of the tile) into registers, written into the slot beside
//     the A tile before the block's barrier. Column tiles go to the XCDs in groups of
//     consecutive ones (as in the stream kernel): a tile's k-row piece is half a
//     128-byte line shared with a neighbouring tile.
#pragma once

#include "gemm_kernel.hpp"

namespace dg {

template <int W_, int TN_, int D_>
struct SkinnyCfg {
  static constexpr int W = W_, TN = TN_, D = D_, NT = W * 64;
  static constexpr int TM = 4;            // 64 rows = 4 sub-tiles of 16
  static constexpr int SMAX = 8;          // most K splits one launch uses
  static constexpr int BN = 16 * W * TN;  // columns per workgroup
  static constexpr int A_PER = 512 / NT;  // 16-byte A chunks per thread per block
  static constexpr int SLOT = 64 * kKBlock + 64 * 4;  // A tile + sfA column
  static constexpr int LDS_BYTES = D * SLOT;
  static constexpr int SLOT_BN = SLOT + 128 * 64;      // + B tile stored [K][N]
  static constexpr int LDS_BYTES_BN = D * SLOT_BN;
  static constexpr int LDS_OUT = 64 * BN * 2;  // bf16 output staging (aliases the slots)
  static_assert(512 % NT == 0, "A chunks split evenly over the threads");
  static_assert(LDS_OUT <= LDS_BYTES, "output staging fits in the pipeline slots");
  static_assert(BN <= 128 && 128 % BN == 0, "a column tile lies inside one 128-block");
  static_assert(D >= 2, "slot reuse needs a barrier in between");
};

struct SkinnyArgs {
  Problem p;
  float* ws;           // [tiles][S][64 * BN] fp32 partials (S > 1)
  uint32_t* counters;  // [tiles], zero between calls
  int32_t S;           // K splits
  int32_t KS;          // K-blocks per split (the last split may have fewer)
  int32_t tiles;       // column tiles
  int32_t group;       // B stored [K][N]: consecutive column tiles per XCD group
};

// Registers of one block in flight.
template <class Cfg>
struct SkinnyStage {
  v8i b[Cfg::TN];
  v4u a[Cfg::A_PER];
  float sa;
};

// Sources of one thread at the unit's first K-block; a K-block advances A by a_step
// and B by b_step bytes (128, or 128 rows of an operand stored [K][M] / [K][N]); b_hi:
// from a lane's first B piece to its second.
template <class Cfg>
struct SkinnySrc {
  const uint8_t* b_row[Cfg::TN];
  const uint8_t* a_src[Cfg::A_PER];
  int a_dst[Cfg::A_PER];
  const uint8_t* sa_src;  // this lane's sfA row, at K-block kb0
  int64_t a_step, b_step, b_hi;
};

// LDS offsets of the MN-contiguous paths: where a lane's two B pieces go in the slot's
// B tile, and its transposing-read offsets for B and the four A row groups.
struct SkinnyLane {
  uint32_t bw0, bw1, b_rd;
  uint32_t a_rd[4];
};

template <class Cfg, bool PACKED>
__device__ __forceinline__ void skinny_issue(SkinnyStage<Cfg>& st, const SkinnySrc<Cfg>& src,
                                             int tc) {
  const int64_t offa = (int64_t)tc * src.a_step, offb = (int64_t)tc * src.b_step;
  st.sa = PACKED ? ue8m0_value(src.sa_src[tc]) : ((const float*)src.sa_src)[tc];
#pragma unroll
  for (int u = 0; u < Cfg::A_PER; ++u) st.a[u] = *(const v4u*)(src.a_src[u] + offa);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const v4u lo = *(const v4u*)(src.b_row[j] + offb);
    const v4u hi = *(const v4u*)(src.b_row[j] + offb + src.b_hi);
    st.b[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
}

// MFMA + promotion of one block whose A tile and sfA column (and, B stored [K][N], B
// tile) are in LDS slot `slot`.
template <class Cfg, int LAY>
__device__ __forceinline__ void skinny_mma(v4f (&acc)[Cfg::TM][Cfg::TN], const uint8_t* slot,
                                           const v8i* bfrag, float sb, int g, int l16,
                                           const SkinnyLane& L) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  const float* sa = (const float*)(slot + 64 * kKBlock);
  v8i af[TM];
  v4f sab[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if constexpr ((LAY & kLayAT) != 0) {
      af[i] = mn_frag(slot, L.a_rd[i]);
    } else {
      const int r = i * 16 + l16;
      const uint8_t* rowp = slot + r * kKBlock;
      const uint4 lo = *(const uint4*)(rowp + ((g ^ swz(r)) << 4));
      const uint4 hi = *(const uint4*)(rowp + (((g + 4) ^ swz(r)) << 4));
      af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                  (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    sab[i] = *(const v4f*)(sa + i * 16 + 4 * g) * sb;
  }
  v8i bf[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if constexpr ((LAY & kLayBN) != 0)
      bf[j] = mn_frag(slot + Cfg::SLOT, L.b_rd);
    else
      bf[j] = bfrag[j];
  }
  v4f part[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      part[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          af[i], bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[i][j][q] = __builtin_fmaf(part[i][j][q], sab[i][q], acc[i][j][q]);
}

// PACKED: sfA in the packed UE8M0 layout (a compile-time choice, so that the fp32
// form carries no trace of it). LAY: kLayAT / kLayBN bits, the operands stored
// MN-contiguous.
template <class Cfg, bool PACKED, int LAY = 0>
__global__ void __launch_bounds__(Cfg::NT) skinny_kernel(SkinnyArgs args) {
  static_assert(LAY == 0 || (Cfg::W == 4 && Cfg::TN == 1),
                "MN-contiguous operands: 64-column workgroups of 4 waves");
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr int TN = Cfg::TN, TM = Cfg::TM, NT = Cfg::NT, BN = Cfg::BN, D = Cfg::D;
  constexpr int A_PER = Cfg::A_PER;
  constexpr int SLOT = (LAY & kLayBN) ? Cfg::SLOT_BN : Cfg::SLOT;
  const Problem& p = args.p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int KB = (int)(K / kKBlock);
  const int S = args.S;
  int tile, split;
  if constexpr ((LAY & kLayBN) != 0) {
    // column tiles in groups of G consecutive ones, group q on XCD q % 8 (workgroup b
    // runs on XCD b % 8), all splits of a tile on its XCD
    const int G = args.group, xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int slot = local / S;
    split = local - slot * S;
    tile = ((slot / G) * 8 + xcd) * G + slot % G;
    if (tile >= args.tiles) return;
  } else {
    tile = blockIdx.x / S;
    split = blockIdx.x - tile * S;
  }
  const int64_t n0 = (int64_t)tile * BN;
  const int kb0 = split * args.KS;
  const int ks = min(args.KS, KB - kb0);  // >= 1 (host guarantees)
  const float* sfb = p.sfB + (int64_t)(n0 / kKBlock) * KB + kb0;

  // ---- per-thread sources. A chunk c (16 bytes) of a block: row c/8, physical chunk
  // c%8 holding the logical chunk the swizzle puts there. Rows past M read row M-1
  // and rows past N clamp to N-1; such outputs are never stored.
  SkinnySrc<Cfg> src;
  SkinnyLane L{};
  if constexpr ((LAY & kLayBN) != 0) {
    // B stored [K][N]: lane l loads 16 columns (chunk l % 4 of the tile, clamped to the
    // last valid chunk: such columns are never stored) of k-rows 32 wave + l / 4 and 16
    // further
    const int kr = wave * 32 + (lane >> 2), c = lane & 3;
    const int valid = (int)((N - n0) >> 4);  // N % 16 == 0
    src.b_row[0] = p.B + ((int64_t)kb0 * kKBlock + kr) * N + n0 + ((c < valid ? c : valid - 1) << 4);
    src.b_step = kKBlock * N;
    src.b_hi = 16 * N;
    L.bw0 = mn_lds_off(kr, c);
    L.bw1 = mn_lds_off(kr + 16, c);
    L.b_rd = mn_read_off(lane, wave);
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int64_t r = n0 + (wave * TN + j) * 16 + l16;
      if (r >= N) r = N - 1;
      src.b_row[j] = p.B + r * K + (int64_t)kb0 * kKBlock + g * 16;
    }
    src.b_step = kKBlock;
    src.b_hi = 64;
  }
  if constexpr ((LAY & kLayAT) != 0) {
    // A stored [K][M] (M % 16 == 0): chunk c is physical chunk c % 4 of k-row c / 4,
    // holding logical chunk (c % 4) ^ swizzle (clamped to the last valid one)
    const int valid = (int)(M >> 4);
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
      const int c = tid + u * NT, kr = c >> 2, pc = c & 3;
      int lc = pc ^ ((kr >> 4) & 3);
      if (lc >= valid) lc = valid - 1;
      src.a_src[u] = p.A + ((int64_t)kb0 * kKBlock + kr) * M + (lc << 4);
      src.a_dst[u] = kr * 64 + (pc << 4);
    }
    src.a_step = kKBlock * M;
#pragma unroll
    for (int i = 0; i < 4; ++i) L.a_rd[i] = mn_read_off(lane, i);
  } else {
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
      const int c = tid + u * NT, row = c >> 3, phys = c & 7;
      const int64_t r = row < M ? row : M - 1;
      src.a_src[u] = p.A + r * K + (int64_t)kb0 * kKBlock + ((phys ^ swz(row)) << 4);
      src.a_dst[u] = row * kKBlock + (phys << 4);
    }
    src.a_step = kKBlock;
  }
  {
    const int64_t r = lane < M ? lane : M - 1;
    src.sa_src = p.sfA + r * sfa_row_bytes(KB, PACKED) + (PACKED ? kb0 : kb0 * 4);
  }

  SkinnyStage<Cfg> st[D];
#pragma unroll
  for (int j = 0; j < D; ++j) skinny_issue<Cfg, PACKED>(st[j], src, j < ks ? j : ks - 1);

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- the pipeline: block t lives in stage/slot t % D (static within the body)
  auto stage_in = [&](int j) {
    uint8_t* slot = lds + j * SLOT;
#pragma unroll
    for (int u = 0; u < A_PER; ++u) *(v4u*)(slot + src.a_dst[u]) = st[j].a[u];
    if (wave == 0) ((float*)(slot + 64 * kKBlock))[lane] = st[j].sa;
    if constexpr ((LAY & kLayBN) != 0) {
      const v8i& v = st[j].b[0];
      *(v4u*)(slot + Cfg::SLOT + L.bw0) =
          v4u{(unsigned)v[0], (unsigned)v[1], (unsigned)v[2], (unsigned)v[3]};
      *(v4u*)(slot + Cfg::SLOT + L.bw1) =
          v4u{(unsigned)v[4], (unsigned)v[5], (unsigned)v[6], (unsigned)v[7]};
    }
    __syncthreads();  // block t's A tile and sfA column (and B tile) are in the slot
  };
  int t0 = 0;
  for (; t0 + D < ks; t0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int t = t0 + j;
      stage_in(j);
      skinny_mma<Cfg, LAY>(acc, lds + j * SLOT, st[j].b, sfb[t], g, l16, L);
      const int tn = t + D;
      skinny_issue<Cfg, PACKED>(st[j], src, tn < ks ? tn : ks - 1);
    }
  }
  // the last D blocks (or fewer): nothing more to issue
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int t = t0 + j;
    stage_in(j);
    if (t < ks) skinny_mma<Cfg, LAY>(acc, lds + j * SLOT, st[j].b, sfb[t], g, l16, L);
  }

  // ---- split reduction (S > 1): partial out, last arriving split sums in order.
  // Partials are written and read with device-scope (sc1) 16-byte buffer accesses,
  // coherent across XCDs without flushing any L2; waiting for every store to
  // complete before the arrival count is taken makes the count a release. The last
  // split fetches all S partials at once (split index clamped, so the load count is
  // fixed), then adds them in split order.
  if (S > 1) {
    constexpr int SMAX = Cfg::SMAX;
    constexpr int per_split = 64 * BN * 4;  // bytes of one split's partial tile
    const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
        args.ws + (int64_t)tile * S * (64 * BN), 0, 0x7FFFFFFF, 0x00020000);
    constexpr int kSc1 = 16;  // cache policy: device scope
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(v4u, acc[i][j]), ws,
            split * per_split + (((wave * TM + i) * TN + j) * 64 + lane) * 16, 0, kSc1);
    if (!splitk_arrive(&args.counters[tile], (uint32_t)S)) return;
    v4u part[SMAX][TM][TN];
#pragma unroll
    for (int sp = 0; sp < SMAX; ++sp) {
      const int sc = sp < S ? sp : S - 1;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          part[sp][i][j] = __builtin_amdgcn_raw_buffer_load_b128(
              ws, sc * per_split + (((wave * TM + i) * TN + j) * 64 + lane) * 16, 0, kSc1);
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

  // ---- bf16 through LDS (aliases the pipeline slots), 16-byte stores
  __syncthreads();
  uint16_t* out_lds = (uint16_t*)lds;  // [64][BN]
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        out_lds[(i * 16 + 4 * g + q) * BN + (wave * TN + j) * 16 + l16] =
            f32_to_bf16_rne(acc[i][j][q]);
  __syncthreads();
  constexpr int CH = 64 * BN / 8;
  for (int c = tid; c < CH; c += NT) {
    const int row = c / (BN / 8), col0 = (c - row * (BN / 8)) * 8;
    if (row < M && n0 + col0 < N)
      __builtin_nontemporal_store(*(const v4u*)(out_lds + row * BN + col0),  // C is not read again
                                  (v4u*)(p.C + (int64_t)row * N + n0 + col0));
  }
}

}  // namespace dg

// pipe_kernel.hpp -- compute-bound FP8 block-scaled GEMM kernel for CDNA4 (gfx950).
//
// One workgroup of 8 waves (two per SIMD) computes one BM x BN output tile
// (256x128 or 128x256); each wave owns a 64x64 sub-tile as 2x2 tiles of 32x32.
//
// Arithmetic (DeepGEMM launch article, deepseek.csdn.net, section 1.2 "precision
// safeguards": FP8 products of one 128-wide K-block are promoted to FP32 and
// scaled before the accumulation across K-blocks):
//   level 1: two chained v_mfma_f32_32x32x64_f8f6f4 (K 0..63 and 64..127 of the
//            block) give the block's unscaled fp32 partial P of a 32x32 tile;
//   level 2: acc += P * (sfA[m][kb] * sfB[n/128][kb]) in fp32 VGPRs.
// The MFMA is issued with B as its first operand and A as its second, so every
// lane of a 32x32 result holds one row m (lane % 32) and 16 columns n. All 16
// values of a lane then share one scale product per K-block, and the 32 columns
// of a tile always sit in one 128-column sfB block.
//
// Operand movement: global memory -> LDS by direct-to-LDS buffer DMA (16 bytes per
// lane), no register staging. Scales move once per three K-blocks, by 12-byte DMAs
// per lane (three consecutive K-blocks of one row of sfA or sfB) into their own LDS
// array. Three LDS stages hold K-blocks kb,
// kb+1, kb+2; while block kb is multiplied, kb+1 and kb+2 are in flight. Each
// stage is its own __shared__ array so that the compiler can tell a DMA into one
// stage from a read of another; the K loop is unrolled by three so every stage
// index is a compile-time constant. Once per K-block each wave waits until its own
// DMAs of the next block have landed (vmcnt), then one workgroup barrier makes
// every wave's DMAs visible and retires all reads of the stage that the following
// DMA overwrites. The barrier sits in the middle of a block's MFMAs, and the next
// block's first fragments are read behind it, so LDS reads spread over the block
// instead of bursting after the barrier.
//
// LDS rows are 128 bytes; the 16-byte chunk c of row r sits at c ^ swz(r), so
// the 16 lanes served together by a 128-bit LDS read hit disjoint banks. The DMA
// applies the swizzle on the global side: lane l of an instruction fills LDS row
// 8q + l/8, chunk l%8, from global chunk (l%8) ^ swz(row).
//
// Out-of-range rows (M or N tails) are clamped to the last row for loading; the
// epilogue stores only produced rows and in-range columns.
#pragma once

#include "gemm_kernel.hpp"
#include "quant_kernel.hpp"

namespace dg {

typedef float v16f __attribute__((ext_vector_type(16)));

// SB_: K-blocks whose scales one scale load brings in (3, or 12 for 128-row tiles).
template <int BM_, int BN_, int SB_ = 3>
struct PipeCfg {
  static constexpr int BM = BM_, BN = BN_, SB = SB_;
  static constexpr int WAVES_M = BM / 64, WAVES_N = BN / 64;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = NW * 64;
  static constexpr int TM = 2, TN = 2;                 // 32x32 tiles per wave (fixed)
  static constexpr int A_DMA = BM * kKBlock / 1024 / NW;  // 1 KB DMA instructions per wave
  static constexpr int B_DMA = BN * kKBlock / 1024 / NW;
  static constexpr int RPW = BM / NW;                  // sfA rows whose scales a wave loads
  static constexpr int OPS_PER_KB = A_DMA + B_DMA;     // operand DMAs per K-block and wave
  static constexpr int OFF_B = BM * kKBlock;
  static constexpr int STAGE = (BM + BN) * kKBlock;
  // M-tiles per raster group: 32 consecutive tiles cover 1024 A rows x 1024 B rows
  static constexpr int GROUP_M = 1024 / BM;
  static_assert(NW == 8, "two waves per SIMD");
  static_assert(BN % 128 == 0, "tile columns nest in 128-column scale blocks");
  static_assert(A_DMA >= 1 && B_DMA >= 1 && RPW <= 32 && 32 % RPW == 0, "DMA split");
  static_assert(SB == 3 || (SB == 12 && BM == 128), "scale batch");
};

constexpr int kPipeStageBytes = 49152;  // (256 + 128) * 128
static_assert(PipeCfg<256, 128>::STAGE == kPipeStageBytes, "stage size");
static_assert(PipeCfg<128, 256>::STAGE == kPipeStageBytes, "stage size");

__shared__ __align__(16) uint8_t pipe_stage0[kPipeStageBytes];
__shared__ __align__(16) uint8_t pipe_stage1[kPipeStageBytes];
__shared__ __align__(16) uint8_t pipe_stage2[kPipeStageBytes];
// Scales. Cfg::SB = 3: those of three consecutive K-blocks; lane l of wave w's 12-byte
// sfA DMA puts row (w * RPW + l % RPW)'s three values at byte w * 1024 + 16 * l of
// pipe_scale, and every wave's sfB DMA writes the same bytes to pipe_sfb: lane l holds
// the tile's sfB row nb0 + min(l, BN/128 - 1) at byte 16 * l (identical concurrent
// writes).
// Cfg::SB = 12 (128-row tiles, long K): those of twelve consecutive K-blocks, loaded
// once per twelve blocks: every row's 48 bytes (fp32) or 16 bytes (the packed UE8M0
// words that hold the twelve bytes) sit at pipe_scale + row * 48 (or 16), as 16-byte
// chunks in lane order over the eight waves' DMAs, and the tile's sfB rows likewise at
// pipe_sfb + row * 48. Each load touches every row of the tile once, so twelve blocks
// per load instead of three cut the cache lines the scale loads touch fourfold
// (prefill 514 -> 506 us, contiguous 368 -> 360 us). With few K-blocks per tile the
// longer set-up it needs costs more than it saves (masked, 16 K-blocks: 142 -> 147 us).
constexpr int kScaleWaveBytes = 1024;
__shared__ __align__(16) uint8_t pipe_scale[8 * kScaleWaveBytes];
__shared__ __align__(16) uint8_t pipe_sfb[1024];

template <int S>
__device__ __forceinline__ uint8_t* pipe_stage() {
  return S == 0 ? pipe_stage0 : (S == 1 ? pipe_stage1 : pipe_stage2);
}

#define DG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with vmcnt = n and lgkmcnt = 0 (expcnt left at its maximum).
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

// blockIdx -> position in the tile order. Workgroups are dealt to the 8 XCDs
// round robin; this gives XCD x a contiguous range of the order so that the
// tiles it runs at the same time share A rows and B columns in its L2.
__device__ __forceinline__ int xcd_tile_order(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Grouped raster: GROUP_M consecutive M-tiles sweep all N-tiles together.
template <int GM>
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GM * tiles_n;
  const int group = t / per_group;
  const int first = group * GM;
  const int gsize = tiles_m - first < GM ? tiles_m - first : GM;
  const int idx = t - group * per_group;
  tm = first + idx % gsize;
  tn = idx / gsize;
}

// DMA sources of one thread: buffer resources for the tile's rows (wave-uniform,
// SGPRs) plus 32-bit per-lane byte offsets; the K-block offset goes in the
// instruction's scalar offset (a_kstep / b_kstep bytes per K-block: 128 for a
// K-contiguous operand, 128 rows of the stored matrix for an MN-contiguous one). The
// scale resources end exactly at the end of sfA and sfB, so reads past the last
// K-block of the last row return zero.
template <class Cfg>
struct PipeThread {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc, sa_rsrc, sb_rsrc;
  uint32_t a_kstep, b_kstep;
  uint32_t a_off[Cfg::A_DMA];
  uint32_t b_off[Cfg::B_DMA];
  uint32_t sa_off;  // this lane's sfA row (and, 128-row tiles, chunk)
  uint32_t sb_off;  // this lane's sfB row (and chunk)
  int sa_shift;     // sfA's scalar offset for K-block kb is (kb >> sa_shift) * 4 bytes:
                    // 0 for fp32 values, 2 for packed UE8M0 words (nonzero = packed)
  int kb_lo;        // first K-block of the run: scale batches start at kb_lo + 12 j
};

// Raw buffer over [p, p + bytes), bytes < 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p,
                                                           int64_t bytes = 0x7FFFFFFF) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0,
                                           (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF),
                                           0x00020000);
}

// The scale DMAs issued with K-block kb's operand DMAs when kb starts a group of three
// blocks (relative to the run's first block): with Cfg::SB = 3 the three blocks'
// scales; with Cfg::SB = 12 twelve blocks' scales when kb also starts a group of
// twelve, and nothing otherwise. Scales are read only at the start of a group of three,
// before the barrier after which this refill is issued, so one buffer serves.
template <class Cfg>
__device__ __forceinline__ void pipe_issue_scales(const PipeThread<Cfg>& th, int kb, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (Cfg::SB == 12) {
    if ((kb - th.kb_lo) % Cfg::SB == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(th.sa_rsrc,
                                               DG_LDS(pipe_scale + wave * kScaleWaveBytes), 16,
                                               th.sa_off, (kb >> th.sa_shift) << 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(th.sb_rsrc, DG_LDS(pipe_sfb), 16, th.sb_off,
                                               kb * 4, 0, 0);
    }
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(th.sa_rsrc,
                                             DG_LDS(pipe_scale + wave * kScaleWaveBytes), 12,
                                             th.sa_off, (kb >> th.sa_shift) << 2, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(th.sb_rsrc, DG_LDS(pipe_sfb), 12, th.sb_off, kb * 4,
                                             0, 0);
  }
#endif
}

// The DMAs of K-block kb into stage S. With SCALES (kb a multiple of 3) the batch
// starts with the scales of K-blocks kb..kb+2 (the wave's share of sfA rows and its
// copy of the tile's sfB rows) into pipe_scale. They go first, so that a wait that
// leaves only the newest OPS_PER_KB operand DMAs in flight covers them too.
template <class Cfg, int S, bool SCALES>
__device__ __forceinline__ void pipe_issue(const PipeThread<Cfg>& th, int kb, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // the LDS-DMA builtin exists in the device pass only
  if (SCALES) pipe_issue_scales<Cfg>(th, kb, wave);
  uint8_t* st = pipe_stage<S>();
  const int koff_a = kb * th.a_kstep, koff_b = kb * th.b_kstep;
#pragma unroll
  for (int q = 0; q < Cfg::A_DMA; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(th.a_rsrc, DG_LDS(st + (wave * Cfg::A_DMA + q) * 1024),
                                             16, th.a_off[q], koff_a, 0, 0);
#pragma unroll
  for (int q = 0; q < Cfg::B_DMA; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        th.b_rsrc, DG_LDS(st + Cfg::OFF_B + (wave * Cfg::B_DMA + q) * 1024), 16, th.b_off[q],
        koff_b, 0, 0);
#endif
}

// Operand DMAs [LO, HI) of K-block kb's batch into stage S (op q < A_DMA: A op q,
// else B op q - A_DMA), the scales first when SCALES and LO == 0: the batch of
// pipe_issue, issued a few instructions at a time.
template <class Cfg, int S, bool SCALES, int LO, int HI>
__device__ __forceinline__ void pipe_issue_ops(const PipeThread<Cfg>& th, int kb, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (SCALES && LO == 0) pipe_issue_scales<Cfg>(th, kb, wave);
  uint8_t* st = pipe_stage<S>();
  const int koff_a = kb * th.a_kstep, koff_b = kb * th.b_kstep;
#pragma unroll
  for (int q = LO; q < HI; ++q) {
    if (q < Cfg::A_DMA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(th.a_rsrc,
                                               DG_LDS(st + (wave * Cfg::A_DMA + q) * 1024), 16,
                                               th.a_off[q], koff_a, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          th.b_rsrc, DG_LDS(st + Cfg::OFF_B + (wave * Cfg::B_DMA + q - Cfg::A_DMA) * 1024), 16,
          th.b_off[q - Cfg::A_DMA], koff_b, 0, 0);
  }
#endif
}

// Byte address of stage S for the fragment reads. Stages 0 and 1 start below 64 KB,
// so their base folds into the 16-bit offset of ds_read; stage 2 starts above it
// and is added at run time from an opaque SGPR, so that the compiler does not keep
// a second hoisted set of per-lane addresses for it.
template <int S>
__device__ __forceinline__ const uint8_t* read_base() {
  if (S < 2) return pipe_stage<S>();
  uint32_t off = 0;
  asm volatile("" : "+s"(off));
  return pipe_stage<S>() + off;
}

__device__ __forceinline__ v8i frag_at(const uint8_t* p, uint32_t lo, uint32_t hi) {
  const v4u x = *(const v4u*)(p + lo);
  const v4u y = *(const v4u*)(p + hi);
  return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

#define DG_FENCE() __builtin_amdgcn_sched_barrier(0)
// An empty volatile asm that reads and rewrites x: the instructions producing x cannot
// move past it. The scheduling fences above bind the machine scheduler only; code
// motion before it (sinking arithmetic into a later basic block) ignores them.
#define DG_PIN(x) asm volatile("" : "+v"(x))

__device__ __forceinline__ v16f mfma32(const v8i& b, const v8i& a, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, 0, 0, 0);
}

// acc[e] += p[e] * s for e in [E0, E0 + 8)
template <int E0>
__device__ __forceinline__ void promote8(v16f& acc, const v16f& p, float s) {
#pragma unroll
  for (int e = E0; e < E0 + 8; ++e) acc[e] = __builtin_fmaf(p[e], s, acc[e]);
}

// Per-lane LDS geometry of a wave's 64x64 sub-tile. A lane reads row (lane % 32)
// of each 32-row tile; chunk pairs {2g, 2g+1} (K half 0) and {4+2g, 5+2g} (K half
// 1), g = lane / 32. The swizzle depends on the row only through lane % 32 (tile
// and wave offsets are multiples of 32 rows), so four byte offsets per operand
// serve every tile; tile 1 is 4096 bytes further.
//
// An MN-contiguous operand (layout bit set) is staged as 128 k-rows of ROW = BM or BN
// bytes (its tile's rows m or n along each k-row), and its 16-byte chunk c of k-row
// k sits at chunk c ^ tswz(k) (tswz below). A fragment is then assembled from four
// transposing 8-byte reads (ds_read_b64_tr_b8), each giving 8 consecutive k of one
// row: in a group of 16 lanes, lanes 2j and 2j+1 point at the two 8-byte halves of
// the 16 consecutive rows of k-row k0 + j, and lane i receives row i of those 16 at
// k0..k0+7. For MFMA lane (r32, g) of tile t, group q = lane / 16 covers rows
// 32t + 16 (q % 2) + 0..15 and k = 32 (q / 2) + 8d + 0..7 in read d. Only two per-lane
// offsets per operand are kept (tile 0 and tile 1); the k-row of read d and K half h
// is the immediate (64h + 8d) * ROW.
__device__ __forceinline__ int tswz(int k, int row_chunks) {
  // 8 consecutive k-rows x the 2 chunks of one 32-row tile hit 16 distinct chunk
  // positions of a 64-bank LDS: whole rows of 16 chunks spread k mod 8 over chunk
  // bits 1..3; half rows (8 chunks, two k-rows per bank sweep) spread k mod 8 / 2
  return row_chunks == 16 ? 2 * (k & 7) : 2 * ((k & 7) >> 1);
}

template <class Cfg, int LAY>
struct PipeLane {
  uint32_t va[4], vb[4];  // MN-contiguous operand: [0], [1] = tile 0, tile 1
  uint32_t sa0, sa1;  // byte offsets in pipe_scale of this lane's two A rows
  uint32_t sb;        // byte offset in pipe_sfb of the wave's sfB row
  // per-lane offset of the transposing reads of 32-row tile t of an MN-contiguous
  // operand whose wave slice starts at row r0 of a tile ROW bytes wide
  template <int ROW>
  __device__ __forceinline__ static uint32_t toff(int lane, int r0, int t) {
    const int q = lane >> 4, p = lane & 15, j = p >> 1, half = p & 1;
    const int krow = 32 * (q >> 1) + j;
    const int c = (r0 + 32 * t + 16 * (q & 1)) >> 4;
    return (uint32_t)(krow * ROW + ((c ^ tswz(krow, ROW / 16)) << 4) + 8 * half);
  }
  __device__ __forceinline__ PipeLane(int wave, int lane, bool packed) {
    const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
    const int r32 = lane & 31, g = lane >> 5;
    const int sw = swz(r32);
    const int chunk[4] = {2 * g, 2 * g + 1, 4 + 2 * g, 5 + 2 * g};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = (uint32_t)((chunk[k] ^ sw) << 4);
      va[k] = (uint32_t)(wm * 64 + r32) * kKBlock + c;
      vb[k] = (uint32_t)Cfg::OFF_B + (uint32_t)(wn * 64 + r32) * kKBlock + c;
    }
    if (LAY & kLayAT) {
      va[0] = toff<Cfg::BM>(lane, wm * 64, 0);
      va[1] = toff<Cfg::BM>(lane, wm * 64, 1);
    }
    if (LAY & kLayBN) {
      vb[0] = (uint32_t)Cfg::OFF_B + toff<Cfg::BN>(lane, wn * 64, 0);
      vb[1] = (uint32_t)Cfg::OFF_B + toff<Cfg::BN>(lane, wn * 64, 1);
    }
    const int ra0 = wm * 64 + r32, ra1 = ra0 + 32;
    if (Cfg::SB == 12) {
      const int row_bytes = packed ? 16 : 4 * Cfg::SB;
      sa0 = (uint32_t)(ra0 * row_bytes);
      sa1 = (uint32_t)(ra1 * row_bytes);
      sb = (uint32_t)(((wn * 64) / 128) * 4 * Cfg::SB);
    } else {
      sa0 = (uint32_t)((ra0 / Cfg::RPW) * kScaleWaveBytes + (ra0 % Cfg::RPW) * 16);
      sa1 = (uint32_t)((ra1 / Cfg::RPW) * kScaleWaveBytes + (ra1 % Cfg::RPW) * 16);
      sb = (uint32_t)(((wn * 64) / 128) * 16);
    }
  }
};

// Both K-half fragments of 32-row tile `tile` (0/1) of the operand whose per-lane
// offsets are v.
__device__ __forceinline__ void read_tile(const uint8_t* st, const uint32_t (&v)[4], int tile,
                                          v8i& h0, v8i& h1) {
  const uint8_t* p = st + tile * 32 * kKBlock;
  h0 = frag_at(p, v[0], v[1]);
  h1 = frag_at(p, v[2], v[3]);
}

// The same fragments of an MN-contiguous operand staged as k-rows of ROW bytes: four
// transposing reads per K half (see PipeLane).
template <int ROW>
__device__ __forceinline__ void read_tile_t(const uint8_t* st, const uint32_t (&v)[4], int tile,
                                            v8i& h0, v8i& h1) {
  const uint8_t* p = st + v[tile];
  const v2i a0 = tr8_at(p), a1 = tr8_at(p + 8 * ROW), a2 = tr8_at(p + 16 * ROW),
            a3 = tr8_at(p + 24 * ROW);
  const v2i b0 = tr8_at(p + 64 * ROW), b1 = tr8_at(p + 72 * ROW), b2 = tr8_at(p + 80 * ROW),
            b3 = tr8_at(p + 88 * ROW);
  h0 = v8i{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
  h1 = v8i{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// A-tile and B-tile fragment reads in the operand's layout.
template <class Cfg, int LAY>
__device__ __forceinline__ void read_a(const uint8_t* st, const PipeLane<Cfg, LAY>& pl, int tile,
                                       v8i& h0, v8i& h1) {
  if (LAY & kLayAT)
    read_tile_t<Cfg::BM>(st, pl.va, tile, h0, h1);
  else
    read_tile(st, pl.va, tile, h0, h1);
}

template <class Cfg, int LAY>
__device__ __forceinline__ void read_b(const uint8_t* st, const PipeLane<Cfg, LAY>& pl, int tile,
                                       v8i& h0, v8i& h1) {
  if (LAY & kLayBN)
    read_tile_t<Cfg::BN>(st, pl.vb, tile, h0, h1);
  else
    read_tile(st, pl.vb, tile, h0, h1);
}

// Fragments a K-block's step starts with: A tile 0 and both B tiles, read during
// the previous step.
struct Frag0 {
  v8i a0, a1, b0, b1, c0, c1;  // A tile 0 (K halves), B tile 0, B tile 1
};

// Scale products of the current three K-blocks for this lane's two A rows.
struct PipeScales {
  float s0[3], s1[3];
};

// One pipeline step for K-block kb held in stage S.
// MFMA order: independent pairs, so a tile's second K half never waits on its first:
//   M1 t00.h0  M2 t01.h0  M3 t00.h1  M4 t01.h1  M5 t10.h0  M6 t11.h0  M7 t10.h1  M8 t11.h1
// (tij = A tile i x B tile j). Each tile's promotion runs in the shadow of the two
// MFMAs after its last one: t00 and t01 during M5-M8, t10 and t11 of block kb during
// M1-M4 of the next step (carries c10, c11).
// After M4, A tile 0 of kb is dead: the wave waits for its own DMAs of block kb+1
// and meets the others at the barrier; block kb+1 is then in LDS and every read of
// block kb is done, so the DMA of block kb+3 refills kb's stage, and A tile 0 and
// B tile 1 of kb+1 are read (B tile 1 into spare registers). B tile 0 of kb+1 is
// read after M7, when kb's is dead. Scheduling fences keep this order; the compiler
// inserts only the LDS waits. The carried promotions are pinned before the barrier:
// in the step that may issue the scale DMAs (a branch after M5) the compiler otherwise
// sinks them past that branch, behind the barrier, and prefill and the contiguous
// layout measured 1-3 % slower that way.
template <class Cfg, int S, int MODE, int LAY>
__device__ __forceinline__ void pipe_step(const PipeThread<Cfg>& th, const PipeLane<Cfg, LAY>& pl,
                                          v16f (&acc)[2][2], Frag0& f, v16f (&carry)[2],
                                          float& carry_s, PipeScales& sc, int kb, int KB,
                                          int wave) {
  constexpr bool HI = MODE == 2;  // the wave's second 32-row A tile holds output rows
  if constexpr (MODE == 0) {
    // a wave with no output rows or columns of its own: only its share of the DMAs
    wait_vm_lgkm0<Cfg::OPS_PER_KB>();
    __builtin_amdgcn_s_barrier();
    DG_FENCE();
    pipe_issue<Cfg, S, S == 0>(th, kb + 3 < KB ? kb + 3 : KB - 1, wave);
    DG_FENCE();
    return;
  }
  const uint8_t* st = read_base<S>();
  const uint8_t* nst = read_base<(S + 1) % 3>();
  const v16f zero = {};

  v8i a10, a11;
  if (HI) read_a(st, pl, 1, a10, a11);
  if (S == 0 && Cfg::SB == 12) {
    // scales of K-blocks kb..kb+2 (landed before the previous barrier), at position
    // r = (kb - kb_lo) % 12 of the twelve-block group starting at b0 = kb - r: three fp32
    // values from float r of the row, or (packed) bytes (b0 % 4) + r .. of the words
    // from b0 / 4 on
    const int r = (kb - th.kb_lo) % Cfg::SB;
    const float* bsf = (const float*)(pipe_sfb + pl.sb) + r;
    float a0[3], a1[3];
    if (th.sa_shift) {
      const int o = ((kb - r) & 3) + r;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        a0[j] = ue8m0_value(pipe_scale[pl.sa0 + o + j]);
        a1[j] = ue8m0_value(pipe_scale[pl.sa1 + o + j]);
      }
    } else {
      const float* x0 = (const float*)(pipe_scale + pl.sa0) + r;
      const float* x1 = (const float*)(pipe_scale + pl.sa1) + r;
#pragma unroll
      for (int j = 0; j < 3; ++j) a0[j] = x0[j], a1[j] = x1[j];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      sc.s0[j] = a0[j] * bsf[j];
      sc.s1[j] = a1[j] * bsf[j];
    }
  } else if (S == 0) {
    // scales of K-blocks kb..kb+2 (landed before the previous barrier): three fp32
    // values, or (packed) bytes kb % 4 .. kb % 4 + 2 of the words from kb / 4 on
    const v4f b = *(const v4f*)(pipe_sfb + pl.sb);
    float a0[3], a1[3];
    if (th.sa_shift) {
      const uint2 w0 = *(const uint2*)(pipe_scale + pl.sa0);
      const uint2 w1 = *(const uint2*)(pipe_scale + pl.sa1);
      const uint64_t q0 = ((uint64_t)w0.y << 32) | w0.x, q1 = ((uint64_t)w1.y << 32) | w1.x;
      const int o = (kb & 3) * 8;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        a0[j] = ue8m0_value((uint32_t)(q0 >> (o + 8 * j)) & 0xFFu);
        a1[j] = ue8m0_value((uint32_t)(q1 >> (o + 8 * j)) & 0xFFu);
      }
    } else {
      const v4f x0 = *(const v4f*)(pipe_scale + pl.sa0);
      const v4f x1 = *(const v4f*)(pipe_scale + pl.sa1);
#pragma unroll
      for (int j = 0; j < 3; ++j) a0[j] = x0[j], a1[j] = x1[j];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      sc.s0[j] = a0[j] * b[j];
      sc.s1[j] = a1[j] * b[j];
    }
  }
  DG_FENCE();
  v16f p00 = mfma32(f.b0, f.a0, zero);  // M1
  if (HI) { promote8<0>(acc[1][0], carry[0], carry_s); DG_PIN(acc[1][0]); }
  DG_FENCE();
  v16f p01 = mfma32(f.c0, f.a0, zero);  // M2
  if (HI) { promote8<8>(acc[1][0], carry[0], carry_s); DG_PIN(acc[1][0]); }
  DG_FENCE();
  p00 = mfma32(f.b1, f.a1, p00);  // M3
  if (HI) { promote8<0>(acc[1][1], carry[1], carry_s); DG_PIN(acc[1][1]); }
  DG_FENCE();
  p01 = mfma32(f.c1, f.a1, p01);  // M4
  if (HI) { promote8<8>(acc[1][1], carry[1], carry_s); DG_PIN(acc[1][1]); }
  DG_FENCE();
  // block kb+1 in LDS, block kb's stage free. Block kb+3's DMAs into it are spread
  // over M5..M8, a quarter behind each (instead of all eight waves queueing a whole
  // batch at the address unit right after the barrier); all of them precede the
  // next step's wait, so its count is unchanged.
  constexpr int OPS = Cfg::OPS_PER_KB, Q1 = (OPS + 3) / 4, Q2 = (2 * OPS + 3) / 4,
                Q3 = (3 * OPS + 3) / 4;
  const int kn = kb + 3 < KB ? kb + 3 : KB - 1;
  wait_vm_lgkm0<Cfg::OPS_PER_KB>();
  __builtin_amdgcn_s_barrier();
  DG_FENCE();
  const float s0 = sc.s0[S], s1 = sc.s1[S];
  read_a(nst, pl, 0, f.a0, f.a1);
  DG_FENCE();
  v16f p10, p11;
  if (HI) p10 = mfma32(f.b0, a10, zero);  // M5
  pipe_issue_ops<Cfg, S, S == 0, 0, Q1>(th, kn, wave);
  v8i c0n, c1n;
  read_b(nst, pl, 1, c0n, c1n);
  promote8<0>(acc[0][0], p00, s0);
  DG_FENCE();
  if (HI) p11 = mfma32(f.c0, a10, zero);  // M6
  pipe_issue_ops<Cfg, S, false, Q1, Q2>(th, kn, wave);
  promote8<8>(acc[0][0], p00, s0);
  DG_FENCE();
  if (HI) p10 = mfma32(f.b1, a11, p10);  // M7
  pipe_issue_ops<Cfg, S, false, Q2, Q3>(th, kn, wave);
  promote8<0>(acc[0][1], p01, s0);
  DG_FENCE();
  read_b(nst, pl, 0, f.b0, f.b1);
  DG_FENCE();
  if (HI) p11 = mfma32(f.c1, a11, p11);  // M8
  pipe_issue_ops<Cfg, S, false, Q3, OPS>(th, kn, wave);
  promote8<8>(acc[0][1], p01, s0);
  DG_FENCE();
  f.c0 = c0n;
  f.c1 = c1n;
  if (HI) {
    carry[0] = p10;
    carry[1] = p11;
  }
  carry_s = s1;
}

// Multiplies rows [m0, m0+BM) of the view by columns [n0, n0+BN) over the K-blocks
// [kb_lo, kb_hi) and leaves the fp32 tile in acc (lane layout: row lane % 32 of each
// 32x32 tile, columns 8*(e/4) + 4*(lane/32) + e%4). Rows at or past v.rows and
// columns at or past N read as zero (the buffer resources end there). MODE 0: the wave
// only moves its share of the tile's operands and leaves acc at zero (its 64 x 64
// sub-tile holds nothing to store); MODE 1: only the sub-tile's first 32 rows hold
// output, and the MFMAs and promotion of its second 32-row A tile are skipped (acc[1]
// stays zero); MODE 2: the whole sub-tile.
// b_hi: tile rows from 128 on come from B rows b_hi further on (and their sfB blocks
// likewise): the up half of a [gate; up] B, b_hi = I - 128. 0 for a plain tile.
template <class Cfg, int MODE, int LAY>
__device__ __forceinline__ void pipe_mainloop_as(const Problem& p, const TileView& v, int kb_lo,
                                                 int kb_hi, v16f (&acc)[Cfg::TM][Cfg::TN],
                                                 int b_hi) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: SGPR addresses
  const int64_t K = p.K, N = p.N;
  const int KB = (int)(K / kKBlock);
  const int NB = (int)((N + kKBlock - 1) / kKBlock);
  const int nb0 = (int)(v.n0 / kKBlock);

  // Offsets relative to the tile's first row stay below BM * K bytes (or BN * K);
  // the host checks that this stays below 2^31.
  PipeThread<Cfg> th;
  {
    const int a_rows = (int)(v.rows - v.m0 < Cfg::BM ? v.rows - v.m0 : Cfg::BM);
    const int b_rows = (int)(N - v.n0 < Cfg::BN ? N - v.n0 : Cfg::BN);
    // rows past the ends are out of the resources' range: the DMA writes zeros and
    // fetches nothing. An MN-contiguous operand's tile is a column range of every
    // stored k-row; its resource runs to the end of the matrix, and chunks past M or N
    // are redirected to the last valid chunk of the k-row (below).
    if (LAY & kLayAT) {
      th.a_rsrc = raw_rsrc(v.A + v.m0, K * v.rows - v.m0);
      th.a_kstep = (uint32_t)(kKBlock * v.rows);
    } else {
      th.a_rsrc = raw_rsrc(v.A + v.m0 * K, (int64_t)a_rows * K);
      th.a_kstep = kKBlock;
    }
    if (LAY & kLayBN) {
      th.b_rsrc = raw_rsrc(v.B + v.n0, K * N - v.n0);
      th.b_kstep = (uint32_t)(kKBlock * N);
    } else {
      th.b_rsrc = raw_rsrc(v.B + v.n0 * K, (int64_t)(b_hi ? Cfg::BN + b_hi : b_rows) * K);
      th.b_kstep = kKBlock;
    }
    const int64_t rb = sfa_row_bytes(KB, p.sfa_packed);
    th.sa_rsrc = raw_rsrc(v.sfA + v.m0 * rb, (v.rows - v.m0) * rb);
    th.sa_shift = p.sfa_packed ? 2 : 0;
    th.sb_rsrc = raw_rsrc(v.sfB + (int64_t)nb0 * KB, (int64_t)(NB - nb0) * KB * 4);
    const int rsub = lane >> 3, c = lane & 7;
#pragma unroll
    for (int q = 0; q < Cfg::A_DMA; ++q) {
      if (LAY & kLayAT) {
        // the DMA's 1 KB fills k-rows of BM bytes in order; lane l writes LDS chunk pc
        // of its k-row, which holds stored chunk pc ^ tswz(k)
        const int byte = (wave * Cfg::A_DMA + q) * 1024 + 16 * lane;
        const int kr = byte / Cfg::BM, pc = (byte % Cfg::BM) >> 4;
        // a chunk past the last row m re-reads the last valid chunk of its k-row, so
        // every address stays inside A (those rows are never stored)
        const int valid = (int)((v.rows - v.m0) >> 4);
        int lc = pc ^ tswz(kr, Cfg::BM / 16);
        if (lc >= valid) lc = valid - 1;
        th.a_off[q] = (uint32_t)kr * (uint32_t)v.rows + (uint32_t)(lc << 4);
      } else {
        const int R = (wave * Cfg::A_DMA + q) * 8 + rsub;
        th.a_off[q] = (uint32_t)R * (uint32_t)K + (uint32_t)((c ^ swz(R)) << 4);
      }
    }
#pragma unroll
    for (int q = 0; q < Cfg::B_DMA; ++q) {
      if (LAY & kLayBN) {
        const int byte = (wave * Cfg::B_DMA + q) * 1024 + 16 * lane;
        const int kr = byte / Cfg::BN, pc = (byte % Cfg::BN) >> 4;
        const int valid = (int)((N - v.n0) >> 4);  // N % 16 == 0
        int lc = pc ^ tswz(kr, Cfg::BN / 16);
        if (lc >= valid) lc = valid - 1;
        th.b_off[q] = (uint32_t)kr * (uint32_t)N + (uint32_t)(lc << 4);
      } else {
        const int R = (wave * Cfg::B_DMA + q) * 8 + rsub;
        const int Rg = R + (R >= 128 ? b_hi : 0);  // row of B (relative to n0)
        th.b_off[q] = (uint32_t)Rg * (uint32_t)K + (uint32_t)((c ^ swz(R)) << 4);
      }
    }
    th.kb_lo = kb_lo;
    if (Cfg::SB == 12) {
      // 16-byte chunk i = 64 wave + lane of the tile's twelve-block scale group: row
      // i / 3, chunk i % 3 (fp32), or row i (packed); lanes past the last chunk repeat
      // it (their LDS bytes are never read)
      int i = wave * 64 + lane, arow = i, chunk = 0;
      if (p.sfa_packed) {
        arow = i < 128 ? i : 127;
      } else {
        if (i >= 384) i = 383;
        arow = i / 3;
        chunk = i - 3 * arow;
      }
      if (arow >= a_rows) arow = a_rows - 1;
      th.sa_off = (uint32_t)arow * (uint32_t)rb + (uint32_t)(chunk * 16);
      // sfB: the tile's BN / 128 rows, three chunks each, in lanes 0 .. 3 BN / 128 - 1
      int l = lane < 3 * (Cfg::BN / 128) ? lane : 3 * (Cfg::BN / 128) - 1;
      int nb = l / 3;
      if (nb >= 1) nb += b_hi / 128;
      if (nb0 + nb >= NB) nb = NB - 1 - nb0;
      th.sb_off = (uint32_t)nb * (uint32_t)KB * 4u + (uint32_t)((l % 3) * 16);
    } else {
      int arow = wave * Cfg::RPW + (lane % Cfg::RPW);
      if (arow >= a_rows) arow = a_rows - 1;
      th.sa_off = (uint32_t)arow * (uint32_t)rb;
      int nb = lane < Cfg::BN / 128 ? lane : Cfg::BN / 128 - 1;
      if (nb >= 1) nb += b_hi / 128;
      if (nb0 + nb >= NB) nb = NB - 1 - nb0;
      th.sb_off = (uint32_t)nb * (uint32_t)KB * 4u;
    }
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};
  v16f carry[2] = {v16f{}, v16f{}};
  float carry_s = 0.f;
  const PipeLane<Cfg, LAY> pl(wave, lane, p.sfa_packed != 0);
  Frag0 f;
  PipeScales sc;

  // prologue: blocks 0 and 1 (and the scales of blocks 0..2) in flight; once block 0
  // has landed everywhere, block 2 starts and the first fragments of block 0 are read
  pipe_issue<Cfg, 0, true>(th, kb_lo, wave);
  pipe_issue<Cfg, 1, false>(th, kb_lo + 1 < kb_hi ? kb_lo + 1 : kb_hi - 1, wave);
  DG_FENCE();
  wait_vm_lgkm0<Cfg::OPS_PER_KB>();
  __builtin_amdgcn_s_barrier();
  DG_FENCE();
  pipe_issue<Cfg, 2, false>(th, kb_lo + 2 < kb_hi ? kb_lo + 2 : kb_hi - 1, wave);
  DG_FENCE();
  if (MODE > 0) {
    read_a(read_base<0>(), pl, 0, f.a0, f.a1);
    read_b(read_base<0>(), pl, 0, f.b0, f.b1);
    read_b(read_base<0>(), pl, 1, f.c0, f.c1);
  }
  DG_FENCE();
  int kb = kb_lo;
  for (; kb + 3 <= kb_hi; kb += 3) {
    pipe_step<Cfg, 0, MODE, LAY>(th, pl, acc, f, carry, carry_s, sc, kb, kb_hi, wave);
    pipe_step<Cfg, 1, MODE, LAY>(th, pl, acc, f, carry, carry_s, sc, kb + 1, kb_hi, wave);
    pipe_step<Cfg, 2, MODE, LAY>(th, pl, acc, f, carry, carry_s, sc, kb + 2, kb_hi, wave);
  }
  if (kb < kb_hi) pipe_step<Cfg, 0, MODE, LAY>(th, pl, acc, f, carry, carry_s, sc, kb, kb_hi, wave);
  if (kb + 1 < kb_hi)
    pipe_step<Cfg, 1, MODE, LAY>(th, pl, acc, f, carry, carry_s, sc, kb + 1, kb_hi, wave);
  if (MODE == 2) {
    promote8<0>(acc[1][0], carry[0], carry_s);
    promote8<8>(acc[1][0], carry[0], carry_s);
    promote8<0>(acc[1][1], carry[1], carry_s);
    promote8<8>(acc[1][1], carry[1], carry_s);
  }
  // every DMA has landed before the LDS can be reused or released
  DG_FENCE();
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  DG_FENCE();
}

// Which 32-row halves of the wave's sub-tile hold output: a half does when its first
// row is below v.rows and the sub-tile's first column below N; `quarters` (bit q for
// the tile's 32-row quarter q) lets the caller rule out quarters whose rows are all
// someone else's (contiguous layout). The three modes pass the same barriers.
template <class Cfg, int LAY = 0>
__device__ __forceinline__ void pipe_mainloop(const Problem& p, const TileView& v, int kb_lo,
                                              int kb_hi, v16f (&acc)[Cfg::TM][Cfg::TN],
                                              uint32_t quarters = ~0u, int b_hi = 0) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const bool cols = v.n0 + wn * 64 < p.N;
  const bool lo = cols && ((quarters >> (2 * wm)) & 1) && v.m0 + wm * 64 < v.rows;
  const bool hi = cols && ((quarters >> (2 * wm + 1)) & 1) && v.m0 + wm * 64 + 32 < v.rows;
  if (hi)
    pipe_mainloop_as<Cfg, 2, LAY>(p, v, kb_lo, kb_hi, acc, b_hi);
  else if (lo)
    pipe_mainloop_as<Cfg, 1, LAY>(p, v, kb_lo, kb_hi, acc, b_hi);
  else
    pipe_mainloop_as<Cfg, 0, LAY>(p, v, kb_lo, kb_hi, acc, b_hi);
}

// bf16 RNE store of a finished tile: produced rows (< valid_rows, and for the
// contiguous layout only rows whose m_indices entry equals `expert`) and in-range
// columns only. A lane of the MFMA result holds 4 columns of one row, so storing
// from registers would put 16 bytes into each of 32 rows per instruction, and the
// L2 would take every one as a partial-line write. Instead each wave passes its
// 64x64 sub-tile through its own 4 KB of LDS stage 2, 32 rows at a time, and reads
// it back with 8 lanes per row: each store instruction then writes 8 whole 128-byte
// row segments, an eighth of the write requests. The stores are non-temporal: C is
// not read again by this kernel, and keeping it out of L2 leaves room for A and B.
// Stage 2 is refilled only after the barrier that follows the next tile's first
// DMAs, which a wave reaches after its store. 16-byte chunk q of staged row r sits
// at chunk q ^ (r & 7), which spreads both the writes (8-byte halves of one chunk
// column from 32 rows) and the reads (a whole row per 8 lanes) evenly over the
// banks.
template <class Cfg, int KIND>
__device__ __forceinline__ void pipe_store(const Problem& p, const TileView& v, int expert,
                                           int valid_rows, const v16f (&acc)[Cfg::TM][Cfg::TN]) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN;
  static_assert(TN == 2 && Cfg::NW * 4096 <= kPipeStageBytes, "64-column sub-tiles, 4 KB per wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t N = p.N;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int r32 = lane & 31, g = lane >> 5;
  uint8_t* lds = pipe_stage2 + wave * 4096;
  const int rr = lane >> 3, ch = lane & 7;  // read side: rows rr + 8k, chunk ch
  const int64_t col = v.n0 + wn * 64 + 8 * ch;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[i][j][4 * e4 + 0]) |
                            ((uint32_t)f32_to_bf16_rne(acc[i][j][4 * e4 + 1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[i][j][4 * e4 + 2]) |
                            ((uint32_t)f32_to_bf16_rne(acc[i][j][4 * e4 + 3]) << 16);
        *(uint2*)(lds + r32 * 128 + (((4 * j + e4) ^ (r32 & 7)) << 4) + 8 * g) =
            make_uint2(lo, hi);
      }
    // the wave's LDS accesses run in order; this keeps the compiler from moving
    // the reads of other lanes' data above the writes (and the next writes above
    // these reads)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    wait_vm_lgkm0<63>();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + rr;
      const v4u d = *(const v4u*)(lds + r * 128 + ((ch ^ rr) << 4));
      const int64_t row = v.m0 + wm * 64 + i * 32 + r;
      bool ok = row < (int64_t)valid_rows && col < N;
      if (KIND == kContiguous && ok) ok = p.m_indices[row] == expert;
      if (ok) __builtin_nontemporal_store(d, (v4u*)(v.C + row * N + col));
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

// Where the fused SwiGLU epilogue writes: e4m3fn codes [rows][I] and fp32 scales
// [rows][I/128] of h = silu(gate) * up (rows as in the GEMM's A).
struct SwigluOut {
  uint8_t* codes;
  float* sf;
  int32_t I;
};

// Fused epilogue of a [gate; up] tile (BM = 128, BN = 256: tile columns 0..127 are
// gate columns n0.., 128..255 the up columns I + n0..). The activation between an
// MoE layer's two grouped GEMMs (DeepGEMM project page, aiproducthub.cn, "core
// features": Mega MoE fuses Linear1, SwiGLU and Linear2) is formed from the fp32
// accumulators and quantized per 1x128 block (h's columns n0..n0+127 of a row are one
// block) by the same rule as the activation quantizer, so the output is the next
// GEMM's A and sfA. A gate wave (wn = 0, 1) and the up wave with the same lanes
// (wn + 2) hold gate and up of the same 64 x 64 positions; each finishes one 32-row
// half of them, so all eight waves share the work:
//   1. the gate wave passes the gate values of rows 32..63 to its up wave, which
//      passes the up values of rows 0..31 back, through LDS (the stages are free);
//   2. each wave forms h = g / (1 + e^-g) * u in fp32 for its 32 x 64 values and each
//      row's max |h| over them; the two waves that share a row's 128 columns combine
//      theirs through LDS;
//   3. codes of h * 2^-e go to an LDS tile, the scale 2^e straight to sf;
//   4. all threads store the tile's produced rows with 16-byte stores.
template <class Cfg, int KIND>
__device__ __forceinline__ void pipe_store_swiglu(const Problem& p, const TileView& v, int expert,
                                                  int valid_rows,
                                                  v16f (&acc)[Cfg::TM][Cfg::TN],
                                                  const SwigluOut& out) {
  static_assert(Cfg::BM == 128 && Cfg::BN == 256, "gate and up halves of 128 columns");
  constexpr int TN = Cfg::TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int r32 = lane & 31, g = lane >> 5;
  const bool up = wn >= 2;
  const int ih = up ? 1 : 0;  // the 32-row half (tile row) this wave finishes
  const int slot = wm * 2 + (wn & 1);
  float* xch = (float*)((slot < 2 ? pipe_stage0 : pipe_stage1) + (slot & 1) * 16384);
  float* give = xch + (up ? 0 : 2048);  // up values of half 0 | gate values of half 1
  const float* take = xch + (up ? 2048 : 0);
  float* rmax_lds = (float*)pipe_scale;  // [wm * 2 + (wn & 1)][64 rows]
  uint8_t* codes_lds = pipe_stage2;      // [128 rows][128 columns]
  // (selects, not acc[ih]: a run-time index would move acc out of registers)
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) give[(j * 16 + e) * 64 + lane] = up ? acc[0][j][e] : acc[1][j][e];
  __syncthreads();
  float hv[TN][16];
  float rm = 0.f;
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float mine = up ? acc[1][j][e] : acc[0][j][e];
      const float other = take[(j * 16 + e) * 64 + lane];
      const float gt = up ? other : mine, u = up ? mine : other;
      // g / (1 + e^-g) as g * rcp(1 + e^-g): 1 ulp reciprocal, no division sequence
      const float h = gt * __builtin_amdgcn_rcpf(1.f + expf(-gt)) * u;
      hv[j][e] = h;
      rm = fmaxf(rm, fabsf(h));
    }
  rm = fmaxf(rm, __shfl_xor(rm, 32, 64));  // lanes r32 and r32 + 32 share a row
  if (g == 0) rmax_lds[slot * 64 + ih * 32 + r32] = rm;
  __syncthreads();
  {
    const int rl = wm * 64 + ih * 32 + r32;  // row within the tile
    const float m = fmaxf(rmax_lds[(wm * 2) * 64 + ih * 32 + r32],
                          rmax_lds[(wm * 2 + 1) * 64 + ih * 32 + r32]);
    const int e = quant_scale_exp(m);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(uint32_t*)(codes_lds + rl * 128 + (wn & 1) * 64 + j * 32 + 8 * q + 4 * g) =
            quant_e4m3fn_x4(ldexpf(hv[j][4 * q], -e), ldexpf(hv[j][4 * q + 1], -e),
                            ldexpf(hv[j][4 * q + 2], -e), ldexpf(hv[j][4 * q + 3], -e));
    if ((wn & 1) == 0 && g == 0) {
      const int64_t row = v.m0 + rl;
      bool ok = row < (int64_t)valid_rows;
      if (KIND == kContiguous && ok) ok = p.m_indices[row] == expert;
      if (ok) out.sf[row * (out.I / 128) + v.n0 / 128] = ldexpf(1.f, e);
    }
  }
  __syncthreads();
#pragma unroll
  for (int c = tid; c < 128 * 8; c += Cfg::NT) {
    const int rl = c >> 3, ch = c & 7;
    const int64_t row = v.m0 + rl;
    bool ok = row < (int64_t)valid_rows;
    if (KIND == kContiguous && ok) ok = p.m_indices[row] == expert;
    if (ok)
      *(uint4*)(out.codes + row * out.I + v.n0 + ch * 16) = *(const uint4*)(codes_lds + rl * 128 + ch * 16);
  }
  __syncthreads();  // the LDS is free again (the contiguous layout may run another pass)
}

template <class Cfg, int KIND, bool SWIGLU = false, int LAY = 0>
__device__ __forceinline__ void pipe_tile(const Problem& p, const TileView& v, int expert,
                                          int valid_rows, uint32_t quarters = ~0u,
                                          SwigluOut sw = SwigluOut{}) {
  v16f acc[Cfg::TM][Cfg::TN];
  if constexpr (SWIGLU) {
    pipe_mainloop<Cfg>(p, v, 0, (int)(p.K / kKBlock), acc, quarters, sw.I - 128);
    pipe_store_swiglu<Cfg, KIND>(p, v, expert, valid_rows, acc, sw);
  } else {
    pipe_mainloop<Cfg, LAY>(p, v, 0, (int)(p.K / kKBlock), acc, quarters);
    pipe_store<Cfg, KIND>(p, v, expert, valid_rows, acc);
  }
}

// Masked layout: live tile `b` of the schedule that lists, expert by expert, the
// ceil(valid_e / BM) x tiles_n tiles of each expert (valid_e = masked_m[e] clamped to
// [0, M]). Workgroups are numbered in that order through xcd_tile_order, so each XCD
// gets an equal contiguous share of the live tiles; expert = -1 past the live count.
// Every lane of every wave computes the same values (wave-wide scans over 64
// experts at a time).
struct MaskedTile {
  int expert, valid, local;
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

template <int BM>
__device__ __forceinline__ MaskedTile masked_tile(const int32_t* masked_m, int G, int M,
                                                  int tiles_n, int b) {
  const int lane = threadIdx.x & 63;
  auto count = [&](int e, int& valid) {
    int v = e < G ? masked_m[e] : 0;
    v = v < 0 ? 0 : (v > M ? M : v);
    valid = v;
    return (v + BM - 1) / BM * tiles_n;
  };
  int live = 0;
  for (int e0 = 0; e0 < G; e0 += 64) {
    int valid;
    const int incl = wave_incl_scan(count(e0 + lane, valid), lane);
    live += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  }
  MaskedTile r{-1, 0, 0};
  if (b >= live) return r;
  const int t = xcd_tile_order(b, live);
  int base = 0;
  for (int e0 = 0; e0 < G; e0 += 64) {
    int valid;
    const int c = count(e0 + lane, valid);
    const int incl = wave_incl_scan(c, lane);
    const uint64_t hit = __ballot(c > 0 && base + incl - c <= t && t < base + incl);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      r.expert = __builtin_amdgcn_readfirstlane(e0 + l);
      r.valid = __builtin_amdgcn_readfirstlane(__shfl(valid, l, 64));
      r.local = __builtin_amdgcn_readfirstlane(t - base - __shfl(incl - c, l, 64));
      return r;
    }
    base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  }
  return r;
}

struct PipeArgs {
  Problem p;
  float* ws;           // split tail: [tile][part][BM * BN] fp32 partials
  uint32_t* counters;  // split tail: one per tile, zero between calls
  int32_t full_tiles;  // dense: tiles computed whole (the first of the tile order)
  int32_t parts;       // dense: K parts of each remaining tile
  int32_t items;       // work items: dense full tiles + split parts, or the grid's tiles
  SwigluOut sw;        // fused SwiGLU epilogue (grouped layouts): outputs and I
};

// Dense tail tile: K-blocks [kb_lo, kb_hi) of tile `tt` (index among the split
// tiles), part `part` of `parts`. Each part writes its fp32 tile with device-scope
// stores and counts its arrival; the last part to arrive adds the parts in part
// order -- a fixed order, so the result is deterministic -- and stores bf16.
template <class Cfg, int LAY>
__device__ __forceinline__ void pipe_split_tile(const PipeArgs& a, const TileView& v, int tt,
                                                int part, int kb_lo, int kb_hi) {
  constexpr int TM = Cfg::TM, TN = Cfg::TN, BMN = Cfg::BM * Cfg::BN;
  v16f acc[TM][TN];
  pipe_mainloop<Cfg, LAY>(a.p, v, kb_lo, kb_hi, acc);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      a.ws + (int64_t)tt * a.parts * BMN, 0, 0x7FFFFFFF, 0x00020000);
  constexpr int kSc1 = 16;  // device scope: the parts run on different XCDs
  auto off = [&](int pt, int i, int j, int q) {
    return (uint32_t)(pt * BMN * 4 + ((((wave * TM + i) * TN + j) * 4 + q) * 64 + lane) * 16);
  };
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_raw_buffer_store_b128(
            v4u{__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                __float_as_uint(acc[i][j][4 * q + 2]), __float_as_uint(acc[i][j][4 * q + 3])},
            ws, off(part, i, j, q), 0, kSc1);
  if (!splitk_arrive(&a.counters[tt], (uint32_t)a.parts)) return;
  v16f sum[TM][TN];
  for (int pt = 0; pt < a.parts; ++pt) {
    v16f x[TM][TN];
    if (pt == part) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) x[i][j] = acc[i][j];
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4u u = __builtin_amdgcn_raw_buffer_load_b128(ws, off(pt, i, j, q), 0, kSc1);
            x[i][j][4 * q] = __uint_as_float(u[0]);
            x[i][j][4 * q + 1] = __uint_as_float(u[1]);
            x[i][j][4 * q + 2] = __uint_as_float(u[2]);
            x[i][j][4 * q + 3] = __uint_as_float(u[3]);
          }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (pt == 0) {
          sum[i][j] = x[i][j];
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) sum[i][j][e] += x[i][j][e];
        }
      }
  }
  if (tid == 0)
    __hip_atomic_store(&a.counters[tt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  pipe_store<Cfg, kDense>(a.p, v, 0, (int)a.p.M, sum);
}

// One work item: a tile (or, dense, a K part of a tail tile). `item` plays the role
// of the workgroup index in the tile order: item i runs on XCD i % 8.
// SWIGLU (grouped layouts, 128x256 tiles): B is [gate; up] with 2 * sw.I rows per
// expert, tile tn covers gate columns 128 tn.. and the matching up columns, and the
// fused epilogue writes quantized h instead of bf16 C.
template <class Cfg, int KIND, bool SWIGLU, int LAY>
__device__ __forceinline__ void pipe_item(const PipeArgs& args, int item) {
  static_assert(LAY == 0 || (KIND == kDense && !SWIGLU), "other layouts: dense GEMM only");
  static_assert(!SWIGLU || KIND != kDense, "the fused epilogue is for the grouped layouts");
  constexpr int NSTEP = SWIGLU ? 128 : Cfg::BN;  // columns between consecutive N-tiles
  const Problem& p = args.p;
  if (KIND == kDense && item >= args.full_tiles) {
    const int h = item - args.full_tiles;
    const int tt = h / args.parts, part = h - tt * args.parts;
    int tm, tn;
    grouped_tile<Cfg::GROUP_M>(args.full_tiles + tt, p.tiles_m, p.tiles_n, tm, tn);
    const int KB = (int)(p.K / kKBlock);
    TileView v;
    v.m0 = (int64_t)tm * Cfg::BM;
    v.n0 = (int64_t)tn * Cfg::BN;
    v.A = p.A;
    v.sfA = p.sfA;
    v.C = p.C;
    v.rows = p.M;
    v.B = p.B;
    v.sfB = p.sfB;
    pipe_split_tile<Cfg, LAY>(args, v, tt, part, part * KB / args.parts,
                              (part + 1) * KB / args.parts);
    return;
  }
  const int NB = (int)((p.N + kKBlock - 1) / kKBlock);
  const int KB = (int)(p.K / kKBlock);
  TileView v;
  int tm, tn;
  if (KIND == kMasked) {
    // only the live tiles are dealt out: the grid covers every expert at full
    // height, the workgroups past the live count leave at once
    const MaskedTile mt = masked_tile<Cfg::BM>(p.masked_m, p.G, (int)p.M, p.tiles_n, item);
    if (mt.expert < 0) return;
    const int e = mt.expert, valid = mt.valid;
    grouped_tile<Cfg::GROUP_M>(mt.local, (valid + Cfg::BM - 1) / Cfg::BM, p.tiles_n, tm, tn);
    v.m0 = (int64_t)tm * Cfg::BM;
    v.n0 = (int64_t)tn * NSTEP;
    v.A = p.A + (int64_t)e * p.M * p.K;
    v.sfA = p.sfA + (int64_t)e * p.M * sfa_row_bytes(KB, p.sfa_packed);
    v.C = p.C + (int64_t)e * p.M * p.N;
    v.B = p.B + (int64_t)e * p.N * p.K;
    v.sfB = p.sfB + (int64_t)e * NB * KB;
    v.rows = valid;  // rows past masked_m are never read
    SwigluOut sw = args.sw;  // this expert's rows of the fused epilogue's outputs
    sw.codes += (int64_t)e * p.M * sw.I;
    sw.sf += (int64_t)e * p.M * (sw.I / 128);
    pipe_tile<Cfg, KIND, SWIGLU>(p, v, e, valid, ~0u, sw);
    return;
  }
  const int t = xcd_tile_order(item, KIND == kDense ? args.full_tiles : args.items);
  grouped_tile<Cfg::GROUP_M>(t, p.tiles_m, p.tiles_n, tm, tn);
  v.m0 = (int64_t)tm * Cfg::BM;
  v.n0 = (int64_t)tn * NSTEP;
  v.A = p.A;
  v.sfA = p.sfA;
  v.C = p.C;
  v.rows = p.M;
  if (KIND == kDense) {
    v.B = p.B;
    v.sfB = p.sfB;
    pipe_tile<Cfg, KIND, false, LAY>(p, v, 0, (int)p.M);
    return;
  }
  // contiguous: one pass per distinct expert id among the tile's rows, in
  // increasing id order (one pass when segments are BM-aligned). s_quarter[q] records
  // that 32-row quarter q holds a row of the current expert; a wave skips the MFMAs
  // of a quarter that holds none (padding, or another expert's rows).
  __shared__ int s_next;
  __shared__ int s_quarter[Cfg::BM / 32];
  if (threadIdx.x < Cfg::BM / 32) s_quarter[threadIdx.x] = -1;
  int id = -1;
  if (threadIdx.x < Cfg::BM) {
    const int64_t row = v.m0 + threadIdx.x;
    if (row < p.M) id = p.m_indices[row];
  }
  int prev = -1;
  for (;;) {
    if (threadIdx.x == 0) s_next = 0x7FFFFFFF;
    __syncthreads();
    if (id > prev && id < p.G) atomicMin(&s_next, id);
    __syncthreads();
    const int e = __builtin_amdgcn_readfirstlane(s_next);
    if (id == e) s_quarter[threadIdx.x >> 5] = e;
    __syncthreads();
    if (e == 0x7FFFFFFF) break;
    uint32_t quarters = 0;
#pragma unroll
    for (int q = 0; q < Cfg::BM / 32; ++q)
      quarters |= (uint32_t)(__builtin_amdgcn_readfirstlane(s_quarter[q]) == e) << q;
    v.B = p.B + (int64_t)e * p.N * p.K;
    v.sfB = p.sfB + (int64_t)e * NB * KB;
    pipe_tile<Cfg, KIND, SWIGLU>(p, v, e, (int)p.M, quarters, args.sw);
    prev = e;
  }
}

// Persistent: at most one workgroup per CU, each taking items blockIdx.x,
// blockIdx.x + gridDim.x, ... (gridDim.x is the item count, or a multiple of 8 when
// smaller, so item i stays on XCD i % 8). A tile's stores drain while the next
// tile's first DMAs are in flight, and no workgroup is dispatched per tile.
template <class Cfg, int KIND, bool SWIGLU = false, int LAY = 0>
__global__ void __launch_bounds__(Cfg::NT) pipe_kernel(PipeArgs args) {
  for (int item = blockIdx.x; item < args.items; item += gridDim.x)
    pipe_item<Cfg, KIND, SWIGLU, LAY>(args, item);
}

}  // namespace dg

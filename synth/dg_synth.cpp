// dg_synth.cpp -- seeded synthetic inputs for the FP8 block-scaled GEMM workloads.
//
// This module only makes inputs. Both the GPU library's tests and benchmark and the
// CPU oracle's tests consume the bytes it writes; it holds none of the GEMM's
// arithmetic and shares no code with the GPU library or the oracle.
//
// Recipe (the workload definitions; the pages give shapes but no data):
//   * values: N(0, 1) in fp32, drawn by an explicit Box-Muller transform from
//     std::mt19937_64 (whose output sequence the C++ standard fixes). A matrix is
//     drawn in chunks of 128 rows; chunk j of stream `seed` uses the generator seeded
//     with seed * 2^20 + j, so chunks can be drawn in parallel and any chunk can be
//     redrawn alone.
//   * operands: each block (1x128 of an activation row, 128x128 of a weight matrix,
//     clipped at the row tail) gets the power-of-two scale s = 2^e with e the least
//     integer such that amax <= 448 * 2^e (s = 1 for an all-zero block), and every
//     value becomes the e4m3fn code nearest to x / s, ties to even. This is input
//     preparation; the oracle has its own quantizer (a plain search) and a CPU test
//     checks the two agree code for code.
//   * MoE routing: Zipf(s) over the non-empty experts' ranks by inverse CDF; ranks
//     map to expert ids through a seeded Fisher-Yates permutation.
//   * masked counts: uniform integers by rejection sampling.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <random>
#include <vector>

namespace {

constexpr int64_t kChunkRows = 128;

inline double unit_open_closed(uint64_t x) {  // (0, 1]
  return (double)((x >> 11) + 1) * 0x1.0p-53;
}
inline double unit_closed_open(uint64_t x) {  // [0, 1)
  return (double)(x >> 11) * 0x1.0p-53;
}

// n normals from one generator, Box-Muller pairs (cos then sin).
void fill_normals(std::mt19937_64& g, float* out, int64_t n) {
  const double two_pi = 6.283185307179586476925286766559;
  int64_t i = 0;
  while (i < n) {
    double u1 = unit_open_closed(g());
    double u2 = unit_closed_open(g());
    double r = std::sqrt(-2.0 * std::log(u1));
    out[i++] = (float)(r * std::cos(two_pi * u2));
    if (i < n) out[i++] = (float)(r * std::sin(two_pi * u2));
  }
}

uint64_t bounded(std::mt19937_64& g, uint64_t bound) {  // uniform in [0, bound)
  const uint64_t limit = (UINT64_MAX / bound) * bound;
  for (;;) {
    uint64_t x = g();
    if (x < limit) return x % bound;
  }
}

// Least e with amax <= 448 * 2^e, read off the fp32 exponent and mantissa.
// 448 = 1.75 * 2^8: with amax = f * 2^ex, f in [0.5, 1), the bound holds at
// e = ex - 9 exactly when 2f <= 1.75, otherwise at e = ex - 8.
inline int scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ex;
  float fr = std::frexp(amax, &ex);
  return (2.0f * fr <= 1.75f) ? ex - 9 : ex - 8;
}

// e4m3fn code of y, |y| <= 448, round to nearest even, sign of zero kept.
inline uint8_t to_e4m3fn(float y) {
  uint32_t b;
  std::memcpy(&b, &y, 4);
  const uint8_t sign = (uint8_t)((b >> 24) & 0x80u);
  const uint32_t a = b & 0x7FFFFFFFu;
  uint8_t mag;
  if (a < 0x3C800000u) {  // |y| < 2^-6: fixed grid of 2^-9
    float ay;
    std::memcpy(&ay, &a, 4);
    mag = (uint8_t)std::nearbyint(ay * 512.0f);
  } else {  // keep 3 of the 23 mantissa bits, RNE, re-bias exponent 127 -> 7
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    mag = (uint8_t)(r - ((127u - 7u) << 3));
  }
  return (uint8_t)(sign | mag);
}

void quantize_rows(const float* x, int64_t R, int64_t C, int64_t br, int64_t bc,
                   uint8_t* codes, float* scales) {
  const int64_t RB = (R + br - 1) / br, CB = C / bc;
  for (int64_t rb = 0; rb < RB; ++rb) {
    const int64_t r0 = rb * br, r1 = std::min(R, r0 + br);
    for (int64_t cb = 0; cb < CB; ++cb) {
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = cb * bc; c < (cb + 1) * bc; ++c)
          amax = std::max(amax, std::fabs(x[r * C + c]));
      const int e = scale_exp(amax);
      scales[rb * CB + cb] = std::ldexp(1.0f, e);
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = cb * bc; c < (cb + 1) * bc; ++c)
          codes[r * C + c] = to_e4m3fn(std::ldexp(x[r * C + c], -e));
    }
  }
}

}  // namespace

extern "C" {

// mt19937_64 output number `index` (1-based) for `seed`; used to check the engine.
uint64_t dgs_mt_output(uint64_t seed, int64_t index) {
  std::mt19937_64 g(seed);
  uint64_t x = 0;
  for (int64_t i = 0; i < index; ++i) x = g();
  return x;
}

// R x C fp32 N(0,1) values, chunked streams (see header).
void dgs_normal_rows(uint64_t seed, int64_t R, int64_t C, float* out) {
  const int64_t chunks = (R + kChunkRows - 1) / kChunkRows;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < chunks; ++j) {
    std::mt19937_64 g(seed * (1ull << 20) + (uint64_t)j);
    const int64_t r0 = j * kChunkRows, r1 = std::min(R, r0 + kChunkRows);
    fill_normals(g, out + r0 * C, (r1 - r0) * C);
  }
}

// Block quantizer for an R x C fp32 matrix; blocks br x bc, C % bc == 0.
void dgs_quantize(const float* x, int64_t R, int64_t C, int64_t br, int64_t bc,
                  uint8_t* codes, float* scales) {
  const int64_t RB = (R + br - 1) / br, CB = C / bc;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t rb = 0; rb < RB; ++rb) {
    const int64_t r0 = rb * br, r1 = std::min(R, r0 + br);
    quantize_rows(x + r0 * C, r1 - r0, C, br, bc, codes + r0 * C, scales + rb * CB);
  }
}

// Draw and quantize an R x C operand in one pass, 128 rows at a time, without
// holding the fp32 matrix (the values are those of dgs_normal_rows). br must be 1
// or 128.
void dgs_make_operand(uint64_t seed, int64_t R, int64_t C, int64_t br, int64_t bc,
                      uint8_t* codes, float* scales) {
  const int64_t chunks = (R + kChunkRows - 1) / kChunkRows, CB = C / bc;
#pragma omp parallel
  {
    std::vector<float> buf((size_t)(kChunkRows * C));
#pragma omp for schedule(dynamic, 1)
    for (int64_t j = 0; j < chunks; ++j) {
      std::mt19937_64 g(seed * (1ull << 20) + (uint64_t)j);
      const int64_t r0 = j * kChunkRows, r1 = std::min(R, r0 + kChunkRows);
      fill_normals(g, buf.data(), (r1 - r0) * C);
      quantize_rows(buf.data(), r1 - r0, C, br, bc, codes + r0 * C,
                    scales + (r0 / br) * CB);
    }
  }
}

// Fisher-Yates permutation of 0..n-1.
void dgs_permutation(uint64_t seed, int32_t n, int32_t* perm) {
  std::mt19937_64 g(seed);
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)bounded(g, (uint64_t)i + 1);
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
}

// Zipf(s) rank counts over ranks 1..n_ranks for n_tokens draws (inverse CDF on the
// fp64 cumulative weights r^-s). counts[r-1] receives rank r's count.
void dgs_zipf_counts(uint64_t seed, int64_t n_tokens, int32_t n_ranks, double s,
                     int32_t* counts) {
  std::vector<double> cum((size_t)n_ranks);
  double total = 0.0;
  for (int32_t r = 1; r <= n_ranks; ++r) {
    total += std::pow((double)r, -s);
    cum[(size_t)r - 1] = total;
  }
  for (int32_t r = 0; r < n_ranks; ++r) counts[r] = 0;
  std::mt19937_64 g(seed);
  for (int64_t t = 0; t < n_tokens; ++t) {
    const double u = unit_closed_open(g()) * total;
    int32_t r = 0;
    while (r < n_ranks - 1 && u >= cum[(size_t)r]) ++r;
    ++counts[r];
  }
}

// n uniform integers in [0, bound).
void dgs_uniform_ints(uint64_t seed, int64_t n, int64_t bound, int32_t* out) {
  std::mt19937_64 g(seed);
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)bounded(g, (uint64_t)bound);
}

}  // extern "C"

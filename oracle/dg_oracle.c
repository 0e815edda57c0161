/*
 * dg_oracle.c -- CPU oracle for the FP8 block-scaled GEMM (dense NT, MoE grouped
 * contiguous, MoE grouped masked).
 *
 * TEST INFRASTRUCTURE. This file is the yardstick the GPU path is checked against.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it. It shares no source, header, table or helper with the HIP library: every
 * format rule it needs (e4m3fn decode, bf16 rounding, power-of-two scale choice) is
 * written out here again from the format definitions.
 *
 * What it computes, and where the pages say so:
 *   - DeepGEMM launch article (deepseek.csdn.net), section 1.2 "precision
 *     safeguards": each block of an operand carries its own scaling factor, and the
 *     FP8 products are promoted to FP32 and accumulated a second time. The result
 *     both levels approximate is the plain block-scaled product
 *         C[m][n] = sum_kb sfA[m][kb] * sfB[n/128][kb] * sum_{k in block kb} a(m,k) b(n,k)
 *     with a(), b() the exact values of the e4m3fn codes. This oracle computes that
 *     sum in fp64, and rounds it once to bf16 (round to nearest, ties to even).
 *   - DeepGEMM project page (aiproducthub.cn), sections "quick start" (call shape
 *     fp8_gemm_nt(a, b, c, a_sf, b_sf), caller-owned output) and "technical
 *     implementation" (MoE grouping along M with N and K fixed; several experts'
 *     tokens concatenated into one contiguous M).
 *   - DeepGEMM launch article, section 4.2 "advanced tuning", and the DeepGEMM
 *     library news page (youleyou.com), "performance": a masked grouped layout for
 *     MoE, one fixed-capacity slab of rows per expert with a valid-row count.
 *
 * Readings taken where the pages are silent (block sizes 1x128 for A and 128x128 for
 * B, K-block 128, OCP e4m3fn with max 448, bf16 output, -1 marks a pad row, rows at
 * or past masked_m[e] are not produced) are the workload definitions'; they are
 * listed with the rest of the design notes.
 *
 * Exactness: every finite e4m3fn value is an integer multiple of 2^-9 below 2^18 in
 * magnitude, so each product is a multiple of 2^-18 below 2^36 units and a 128-term
 * block sum stays below 2^43 units: fp64 holds every block partial exactly. With
 * power-of-two scales the scaled block term is exact too; the only rounding before
 * the final bf16 step is the fp64 sum over K-blocks.
 *
 * Precision: fp64 throughout. Plain loops, no blocking, no SIMD intrinsics. OpenMP
 * only splits independent output rows across host threads.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DGO_KBLOCK 128

/* ------------------------------------------------------------------ formats */

/* Exact value of an OCP e4m3fn code (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; no infinities; exponent 15 with mantissa 7 is NaN). */
double dgo_e4m3fn_value(uint8_t code) {
  int sign = code >> 7;
  int E = (code >> 3) & 15;
  int F = code & 7;
  double mag;
  if (E == 15 && F == 7) return NAN;
  if (E == 0)
    mag = ldexp((double)F, -9);          /* subnormal: (F/8) * 2^(1-7)    */
  else
    mag = ldexp((double)(8 + F), E - 10); /* normal: (1 + F/8) * 2^(E-7) */
  return sign ? -mag : mag;
}

/* bf16 bit pattern of v, rounded to nearest with ties to even, straight from fp64
 * (one rounding, no fp32 intermediate). bf16 keeps 8 significant bits, the fp32
 * exponent range, subnormals down to 2^-133; overflow goes to infinity. */
uint16_t dgo_bf16_rne(double v) {
  uint16_t sign;
  double a, m, r, res;
  int e, q;
  float f;
  uint32_t bits;
  if (isnan(v)) return (uint16_t)0x7FC0;
  sign = signbit(v) ? (uint16_t)0x8000 : (uint16_t)0;
  a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  frexp(a, &e);           /* a = f * 2^e with f in [0.5, 1): leading bit 2^(e-1) */
  q = (e - 1) - 7;        /* weight of the 8th significant bit                   */
  if (q < -133) q = -133; /* subnormal range: fixed quantum 2^-133               */
  m = ldexp(a, -q);       /* exact: a in units of the quantum                    */
  r = nearbyint(m);       /* default rounding mode: nearest, ties to even        */
  res = ldexp(r, q);
  if (res > ldexp(255.0, 120)) return (uint16_t)(sign | 0x7F80); /* > max finite */
  f = (float)res;         /* exact: res has <= 8 significant bits in fp32 range  */
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

void dgo_bf16_rne_array(const double* in, uint16_t* out, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = dgo_bf16_rne(in[i]);
}

/* ------------------------------------------------------------------ GEMM */

/* One output element of the block-scaled product: a_row is K codes, b_row is K
 * codes, sa is the row's KB scales, sb the KB scales of the row's 128-block of B. */
static double dgo_scaled_dot(const uint8_t* a_row, const uint8_t* b_row,
                             const float* sa, const float* sb, int64_t K,
                             const double* val) {
  int64_t KB = K / DGO_KBLOCK, kb, k;
  double acc = 0.0;
  for (kb = 0; kb < KB; ++kb) {
    double block = 0.0; /* exact, see header */
    for (k = kb * DGO_KBLOCK; k < (kb + 1) * DGO_KBLOCK; ++k)
      block += val[a_row[k]] * val[b_row[k]];
    acc += block * (double)sa[kb] * (double)sb[kb];
  }
  return acc;
}

static void dgo_value_table(double* val) {
  int c;
  for (c = 0; c < 256; ++c) val[c] = dgo_e4m3fn_value((uint8_t)c);
}

/* Dense NT: A [M][K] codes, B [N][K] codes, sfA [M][K/128], sfB [ceil(N/128)][K/128].
 * Writes the fp64 value of every C[m][n] into C_exact [M][N]. */
void dgo_gemm_nt(const uint8_t* A, const uint8_t* B, const float* sfA, const float* sfB,
                 int64_t M, int64_t N, int64_t K, double* C_exact) {
  double val[256];
  int64_t KB = K / DGO_KBLOCK, m;
  dgo_value_table(val);
#pragma omp parallel for schedule(dynamic, 1)
  for (m = 0; m < M; ++m) {
    int64_t n;
    for (n = 0; n < N; ++n)
      C_exact[m * N + n] = dgo_scaled_dot(A + m * K, B + n * K, sfA + m * KB,
                                          sfB + (n / DGO_KBLOCK) * KB, K, val);
  }
}

/* Dense GEMM in the other memory layouts (DeepGEMM project page, aiproducthub.cn,
 * "core features": NT/TN/NN/TT layouts of one GEMM family). C = op(A) op(B) with the
 * same block scaling: a(m, k) is A[m][k] (A stored [M][K]) or, with a_t, A[k][m] (A
 * stored [K][M]); b(n, k) is B[n][k] (B stored [N][K]) or, with b_n, B[k][n] (B stored
 * [K][N]). sfA [M][K/128] and sfB [ceil(N/128)][K/128] as for NT. Written with the
 * strided indexing spelled out; every block sum is exact as in dgo_scaled_dot. */
void dgo_gemm_layout(const uint8_t* A, const uint8_t* B, const float* sfA, const float* sfB,
                     int64_t M, int64_t N, int64_t K, int a_t, int b_n, double* C_exact) {
  double val[256];
  int64_t KB = K / DGO_KBLOCK, m;
  dgo_value_table(val);
#pragma omp parallel for schedule(dynamic, 1)
  for (m = 0; m < M; ++m) {
    int64_t n, kb, k;
    for (n = 0; n < N; ++n) {
      double acc = 0.0;
      for (kb = 0; kb < KB; ++kb) {
        double block = 0.0;
        for (k = kb * DGO_KBLOCK; k < (kb + 1) * DGO_KBLOCK; ++k) {
          uint8_t a = a_t ? A[k * M + m] : A[m * K + k];
          uint8_t b = b_n ? B[k * N + n] : B[n * K + k];
          block += val[a] * val[b];
        }
        acc += block * (double)sfA[m * KB + kb] * (double)sfB[(n / DGO_KBLOCK) * KB + kb];
      }
      C_exact[m * N + n] = acc;
    }
  }
}

/* Dense NT at chosen output positions (m_idx[i], n_idx[i]), i < count. */
void dgo_gemm_nt_at(const uint8_t* A, const uint8_t* B, const float* sfA, const float* sfB,
                    int64_t M, int64_t N, int64_t K, const int64_t* m_idx,
                    const int64_t* n_idx, int64_t count, double* out) {
  double val[256];
  int64_t KB = K / DGO_KBLOCK, i;
  (void)M;
  (void)N;
  dgo_value_table(val);
#pragma omp parallel for schedule(dynamic, 64)
  for (i = 0; i < count; ++i) {
    int64_t m = m_idx[i], n = n_idx[i];
    out[i] = dgo_scaled_dot(A + m * K, B + n * K, sfA + m * KB,
                            sfB + (n / DGO_KBLOCK) * KB, K, val);
  }
}

/* MoE grouped, contiguous layout. A [M_total][K], B [G][N][K], sfA [M_total][K/128],
 * sfB [G][ceil(N/128)][K/128], m_indices [M_total]. Row r belongs to expert
 * m_indices[r]; any id outside [0, G) (the pad marker is -1) marks a row that is
 * not produced: produced[r] = 0 and C_exact's row r is left as it was. */
void dgo_grouped_contiguous(const uint8_t* A, const uint8_t* B, const float* sfA,
                            const float* sfB, const int32_t* m_indices, int64_t M_total,
                            int64_t N, int64_t K, int32_t G, double* C_exact,
                            uint8_t* produced) {
  double val[256];
  int64_t KB = K / DGO_KBLOCK, NB = (N + DGO_KBLOCK - 1) / DGO_KBLOCK, r;
  dgo_value_table(val);
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < M_total; ++r) {
    int32_t e = m_indices[r];
    int64_t n;
    if (e < 0 || e >= G) {
      produced[r] = 0;
      continue;
    }
    produced[r] = 1;
    for (n = 0; n < N; ++n)
      C_exact[r * N + n] = dgo_scaled_dot(
          A + r * K, B + ((int64_t)e * N + n) * K, sfA + r * KB,
          sfB + ((int64_t)e * NB + n / DGO_KBLOCK) * KB, K, val);
  }
}

/* Contiguous layout at chosen positions (r_idx[i], n_idx[i]); rows whose id is out
 * of [0, G) give NaN (not produced). */
void dgo_grouped_contiguous_at(const uint8_t* A, const uint8_t* B, const float* sfA,
                               const float* sfB, const int32_t* m_indices, int64_t M_total,
                               int64_t N, int64_t K, int32_t G, const int64_t* r_idx,
                               const int64_t* n_idx, int64_t count, double* out) {
  double val[256];
  int64_t KB = K / DGO_KBLOCK, NB = (N + DGO_KBLOCK - 1) / DGO_KBLOCK, i;
  (void)M_total;
  dgo_value_table(val);
#pragma omp parallel for schedule(dynamic, 64)
  for (i = 0; i < count; ++i) {
    int64_t r = r_idx[i], n = n_idx[i];
    int32_t e = m_indices[r];
    if (e < 0 || e >= G) {
      out[i] = NAN;
      continue;
    }
    out[i] = dgo_scaled_dot(A + r * K, B + ((int64_t)e * N + n) * K, sfA + r * KB,
                            sfB + ((int64_t)e * NB + n / DGO_KBLOCK) * KB, K, val);
  }
}

/* MoE grouped, masked layout. A [G][M_max][K], B [G][N][K], sfA [G][M_max][K/128],
 * sfB [G][ceil(N/128)][K/128], masked_m [G]. Expert e produces its rows
 * m < masked_m[e] (the count taken within [0, M_max]); the other rows are not
 * produced: produced[e*M_max + m] = 0 and C_exact is left as it was there. */
void dgo_grouped_masked(const uint8_t* A, const uint8_t* B, const float* sfA,
                        const float* sfB, const int32_t* masked_m, int32_t G, int64_t M_max,
                        int64_t N, int64_t K, double* C_exact, uint8_t* produced) {
  double val[256];
  int64_t KB = K / DGO_KBLOCK, NB = (N + DGO_KBLOCK - 1) / DGO_KBLOCK, row;
  dgo_value_table(val);
#pragma omp parallel for schedule(dynamic, 1)
  for (row = 0; row < (int64_t)G * M_max; ++row) {
    int64_t e = row / M_max, m = row % M_max, n;
    int64_t valid = masked_m[e];
    if (valid < 0) valid = 0;
    if (valid > M_max) valid = M_max;
    if (m >= valid) {
      produced[row] = 0;
      continue;
    }
    produced[row] = 1;
    for (n = 0; n < N; ++n)
      C_exact[row * N + n] = dgo_scaled_dot(
          A + row * K, B + (e * N + n) * K, sfA + row * KB,
          sfB + (e * NB + n / DGO_KBLOCK) * KB, K, val);
  }
}

/* Masked layout at chosen positions (e_idx[i], m_idx[i], n_idx[i]); rows that are
 * not produced give NaN. */
void dgo_grouped_masked_at(const uint8_t* A, const uint8_t* B, const float* sfA,
                           const float* sfB, const int32_t* masked_m, int32_t G,
                           int64_t M_max, int64_t N, int64_t K, const int64_t* e_idx,
                           const int64_t* m_idx, const int64_t* n_idx, int64_t count,
                           double* out) {
  double val[256];
  int64_t KB = K / DGO_KBLOCK, NB = (N + DGO_KBLOCK - 1) / DGO_KBLOCK, i;
  (void)G;
  dgo_value_table(val);
#pragma omp parallel for schedule(dynamic, 64)
  for (i = 0; i < count; ++i) {
    int64_t e = e_idx[i], m = m_idx[i], n = n_idx[i], row = e * M_max + m;
    int64_t valid = masked_m[e];
    if (valid < 0) valid = 0;
    if (valid > M_max) valid = M_max;
    if (m >= valid) {
      out[i] = NAN;
      continue;
    }
    out[i] = dgo_scaled_dot(A + row * K, B + (e * N + n) * K, sfA + row * KB,
                            sfB + (e * NB + n / DGO_KBLOCK) * KB, K, val);
  }
}

/* ------------------------------------------------------------------ quantizer */
/*
 * Block quantizer (the step that makes the operands; launch article section 1.2:
 * each block gets a scale chosen so that its values do not overflow the FP8 range).
 * Reading: the scale is the power of two s = 2^e with e the least integer such that
 * amax <= 448 * 2^e (amax = largest |x| in the block; amax = 0 gives s = 1), and each
 * code is the e4m3fn value nearest to x / s, ties to the even code, zero keeping the
 * sign of x. Written as a search so that it can be read off the definition: it is
 * the oracle for any faster quantizer, not a fast one itself.
 */

/* Least e with amax <= 448 * 2^e. */
int dgo_scale_exponent(double amax) {
  int e = 0;
  if (!(amax > 0.0)) return 0;
  while (amax > ldexp(448.0, e)) ++e;
  while (amax <= ldexp(448.0, e - 1)) --e;
  return e;
}

/* Nearest e4m3fn code to y (|y| <= 448), ties to the even code. */
uint8_t dgo_e4m3fn_nearest(double y) {
  double a = fabs(y), best_d = INFINITY;
  int c, best = 0;
  for (c = 0; c <= 126; ++c) { /* every finite non-negative code, in value order */
    double d = fabs(a - dgo_e4m3fn_value((uint8_t)c));
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best_d = d;
      best = c;
    }
  }
  return (uint8_t)(signbit(y) ? (0x80 | best) : best);
}

/* x is R x C fp32 row-major; blocks are br rows x bc columns (the last block row
 * may be short). codes R x C; scales ceil(R/br) x (C/bc) fp32. C % bc == 0. */
void dgo_quantize_blocks(const float* x, int64_t R, int64_t C, int64_t br, int64_t bc,
                         uint8_t* codes, float* scales) {
  int64_t RB = (R + br - 1) / br, CB = C / bc, blk;
#pragma omp parallel for schedule(dynamic, 1)
  for (blk = 0; blk < RB * CB; ++blk) {
    int64_t rb = blk / CB, cb = blk % CB, r, c;
    int64_t r1 = (rb + 1) * br < R ? (rb + 1) * br : R;
    double amax = 0.0;
    int e;
    for (r = rb * br; r < r1; ++r)
      for (c = cb * bc; c < (cb + 1) * bc; ++c)
        if (fabs((double)x[r * C + c]) > amax) amax = fabs((double)x[r * C + c]);
    e = dgo_scale_exponent(amax);
    scales[rb * CB + cb] = (float)ldexp(1.0, e);
    for (r = rb * br; r < r1; ++r)
      for (c = cb * bc; c < (cb + 1) * bc; ++c)
        codes[r * C + c] = dgo_e4m3fn_nearest(ldexp((double)x[r * C + c], -e));
  }
}

/* ------------------------------------------------------------------ SwiGLU */
/*
 * The activation between an MoE layer's two grouped GEMMs (DeepGEMM project page,
 * aiproducthub.cn, "core features": Mega MoE fuses Linear1, SwiGLU and Linear2).
 * Reading: Linear1's output row holds the gate half in columns [0, I) and the up
 * half in [I, 2I); the activation is h[j] = silu(gate[j]) * up[j] with
 * silu(x) = x / (1 + exp(-x)), in fp64. gu is [rows][2I], h is [rows][I].
 */
void dgo_swiglu(const double* gu, int64_t rows, int64_t I, double* h) {
  int64_t r, j;
  for (r = 0; r < rows; ++r)
    for (j = 0; j < I; ++j) {
      double g = gu[r * 2 * I + j], u = gu[r * 2 * I + I + j];
      h[r * I + j] = g / (1.0 + exp(-g)) * u;
    }
}

/* ------------------------------------------------------------------ UE8M0 scales */
/*
 * Packed UE8M0 layout of the LHS scaling factors (DeepGEMM project page,
 * aiproducthub.cn, "technical implementation": an exponent-only packed layout for
 * the LHS scales to reduce memory traffic). Reading: each power-of-two scale 2^e is
 * stored as the unsigned byte e + 127 (the UE8M0 format: an 8-bit exponent, no sign,
 * no mantissa), four consecutive K-blocks per little-endian 32-bit word, rows padded
 * to whole words: byte j of word w of a row is K-block 4w + j. Written out: the byte
 * with value b means 2^(b - 127) (b = 255 is not a scale).
 */
void dgo_unpack_ue8m0(const uint32_t* packed, int64_t rows, int64_t KB, float* out) {
  int64_t words = (KB + 3) / 4, r, kb;
  for (r = 0; r < rows; ++r)
    for (kb = 0; kb < KB; ++kb) {
      uint32_t w = packed[r * words + kb / 4];
      unsigned b = (w >> (8 * (kb % 4))) & 0xFFu;
      out[r * KB + kb] = (float)ldexp(1.0, (int)b - 127);
    }
}

int dgo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

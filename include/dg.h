/*
 * dg.h -- C ABI of the MI355X (gfx950) FP8 block-scaled GEMM library (libdg.so).
 *
 * The operation: an FP8 GEMM where every operand block carries its own fp32
 * scaling factor and the FP8 products are promoted to FP32 for a second-level
 * accumulation across K-blocks (DeepGEMM launch article, deepseek.csdn.net,
 * section 1.2 "precision safeguards"). In the library's layouts:
 *
 *     C[m][n] = bf16_rne( sum_{kb < K/128} sfA[m][kb] * sfB[n/128][kb]
 *                         * sum_{k in [128kb, 128kb+128)} a(m,k) * b(n,k) )
 *
 * with a(), b() the values of OCP e4m3fn codes (max 448, no infinities).
 * Granularity: A is scaled per 1x128 (row, K-block), B per 128x128 block; K-block
 * 128 for both. The call shape follows the DeepGEMM project page (aiproducthub.cn),
 * "quick start": fp8_gemm_nt(a, b, c, a_sf, b_sf) and
 * m_grouped_fp8_gemm_nt_contiguous(...), the caller passing the output buffer. The
 * masked grouped form is the MoE interface of the launch article's section 4.2
 * "advanced tuning" (also the library news page, youleyou.com, "performance").
 *
 * Conventions shared by every call
 *  - Every pointer is DEVICE memory owned by the caller; the library never
 *    allocates, frees or keeps a user buffer. All matrices are row-major and
 *    dense (leading dimension = row length).
 *  - Library-owned memory: some calls use device buffers that the library
 *    allocates per (device, stream) the first time a call needs them (hipMalloc,
 *    and a hipMemsetAsync that zeroes the counters):
 *      - fp32 partial tiles and arrival counters, for calls that split K across
 *        workgroups (the M <= 64 kernels, and the last partial round of tiles of a
 *        larger dense GEMM);
 *      - transposed operand copies, for the NN / TN / TT calls.
 *    Calls on one stream share them in stream order; calls on different streams
 *    never share them. The buffers only grow. An outgrown buffer is retired, not
 *    freed: it stays allocated until dg_release_workspaces() or the end of the
 *    process, so a HIP graph captured before the growth still finds its buffers.
 *  - HIP graph capture: a call that needs no larger buffer allocates nothing, so a
 *    call may be captured once the same shape (or a larger one) has run on that
 *    stream outside capture. A call that would have to grow a buffer while its
 *    stream is capturing returns DG_ERR_CAPTURE and records nothing. A graph's
 *    launches use the capture stream's buffers: replay it on that stream, or
 *    otherwise keep its replays ordered with eager calls on that stream (two
 *    overlapping users of one counter set give wrong results).
 *  - A and B hold e4m3fn codes (1 byte). "NT": both are K-contiguous, B is [N][K].
 *  - C is bf16 (2 bytes), written with one round-to-nearest-even from the fp32
 *    accumulator. Only the output rows the call produces are written.
 *  - sfA, sfB are fp32. Any finite positive value works; with powers of two (the
 *    configured workloads) every scaling step is exact.
 *  - K % 128 == 0 (K > 0 when any output is produced), N % 16 == 0.
 *    A, B, C must be 16-byte aligned, sfA and sfB 4-byte aligned.
 *  - hip_stream is a hipStream_t (NULL = the default stream). The call only
 *    enqueues work and returns; device faults surface at the caller's next
 *    synchronisation. Calls on one stream run in order.
 *  - Results are bitwise deterministic for a given shape (no atomics touch C).
 *  - Errors: every argument check runs on the host before any HIP call and returns
 *    a status without touching the GPU; nothing is thrown across the ABI. A
 *    launch failure returns DG_ERR_LAUNCH. dg_last_error_detail() gives a
 *    thread-local message for the last failing call on the calling thread.
 *  - Zero-sized work (M, N or G*M_max == 0) returns DG_OK and launches nothing.
 *  - Environment: DG_PRINT_CONFIGS=1 prints the tile configuration chosen for each
 *    new (kind, shape) to stderr, and for the NN / TN / TT calls whether the operands
 *    are read in place or through a transposed copy (which uses a library-owned
 *    buffer); DG_FORCE_CONFIG=<name> overrides the choice (tuning only, see
 *    dg_config_name).
 */
#ifndef DG_H_
#define DG_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_status {
  DG_OK = 0,
  DG_ERR_NULL_POINTER = 1,      /* a required pointer is NULL                    */
  DG_ERR_BAD_SHAPE = 2,         /* negative size, K % 128 != 0, N % 16 != 0, G<1, */
                                /* or an unknown dg_dtype                         */
  DG_ERR_UNSUPPORTED_SHAPE = 3, /* valid but beyond what the kernels index       */
  DG_ERR_MISALIGNED = 4,        /* A/B/C not 16-byte or scales not 4-byte aligned */
  DG_ERR_NO_DEVICE = 5,         /* no usable gfx950 device                       */
  DG_ERR_LAUNCH = 6,            /* the kernel launch itself failed               */
  DG_ERR_CAPTURE = 7            /* the call would allocate while its stream is    */
                                /* being captured into a HIP graph                */
} dg_status;

/*
 * Dense NT GEMM (project page, "quick start": fp8_gemm_nt).
 *   A   e4m3fn [M][K]            sfA fp32 [M][K/128]
 *   B   e4m3fn [N][K]            sfB fp32 [ceil(N/128)][K/128]
 *   C   bf16   [M][N]            every element written
 */
dg_status dg_fp8_gemm_nt(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K,
                         void* hip_stream);

/*
 * dg_fp8_gemm_nt without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture (also before the shape has run eagerly),
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, results and
 * errors as dg_fp8_gemm_nt (bitwise the same output); the call allocates nothing and
 * records no memset. The split-K partials and arrival counters it needs live in one
 * fixed device array per GPU, part of the library's code object and held until the
 * process ends: at most 32 MiB of partials and 4096 counters, which covers every
 * shape the configuration table serves (a shape needing more returns
 * DG_ERR_UNSUPPORTED_SHAPE). Every call on a GPU shares that GPU's array and leaves
 * its counters at zero; calls that overlap in time on one GPU (on different streams,
 * or graph replays concurrent with eager calls) race and give wrong results.
 */
dg_status dg_fp8_gemm_nt_noalloc(const void* A, const void* B, void* C, const float* sfA,
                                 const float* sfB, int64_t M, int64_t N, int64_t K,
                                 void* hip_stream);

/*
 * The same dense GEMM in the other memory layouts of one GEMM family (project page,
 * "core features": NT / TN / NN / TT layouts, for forward, backward and inference):
 * C = op(A) op(B) with op = N (as stored) or T (transposed), i.e.
 *   dg_fp8_gemm_nn:  A e4m3fn [M][K],  B e4m3fn [K][N]
 *   dg_fp8_gemm_tn:  A e4m3fn [K][M],  B e4m3fn [K][N]
 *   dg_fp8_gemm_tt:  A e4m3fn [K][M],  B e4m3fn [N][K]
 * (dg_fp8_gemm_nt above is A [M][K], B [N][K]). The scales keep their meaning and
 * layout: sfA fp32 [M][K/128] (row m, K-block kb), sfB fp32 [ceil(N/128)][K/128]; C is
 * bf16 [M][N]. Same shape, alignment and error rules as dg_fp8_gemm_nt; the results
 * equal dg_fp8_gemm_nt's on the transposed operands bit for bit. The operands are
 * read in place, on the kernel the NT call of the same shape uses, when A stored
 * [K][M] has M % 16 == 0 and
 *   - M > 64: K*M, K*N < 2^31 (nothing is allocated, as for the NT call);
 *   - M <= 64: 1280*N < 2^31 when the split-K stream kernel serves the shape (K >= 2048
 *     with at most 10 K-blocks per split, e.g. 64x2112x7168; DG_PRINT_CONFIGS names
 *     the kernel), no further condition on the rolling kernel (e.g. 64x32768x512).
 * Otherwise an operand that is not K-contiguous is first transposed into a
 * library-owned buffer of the stream (M*K or N*K bytes, kept and reused by later calls
 * on that stream, released by dg_release_workspaces() or at the end of the process).
 */
dg_status dg_fp8_gemm_nn(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* hip_stream);
dg_status dg_fp8_gemm_tn(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* hip_stream);
dg_status dg_fp8_gemm_tt(const void* A, const void* B, void* C, const float* sfA,
                         const float* sfB, int64_t M, int64_t N, int64_t K, void* hip_stream);

/*
 * MoE grouped GEMM, contiguous layout (project page, "technical implementation":
 * several experts' token rows concatenated along M, N and K shared).
 *   A   e4m3fn [M_total][K]      sfA fp32 [M_total][K/128]
 *   B   e4m3fn [G][N][K]         sfB fp32 [G][ceil(N/128)][K/128]
 *   C   bf16   [M_total][N]
 *   m_indices int32 [M_total] (device): row r is multiplied by expert
 *   m_indices[r]'s B. A value outside [0, G) -- the pad marker is -1 -- marks a row
 *   that is neither read into any output nor written: C keeps its bytes there.
 * Performance contract: each expert's rows form one segment whose start is a
 * multiple of 128 (pad rows fill the gap). Any m_indices gives correct results;
 * 128-row groups that mix experts only cost extra passes.
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* A, const void* B, void* C,
                                              const float* sfA, const float* sfB,
                                              const int32_t* m_indices, int64_t M_total,
                                              int64_t N, int64_t K, int32_t G,
                                              void* hip_stream);

/*
 * MoE grouped GEMM, masked layout (launch article section 4.2; news page,
 * "performance"): each expert owns a fixed-capacity slab of M_max rows, of which
 * the first masked_m[e] are valid.
 *   A   e4m3fn [G][M_max][K]     sfA fp32 [G][M_max][K/128]
 *   B   e4m3fn [G][N][K]         sfB fp32 [G][ceil(N/128)][K/128]
 *   C   bf16   [G][M_max][N]
 *   masked_m int32 [G] (device), read on the device (no host sync); a value
 *   outside [0, M_max] is clamped into it. Rows m >= masked_m[e] are neither read
 *   nor written.
 *   expected_m: host-side hint of the typical masked_m, used only to pick a tile
 *   configuration (<= 0 means M_max). It never changes the result.
 */
dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* A, const void* B, void* C,
                                          const float* sfA, const float* sfB,
                                          const int32_t* masked_m, int32_t G,
                                          int64_t M_max, int64_t N, int64_t K,
                                          int64_t expected_m, void* hip_stream);

/*
 * The same three calls with sfA in the packed UE8M0 layout, the exponent-only form
 * of the LHS scaling factors that the project page (aiproducthub.cn, "technical
 * implementation") names as a way to cut scale traffic. Every sfA value must then be
 * a power of two 2^(b - 127), b in [0, 254]; the byte b stands for it:
 *   sfA  uint32 [rows][ceil(K/512)]: byte j (little-endian) of word w in row m is
 *        b for K-block 4w + j of row m; bytes past K/128 in a row's last word are
 *        not read. rows = M (dense), M_total (contiguous), G * M_max (masked, as
 *        [G][M_max][ceil(K/512)]).
 * A byte of 255 (NaN in the OCP MX format) is not a scale; results are unspecified.
 * Everything else (other operands, sfB in fp32, errors, untouched rows) is as in the
 * fp32-scale calls, and with equal scales the outputs are bitwise the same.
 */
dg_status dg_fp8_gemm_nt_ue8m0(const void* A, const void* B, void* C, const uint32_t* sfA,
                               const float* sfB, int64_t M, int64_t N, int64_t K,
                               void* hip_stream);

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* A, const void* B, void* C,
                                                    const uint32_t* sfA, const float* sfB,
                                                    const int32_t* m_indices, int64_t M_total,
                                                    int64_t N, int64_t K, int32_t G,
                                                    void* hip_stream);

dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* A, const void* B, void* C,
                                                const uint32_t* sfA, const float* sfB,
                                                const int32_t* masked_m, int32_t G,
                                                int64_t M_max, int64_t N, int64_t K,
                                                int64_t expected_m, void* hip_stream);

/*
 * Grouped GEMM with a fused SwiGLU + requantization epilogue: the first GEMM of an
 * MoE layer (Linear1) together with the activation between it and the second (the
 * DeepGEMM project page, aiproducthub.cn, "core features": Mega MoE fuses Linear1,
 * SwiGLU and Linear2). Per expert, B holds the gate projection in rows [0, I) and the
 * up projection in rows [I, 2I):
 *   A      e4m3fn [rows][K]            sfA  fp32 [rows][K/128]
 *   B      e4m3fn [G][2I][K]           sfB  fp32 [G][2I/128][K/128]
 *   codes  e4m3fn [rows][I] (output)   sf   fp32 [rows][I/128] (output)
 * with rows = M_total (contiguous, m_indices as in the contiguous GEMM) or G * M_max
 * (masked, as [G][M_max][...], masked_m as in the masked GEMM). For each produced
 * row, with g and u the fp32 block-scaled products of the gate and up columns
 * (two-level accumulation as in the GEMM calls):
 *   h[j] = silu(g[j]) * u[j],  silu(x) = x / (1 + e^-x), in fp32 (the division as
 *   a multiplication by the 1-ulp hardware reciprocal: h within a few ulps);
 * then h is quantized per 1x128 block exactly as dg_quantize_fp8_1x128 quantizes its
 * input: these outputs are the next GEMM's A operand and sfA. Rows that are not
 * produced (pad rows, rows >= masked_m[e]) are not written in codes or sf.
 * I % 128 == 0; A, B and codes 16-byte aligned, the scale and index arrays 4-byte
 * aligned; K/128 <= 32768 and (I + 256) * K < 2^31. Stream, ownership and error
 * conventions as above.
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_swiglu(const void* A, const void* B, void* codes,
                                                     float* sf, const float* sfA,
                                                     const float* sfB, const int32_t* m_indices,
                                                     int64_t M_total, int64_t I, int64_t K,
                                                     int32_t G, void* hip_stream);

dg_status dg_m_grouped_fp8_gemm_nt_masked_swiglu(const void* A, const void* B, void* codes,
                                                 float* sf, const float* sfA, const float* sfB,
                                                 const int32_t* masked_m, int32_t G,
                                                 int64_t M_max, int64_t I, int64_t K,
                                                 void* hip_stream);

/*
 * Per-token 1x128 activation quantizer: the step that turns activations into the
 * A operand and sfA of the calls above (one scaling factor per small block, each
 * block then spanning the FP8 range on its own: launch article, section 1.2).
 *   x      [M][K] row-major, fp32 (x_dtype = DG_DTYPE_F32) or bf16 (DG_DTYPE_BF16)
 *   codes  e4m3fn [M][K] (output)       sf  fp32 [M][K/128] (output)
 * For each block of 128 values (row m, K-block kb): amax = max |x|; e = the least
 * integer with amax <= 448 * 2^e (e = 0 when amax = 0); sf[m][kb] = 2^e as fp32;
 * each code is the e4m3fn value nearest to x / 2^e, ties to the even code, a zero
 * keeping the sign of x. Exact for every finite input (fp32 subnormals included;
 * 2^e below the fp32 range stores 0, as a float conversion of 2^e would); codes
 * and scales of a block holding an infinity or NaN are unspecified.
 * K % 128 == 0; x and codes 16-byte aligned, sf 4-byte aligned; M * K <= 2^40.
 * M == 0 or K == 0 returns DG_OK and launches nothing. Same stream, ownership and
 * error conventions as the GEMM calls.
 */
typedef enum dg_dtype { DG_DTYPE_F32 = 0, DG_DTYPE_BF16 = 1 } dg_dtype;

dg_status dg_quantize_fp8_1x128(const void* x, int32_t x_dtype, void* codes, float* sf,
                                int64_t M, int64_t K, void* hip_stream);

/*
 * Frees every library-owned buffer (split-K partials and counters, transposed operand
 * copies, retired buffers) on every device, after waiting for each such device to go
 * idle (hipDeviceSynchronize). The caller guarantees that no library call is in
 * flight on another thread and that no HIP graph holding a library call is replayed
 * afterwards; later calls allocate afresh. Not callable during a stream capture.
 * Returns DG_OK, or DG_ERR_LAUNCH if a synchronisation fails.
 */
dg_status dg_release_workspaces(void);

/* Identifier of the sources this library was built from (a hash of the kernel
 * sources and this header), so that a caller can tell a stale build. */
const char* dg_build_id(void);

/* Static string naming a status. */
const char* dg_status_string(dg_status s);

/* Thread-local description of the last failing call on this thread ("" if none). */
const char* dg_last_error_detail(void);

/*
 * Describe the tile configuration a call with these arguments would use, as a
 * NUL-terminated string written to buf (at most len bytes). kind: 0 dense,
 * 1 contiguous, 2 masked; for dense pass G = 1, for masked pass M = M_max and
 * expected_m. Host only; returns DG_ERR_BAD_SHAPE for kinds it does not know.
 */
dg_status dg_describe_config(int32_t kind, int64_t M, int64_t N, int64_t K, int32_t G,
                             int64_t expected_m, char* buf, int64_t len);

/*
 * The compiled-in tile configurations, for tuning and diagnostics: their number and
 * the name of configuration i (NULL when i is out of range). Setting the environment
 * variable DG_FORCE_CONFIG=<name> makes every later call that the configuration can
 * serve use it (calls it cannot serve keep the table's choice).
 */
int32_t dg_num_configs(void);
const char* dg_config_name(int32_t i);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */

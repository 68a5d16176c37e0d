/*
 * fp8_oracle.h -- plain, slow CPU oracle for FP8 quantization and scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the test suite, the smoke entry point and the CPU
 * baseline leg of the benchmark use it.  It shares no source, header, table or
 * helper with the HIP library.
 *
 * Every function restates, in the plainest arithmetic available (IEEE fp32
 * where the method is defined in fp32, fp64 otherwise), what the pages define:
 *
 *  - "How to Enable FP8 Training in NanoChat", section "FP8 Training Modes
 *    Explained": E4M3 = 4 exponent + 3 mantissa bits, E5M2 = 5 + 2.
 *  - "#84 FP8 Precision" (speedrun lab card), sections "Explanation" and
 *    "Hardware precision": weights are divided by a scale before the FP8
 *    cast; _scaled_mm(x, w_fp8, scale_a, scale_b) multiplies the scales back;
 *    the FP8 copy is re-quantized from the bf16 master after each optimizer
 *    step.
 *  - "FP8 stability guardrails" (zenaique explainer), section "Why FP8 is
 *    tempting and why it is fragile": E4M3 max 448, E5M2 max about 57344;
 *    values above the max overflow or saturate, values far below underflow to
 *    zero.  Section "Real products": fine-grained tile and block scaling.
 *
 * Parity pins for every function live in tests/test_oracle_*.py and
 * the C programs under tests/pins (enumeration, closed forms, exhaustive brute force, library
 * cross-checks).  No function here is "parity unpinned".
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };
enum { ORC_BF16 = 0, ORC_FP32 = 1 };
enum { ORC_TENSOR = 0, ORC_ROW_1x128 = 1, ORC_BLOCK_128x128 = 2 };
enum { ORC_FROM_AMAX = 0, ORC_GIVEN = 1 };
enum { ORC_EV_NONE = 0, ORC_EV_SATURATED = 1, ORC_EV_UNDERFLOW = 2, ORC_EV_NAN = 3 };

typedef struct {
    uint64_t saturated;      /* finite v whose unbounded RNE result exceeds fmax, and +-Inf inputs */
    uint64_t underflow;      /* non-zero x whose code is +-0 */
    uint64_t nan;            /* NaN inputs */
    uint64_t nonfinite_out;  /* GEMM outputs that are not finite in bf16 */
} orc_counters;

/* Format constants. */
double orc_fmax(int fmt);
int    orc_mant_bits(int fmt);
int    orc_exp_bits(int fmt);

/* Value of one FP8 code (NaN codes give NAN, E5M2 Inf codes give +-INFINITY). */
double orc_decode(int fmt, uint8_t code);

/* Encode an fp32 value v = fl32(x/s) onto the format grid: round to nearest,
 * ties to even, unbounded exponent above, gradual underflow below; then
 * saturate to +-fmax.  src_nonzero tells whether the source element x was
 * non-zero (an underflow is only counted for x != 0).  *event receives one
 * of ORC_EV_*. */
uint8_t orc_encode(int fmt, float v, int src_nonzero, int* event);

/* Quantize one element: v = fl32(x/s) (IEEE fp32 division), then orc_encode;
 * a NaN quotient gets the code 0x7F with sign(x) xor sign(s). */
uint8_t orc_cast_one(int fmt, float x, float s, orc_counters* ctr);

/* Read element idx of a bf16 (uint16 bit pattern) or fp32 array as fp32. */
float orc_load(const void* x, int dtype, int64_t idx);

/* max |x| over the finite elements of rows [r0,r1) x cols [c0,c1) (0 if none). */
float orc_amax_rect(const void* x, int dtype, int64_t ld,
                    int64_t r0, int64_t r1, int64_t c0, int64_t c1);

/* s = fl32(amax / fmax); amax == 0 gives 1; results below FLT_MIN become FLT_MIN. */
float orc_scale_from_amax(int fmt, float amax);

/* Number of scale entries for a granularity: 1, rows*ceil(cols/128) or
 * ceil(rows/128)*ceil(cols/128). */
int64_t orc_scale_count(int gran, int64_t rows, int64_t cols);

/* amax per granularity into out[orc_scale_count()] (row-major scale grid). */
void orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
              int gran, float* out);

/* Full quantize: for each scaling group (tensor / 1x128 row tile / 128x128
 * block), s = given or from amax, then q = encode(fl32(x/s)).  q is
 * [rows, cols] with leading dimension ldq; qt (nullable) receives the byte
 * transpose [cols, rows] with leading dimension ldqt.  Counters accumulate
 * into *ctr (nullable).  Returns 0 on success, -1 on bad arguments. */
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 int fmt, int gran, int mode, float* scale,
                 uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                 orc_counters* ctr);

/* Exact-as-fp64 scaled GEMM, TN layout: a [m,k] (lda), b [n,k] (ldb),
 * y [m,n] (ldy) in fp64 before any output rounding.
 *   (TENSOR, TENSOR):           y = s_a[0]*s_b[0] * sum_k dec(a)dec(b)
 *   (ROW_1x128, BLOCK_128x128): y = sum_kb s_a[m*(k/128)+kb] * s_b[(n/128)*(k/128)+kb]
 *                                       * sum_{k in kb} dec(a)dec(b)
 * Per-block partial sums are accumulated in fp64.  Returns -1 for an
 * unsupported granularity pair or k%128 != 0 in block mode. */
int orc_gemm(const uint8_t* a, int fa, int64_t lda, const float* sa, int ga,
             const uint8_t* b, int fb, int64_t ldb, const float* sb, int gb,
             int64_t m, int64_t n, int64_t k, double* y, int64_t ldy);

/* Same definition evaluated only at npts output positions (pm[i], pn[i]). */
int orc_gemm_points(const uint8_t* a, int fa, int64_t lda, const float* sa, int ga,
                    const uint8_t* b, int fb, int64_t ldb, const float* sb, int gb,
                    int64_t m, int64_t n, int64_t k,
                    const int64_t* pm, const int64_t* pn, int64_t npts, double* out);

/* Round a real value to bf16 (8 significant bits, RNE, overflow to +-Inf);
 * returns the bf16 bit pattern. */
uint16_t orc_bf16_rne(double y);

/* Count of non-finite bf16 outputs of y (used for the nonfinite_out counter). */
uint64_t orc_count_nonfinite_bf16(const double* y, int64_t count);

/* Threads the OpenMP loops in this file use. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif

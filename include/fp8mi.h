/*
 * fp8mi.h -- C ABI of the MI355X (gfx950) FP8 scaled-matmul library.
 *
 * Three operations, as the pages describe them:
 *   1. amax and a saturating round-to-nearest-even cast of bf16 (or fp32)
 *      tensors to FP8 E4M3 (max 448) or E5M2 (max 57344), with one scale per
 *      tensor, per 1x128 row tile or per 128x128 block;
 *   2. the scaled GEMM y = (s_a A_q)(s_b B_q)^T, fp32 accumulation, bf16 out;
 *   3. the FP8 weight-copy cache, re-quantized from the master weights after
 *      every optimizer step.
 *
 * Conventions for every entry point:
 *   - All tensor, scale, counter and workspace pointers are DEVICE pointers
 *     owned by the caller.  The library never allocates device memory, never
 *     frees caller memory and keeps no mutable global state (apart from the
 *     per-device architecture probe and the thread-local error text).
 *   - Every call only enqueues work on `stream` (NULL = the default stream)
 *     and returns; it never synchronizes the host.  Scales computed on the
 *     device stay on the device.
 *   - Arguments are checked on the host BEFORE anything is enqueued; a call
 *     that returns an error has enqueued nothing.  Device-side values (scales
 *     given by the caller) are not inspected on the host.
 *   - Row-major throughout.  "ld" arguments are leading dimensions in
 *     elements of the tensor they belong to.
 *   - Nothing throws or aborts across the ABI.  FP8_ERR_HIP carries detail in
 *     fp8_last_error() (thread-local).
 *   - Only gfx950 devices are accepted: any other device returns
 *     FP8_ERR_UNSUPPORTED_DEVICE and nothing falls back to another path.
 *
 * FP8 encodings are the OCP ones (E4M3FN: bias 7, no Inf, S.1111.111 = NaN;
 * E5M2: bias 15, IEEE-style Inf/NaN); these are the formats whose maxima are
 * 448 and 57344 ("FP8 stability guardrails", section "Why FP8 is tempting and
 * why it is fragile"; bit splits in "How to Enable FP8 Training in NanoChat",
 * section "FP8 Training Modes Explained").
 */
#ifndef FP8MI_H
#define FP8MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle, declared here so that this header needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

#define FP8MI_ABI_VERSION 1

typedef enum {
    FP8_OK = 0,
    FP8_ERR_INVALID_ARG = 1,        /* null pointer, negative size, bad ld, bad enum, bad alignment */
    FP8_ERR_UNSUPPORTED_SHAPE = 2,  /* a shape / granularity combination the operation does not take */
    FP8_ERR_UNSUPPORTED_DEVICE = 3, /* current device is not gfx950 */
    FP8_ERR_HIP = 4                 /* a HIP runtime call or launch failed; see fp8_last_error() */
} fp8_status;

typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format;
typedef enum { FP8_IN_BF16 = 0, FP8_IN_FP32 = 1 } fp8_dtype;
typedef enum {
    FP8_TENSOR = 0, FP8_ROW_1x128 = 1, FP8_BLOCK_128x128 = 2,
    /* GEMM operands only: 1x128 / 128x128 scales that are powers of two */
    FP8_ROW_1x128_POW2 = 3, FP8_BLOCK_128x128_POW2 = 4
} fp8_granularity;
typedef enum { FP8_SCALE_FROM_AMAX = 0, FP8_SCALE_GIVEN = 1, FP8_SCALE_FROM_AMAX_POW2 = 2 } fp8_scale_mode;

/* Telemetry: counts of clipping and overflow events (the NanoChat page's FAQ
 * recommends logging them; the guardrails explainer lists overflow counters
 * among its checks).  Lives in device memory;
 * every call that takes a non-NULL pointer ADDS its events with integer
 * atomics.  Reset with fp8_counters_reset().
 *   saturated     - elements whose value x/s, rounded to nearest-even on the
 *                   format's grid with no upper exponent bound, exceeds the
 *                   format maximum (written as +-max), plus +-Inf inputs;
 *   underflow     - non-zero inputs whose code is +-0 (sign kept);
 *   nan           - NaN inputs (written as 0x7F | sign);
 *   nonfinite_out - GEMM outputs that are +-Inf or NaN in bf16. */
typedef struct {
    uint64_t saturated;
    uint64_t underflow;
    uint64_t nan;
    uint64_t nonfinite_out;
} fp8_counters;

int32_t     fp8_abi_version(void);
const char* fp8_status_string(fp8_status s);
const char* fp8_last_error(void);

/* ------------------------------------------------------------------ amax
 * max |x| over the finite elements of each scaling group (the guardrails
 * explainer derives scales from the measured range of the data, and keeps an
 * amax history in its section "Real products").
 *   x      [rows, cols], leading dimension ld >= cols, bf16 or fp32.
 *   amax   out: 1 float (TENSOR), [rows, ceil(cols/128)] (ROW_1x128) or
 *          [ceil(rows/128), ceil(cols/128)] (BLOCK_128x128), row-major.
 *          A group with no finite element gets 0.
 *   workspace  TENSOR needs fp8_amax_workspace_size() bytes (partial maxima);
 *          other granularities need none (may be NULL).  Its contents on
 *          entry do not matter, and it must not be in use by another call at
 *          the same time.
 * Sizes of zero are allowed (TENSOR writes 0). */
size_t     fp8_amax_workspace_size(int64_t rows, int64_t cols, fp8_granularity gran);
fp8_status fp8_amax(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                    fp8_granularity gran, float* amax,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ quantize
 * Scale, then cast: for each element of each scaling group
 *     v = fl32(x / s)                    (IEEE fp32 division, exactly rounded)
 *     q = round-to-nearest-even(v) on the format's grid, saturated to +-max
 * (#84 lab card, section "Explanation": the weight is divided by its scale
 * and then cast to FP8; the guardrails explainer: values past the format's
 * maximum saturate and very small ones become zero).  NaN -> 0x7F|sign,
 * +-Inf -> +-max.
 *   mode FROM_AMAX: s = fl32(amax / fmax) per group (fmax 448 or 57344);
 *       amax == 0 gives s = 1; s below FLT_MIN is raised to FLT_MIN.  The
 *       scales are WRITTEN to `scale`.
 *   mode GIVEN: the caller's scales are READ from `scale` (a "learned" or
 *       fixed scale, #84 lab card, "Hardware precision") and used as they
 *       are; they should be finite and > 0.
 *   mode FROM_AMAX_POW2: per group, the smallest power of two s with
 *       amax / s <= fmax (real quotient; 1 for amax 0, at least 2^-126),
 *       WRITTEN to `scale` as fp32.  Not on the pages: their fine-grained
 *       scaling with scales the gfx950 MFMA can apply itself (an fp32 power
 *       of two's exponent field is its E8M0 code); the division is exact and
 *       nothing saturates.  Such scales feed the _POW2 GEMM pair below.
 *   scale  1 float / [rows, ceil(cols/128)] / [ceil(rows/128), ceil(cols/128)]
 *          row-major, as for fp8_amax.  These are DEQUANTIZATION multipliers
 *          (x ~ s * decode(q)), the scale_a / scale_b of the scaled GEMM.
 *   q      out [rows, cols] bytes, leading dimension ldq >= cols.
 *   q_t    optional out (NULL = none): the byte transpose [cols, rows],
 *          leading dimension ldq_t >= rows.  TENSOR and BLOCK_128x128 only
 *          (a 1x128 row tile does not transpose into a 1x128 row tile:
 *          FP8_ERR_UNSUPPORTED_SHAPE).  When rows is a multiple of 64 KiB
 *          (e.g. 65536 tokens), pad ldq_t (by 256, say): rows that lie a
 *          multiple of 64 KiB apart share HBM channels, which slows both
 *          this write and a GEMM that reads q_t as an operand.
 *   ctr    optional counters (NULL = none).
 *   workspace  TENSOR + FROM_AMAX needs fp8_quantize_workspace_size() bytes;
 *          the other modes need none.  Its contents on entry do not matter,
 *          and it must not be in use by another call at the same time.  A
 *          small per-tensor call (bf16, whole 128x128 tiles, at most 256
 *          tiles and one per CU, 8-byte aligned workspace) runs as one
 *          launch whose workgroups exchange their tile maxima through the
 *          workspace, matched to the call by a counter kept there.
 * Alignment: x, q, q_t any; fast vector paths are taken when rows start on
 * 16-byte boundaries. */
size_t     fp8_quantize_workspace_size(int64_t rows, int64_t cols, fp8_granularity gran,
                                       fp8_scale_mode mode);
fp8_status fp8_quantize(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                        fp8_format fmt, fp8_granularity gran, fp8_scale_mode mode,
                        float* scale,
                        uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                        fp8_counters* ctr,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fp8_quantize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It computes exactly what fp8_quantize
 * does with the same arguments.  The per-tensor amax partials it needs
 * (TENSOR with FROM_AMAX or FROM_AMAX_POW2) go to a scratch array the
 * library holds in device memory: 8 KiB per device, loaded with the library
 * and kept until the process ends; its address is resolved once per device
 * on the first call made with that device current.  No size needs more than
 * those 8 KiB (a call that would gets FP8_ERR_UNSUPPORTED_SHAPE).  Every call
 * on a device shares that device's scratch, and nothing in it has to start
 * at zero (each call writes the partials it reads); calls that overlap in
 * time on one device -- on different streams, or from different threads
 * without ordering -- race on it and may produce wrong scales.  Calls on
 * one stream are ordered and safe. */
fp8_status fp8_quantize_noalloc(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                                fp8_format fmt, fp8_granularity gran, fp8_scale_mode mode,
                                float* scale,
                                uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                                fp8_counters* ctr, hipStream_t stream);

/* ------------------------------------------------------------------ delayed scaling
 * Per-tensor quantize with delayed scaling and an amax history (the
 * guardrails explainer, "Real products": Transformer Engine's delayed
 * scaling with amax history tracking).  One call:
 *     s = the FROM_AMAX rule applied to max(amax_history[0 .. history_len))
 *         (0 -> 1, below FLT_MIN -> FLT_MIN), written to scale[0];
 *     q (and q_t) = the cast of x with s, exactly as fp8_quantize(GIVEN, s),
 *         counters included (an element above the recorded amax saturates
 *         and is counted);
 *     then amax_history[*history_pos] = amax(x) (finite maximum of |x|) and
 *         *history_pos = (*history_pos + 1) % history_len.
 * The tensor's own amax does not enter its own cast; a history of length 1
 * holding this tensor's amax reproduces fp8_quantize(FROM_AMAX).
 *   amax_history  device float[history_len], entries finite and >= 0
 *                 (start from zeros: the first cast then uses s = 1);
 *   history_pos   device int32, the slot of the oldest entry (taken modulo
 *                 history_len);  1 <= history_len <= 4096.
 * A bf16 tensor whose rows and cols are multiples of 128, with 16-byte
 * aligned rows and a transposed copy, is read once (the cast collects the
 * amax on the way); other layouts read x twice (amax pass, then cast), with
 * identical results.  Other arguments as fp8_quantize (TENSOR granularity).
 * workspace: fp8_quantize_delayed_workspace_size() bytes. */
size_t     fp8_quantize_delayed_workspace_size(int64_t rows, int64_t cols);
fp8_status fp8_quantize_delayed(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                                fp8_format fmt, float* amax_history, int32_t* history_pos,
                                int32_t history_len, float* scale,
                                uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                                fp8_counters* ctr,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ scaled GEMM
 * y = (s_a A_q)(s_b B_q)^T in the TN layout that _scaled_mm(x, w_fp8,
 * scale_a, scale_b) implies (#84 lab card, code excerpt and "Explanation":
 * the weight operand is K-contiguous):
 *   a  [m, k] FP8 bytes, lda >= k;  b  [n, k] FP8 bytes, ldb >= k;
 *   c  [m, n] bf16 out, ldc >= n.   fa, fb: any of E4M3 / E5M2.
 * Scale pairs:
 *   (TENSOR, TENSOR)            y = bf16(s_a[0] s_b[0] sum_k A B)
 *   (ROW_1x128, BLOCK_128x128)  y = bf16(sum_kb s_a[m, kb] s_b[n/128, kb] sum_{k in kb} A B)
 *       ("fine grained tile and block scaling", guardrails explainer,
 *       "Real products"); s_a is [m, k/128], s_b is [ceil(n/128), k/128],
 *       row-major; needs k % 128 == 0.
 *   (ROW_1x128_POW2, BLOCK_128x128_POW2)  the same sum, for scales that are
 *       powers of two (as fp8_quantize(FROM_AMAX_POW2) writes them): the
 *       matrix cores apply them as E8M0 exponents inside each MFMA, with no
 *       per-block promotion on the VALU.  Only the exponent field of each
 *       scale is read.  Not on the pages (their fine-grained scaling, in the
 *       form gfx950's scaled MFMA takes).
 * Products are accumulated in fp32 by the MFMA units; the epilogue rounds to
 * bf16 (nearest even).  Any other pair: FP8_ERR_UNSUPPORTED_SHAPE.
 * Shape rules: k % 16 == 0, lda % 16 == 0, ldb % 16 == 0, a and b 16-byte
 * aligned, lda and ldb below 2^22, ldc below 2^21 (else
 * FP8_ERR_UNSUPPORTED_SHAPE); m, n any >= 0; k == 0 writes zeros.
 * workspace: when fp8_scaled_mm_workspace_size() > 0 the call may split the K
 * dimension into slices reduced in a fixed order (deterministic); a smaller
 * workspace (or NULL) runs without the split (same result to tolerance,
 * different rounding order).
 * ctr: nonfinite_out counts outputs that are Inf/NaN in bf16. */
size_t     fp8_scaled_mm_workspace_size(int64_t m, int64_t n, int64_t k,
                                        fp8_granularity ga, fp8_granularity gb);
fp8_status fp8_scaled_mm(const uint8_t* a, fp8_format fa, int64_t lda,
                         const float* scale_a, fp8_granularity ga,
                         const uint8_t* b, fp8_format fb, int64_t ldb,
                         const float* scale_b, fp8_granularity gb,
                         int64_t m, int64_t n, int64_t k,
                         void* c_bf16, int64_t ldc,
                         void* workspace, size_t workspace_bytes,
                         fp8_counters* ctr, hipStream_t stream);

/* ------------------------------------------------------------------ quantize + GEMM
 * The forward projection with its activation quantized on the way into the
 * GEMM: x is bf16 [m, k]; one call computes
 *     s_a = the FROM_AMAX per-tensor scale of x (written to scale_a),
 *     q   = the codes of x exactly as fp8_quantize(x, fa, TENSOR, FROM_AMAX)
 *           gives them (written to xq and/or its transpose xq_t when those
 *           are non-NULL; counters added to ctr),
 *     y   = bf16(s_a s_b sum_k q[m,k] B[n,k]) into c, as fp8_scaled_mm
 *           (TENSOR, TENSOR) on those codes would.
 * x is read twice (an amax pass, then the GEMM's operand load, which casts
 * each 192 x 768 block of rows into LDS once) and the codes need not go
 * through HBM for the forward product ("FP8 stability guardrails", section
 * "Why FP8 is tempting and why it is fragile": FP8 halves the activation's
 * memory traffic; "#84 FP8 Precision", code excerpt: the scaled product).
 *   x     bf16 [m, k], ldx % 8 == 0, 16-byte aligned.
 *   xq    optional [m, k] codes, ldxq % 16 == 0, 16-byte aligned.
 *   xq_t  optional [k, m] codes (the dW operand of the backward pass);
 *         4-byte stores when xq_t and ldxq_t are 4-byte aligned, byte stores
 *         otherwise (pad ldxq_t when m is a multiple of 64 KiB, as for
 *         fp8_quantize).
 *   b     [n, k] codes, ldb % 16 == 0, 16-byte aligned; scale_b per tensor.
 *   c     bf16 [m, n]; n and ldc multiples of 4, 8-byte aligned.
 * Shapes: k == 768 (one panel of A codes fills the LDS), ldx and ldb below
 * 2^22, ldc below 2^21; other shapes FP8_ERR_UNSUPPORTED_SHAPE (use
 * fp8_quantize + fp8_scaled_mm).  m == 0 writes scale 1 only.
 * workspace: fp8_quantize_scaled_mm_workspace_size() bytes (amax partials). */
size_t     fp8_quantize_scaled_mm_workspace_size(int64_t m, int64_t n, int64_t k);
fp8_status fp8_quantize_scaled_mm(const void* x, int64_t ldx, fp8_format fa, float* scale_a,
                                  uint8_t* xq, int64_t ldxq, uint8_t* xq_t, int64_t ldxq_t,
                                  const uint8_t* b, fp8_format fb, int64_t ldb, const float* scale_b,
                                  int64_t m, int64_t n, int64_t k,
                                  void* c_bf16, int64_t ldc, fp8_counters* ctr,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ weight cache
 * The FP8 compute copy of master weights, rebuilt from the bf16 master after
 * every optimizer step and kept for the next forward pass (#84 lab card,
 * "Hardware precision"; quantize_weights_fp8 in its second code excerpt).
 * Each descriptor names caller-owned device storage:
 *   rows, cols  shape of the master [rows, cols] (contiguous, ld = cols);
 *   fmt, gran   format and granularity (TENSOR or BLOCK_128x128 here);
 *   q           [rows, cols] bytes; q_t optional [cols, rows] bytes (the
 *               K-contiguous operand for the transposed GEMM);
 *   scale       1 float (TENSOR) or the block grid (BLOCK_128x128);
 *   ctr         optional counters.
 * fp8_requant_weights() re-quantizes every cache from its master with a
 * fresh amax scale (current scaling).  The caches go in groups of up to 24;
 * each group takes at most three launches: one amax pass over its TENSOR
 * caches (left out when it has none), one cast pass over the whole tiles of
 * its bf16 caches and one over every other tile (left out when there is
 * none), TENSOR caches with the scale of their amax pass, BLOCK caches with
 * each block's own amax.  An empty TENSOR cache gets scale 1 from a launch of its own.
 * A call with one cache runs fp8_quantize's kernels for it (as many
 * launches, the faster tile kernels).  The result is byte-identical to fp8_quantize(master, FROM_AMAX) of each,
 * counters included.  rows and cols below 2^31.  masters[i] is a
 * device pointer, master_dtypes[i] its dtype; the three arrays are HOST arrays
 * of length count.  Workspace: fp8_requant_workspace_size(). */
typedef struct {
    int64_t rows, cols;
    fp8_format fmt;
    fp8_granularity gran;
    uint8_t* q;
    uint8_t* q_t;
    float* scale;
    fp8_counters* ctr;
} fp8_weight_cache;

size_t     fp8_requant_workspace_size(const fp8_weight_cache* caches, int32_t count);
fp8_status fp8_requant_weights(const fp8_weight_cache* caches, const void* const* masters,
                               const fp8_dtype* master_dtypes, int32_t count,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Zero a counter block on `stream` (a small fill kernel, safe to capture). */
fp8_status fp8_counters_reset(fp8_counters* ctr, hipStream_t stream);

/* Testing aid for the one-launch path of small per-tensor quantize calls
 * (see fp8_quantize's workspace).  Each workgroup waits, a bounded number of
 * polls, for every tile's maximum; one whose wait runs out reads the whole
 * tensor itself (the same scale and codes, slower).  Sets that bound for
 * the calls that follow, from any thread (0: every workgroup reads the
 * whole tensor), and returns the previous one; the default is 16384. */
int32_t fp8_debug_set_wait_limit(int32_t polls);

#ifdef __cplusplus
}
#endif
#endif

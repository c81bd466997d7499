/*
 * archead.h -- C ABI of the packed ARCHead LM-head forward for MI355X (gfx950).
 *
 * The operation (ARCHead paper, "Activation-Metric Residual Correction for
 * LLM Output Heads", section 3.2):
 *   eq 3  W_d   = Q5(A_c) Q8(B_c) + Q_SC4(W - A_c B_c)
 *   eq 6  W_hat = W_d + A_w B_w                (A_w, B_w stored as row/group
 *                                               INT8, text after eq 7)
 *   eq 7  logits = X W_d^T + (X B_w^T) A_w^T   (factored: no dense W_hat)
 * In the stored fields (section 3.3, state-dict accounting paragraph):
 *   W_hat[v,j] = sA[v] sum_i A5[v,i] sB[i] B8[i,j]
 *              + sR[v, j/g] R4[v,j]
 *              + sC[v] sum_i C8[v,i] sD[i, j/g] D8[i,j]
 *   logits[m,v] = sum_j X[m,j] W_hat[v,j]
 * Notation follows the paper's statement of the problem (section 3.4
 * inputs): vocabulary V, hidden size d (the paper's D), core rank k (r_c),
 * correction rank r (r_r), group size g, and M hidden states.
 *
 * Canonical HOST layout of the packed fields (all row-major):
 *   A5  int8     V x k      values in [-16, 15] (5-bit core factor)
 *   sA  uint16   V          fp16 bit patterns, one scale per row
 *   B8  int8     k x d      8-bit core factor
 *   sB  uint16   k          fp16, one scale per row
 *   R4  uint8    V x d/2    SC4 residual: byte [v,c] = column 2c in the low
 *                           nibble, column 2c+1 in the high nibble, 4-bit
 *                           two's complement
 *   sR  uint16   V x d/g    fp16, one scale per (row, g-column group)
 *   C8  int8     V x r      quantised A_w (row-wise INT8)
 *   sC  uint16   V          fp16, one scale per row
 *   D8  int8     r x d      quantised B_w (group-wise INT8)
 *   sD  uint16   r x d/g    fp16, one scale per (row, g-column group)
 * The library re-lays these out into its own device layout at load time
 * (A5 at 5 bits per value) and never keeps a dense W_hat anywhere.
 *
 * Streams: every call that touches the device takes a hipStream_t (as void*;
 * NULL = the null stream).  Kernels are enqueued on that stream; the library
 * never synchronises it on the forward path and never allocates there once
 * the workspace is large enough (see archead_reserve).  The forward calls of
 * one handle share its workspace (including the work counters of the
 * one-launch GEMV path): enqueue them on one stream, or order them with
 * events; forward calls of one handle that overlap on the device race.
 *
 * Errors: every entry point returns an archead_status and never throws or
 * aborts.  Arguments are validated before anything is enqueued.  A HIP
 * failure maps to ARCHEAD_EHIP; archead_last_error() returns a thread-local
 * text with the detail of the last failure on the calling thread.  NaN or
 * Inf scales are not checked: they propagate into the logits.
 */
#ifndef ARCHEAD_H
#define ARCHEAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ARCHEAD_ABI_VERSION 1

typedef struct archead_head *archead_t;

typedef enum archead_status {
    ARCHEAD_OK = 0,
    ARCHEAD_EINVAL = 1, /* NULL pointer, bad handle, negative size, bad path */
    ARCHEAD_ESHAPE = 2, /* shape the layout does not support (see pack_load) */
    ARCHEAD_ERANGE = 3, /* a field value outside its integer range          */
    ARCHEAD_ENOMEM = 4, /* device or host allocation failed                 */
    ARCHEAD_EHIP = 5    /* a HIP runtime call failed                        */
} archead_status;

/* Allocation-failure injection (for tests of callers' error handling): when
 * the environment variable ARCHEAD_TEST_ALLOC_LIMIT holds a byte count, every
 * device allocation the library would make above that size -- the packed
 * block of archead_pack_load, a workspace growth (archead_reserve and the
 * forward calls), each buffer of archead_build and archead_quantize -- is
 * refused before any HIP call and the entry point returns ARCHEAD_ENOMEM with
 * its state unchanged (a handle keeps its old workspace).  The variable is
 * read at every allocation; unset or empty, it has no effect. */

/* Kernel families for the vocabulary-tile step (archead_forward_path).
 * GEMV runs the whole forward (projection, vocabulary tiles, argmax) as one
 * kernel launch; it takes d a multiple of 512 and M = 1, or M = 2 with
 * g = 128 (otherwise ARCHEAD_ESHAPE).  SKINNY runs as one launch too at M = 1 when d is a
 * multiple of 512 and g = 128, and otherwise, like LDS, launches the
 * projection, the vocabulary tiles and the argmax reduction as separate
 * kernels; both take any M. */
typedef enum archead_path {
    ARCHEAD_PATH_AUTO = 0,   /* LDS for M >= 128, else SKINNY; GEMV instead at
                                M = 1 when SKINNY cannot run as one launch
                                (g != 128) but GEMV can                       */
    ARCHEAD_PATH_GEMV = 1,   /* VALU dot2 GEMV, one launch, M <= 2             */
    ARCHEAD_PATH_SKINNY = 2, /* register-dequantised MFMA, W streamed once     */
    ARCHEAD_PATH_LDS = 3     /* LDS-staged fp16-dequantised MFMA, large M      */
} archead_path;

/*
 * archead_pack_load -- build a device-resident packed head.
 *
 * Defines: the packed module of ARCHead paper section 3.3 (registers only
 * the SC4 residual and its scales, the quantised core factors, the quantised
 * correction factors and shape metadata; the dense V x D head is not kept).
 *
 * V, d, k, r, g  shape (see above).  Supported: V >= 1, V < 2^31;
 *                d a multiple of 128 in [128, 2^20] (the kernels stream the
 *                residual in 128-column K-chunks, one 16-byte load per lane,
 *                and read X in the same chunks straight from the caller's
 *                buffer, so a ragged last chunk would need a padded copy of
 *                X on every call; hidden sizes of LLM heads are multiples of
 *                128); g a multiple of 32 dividing d;
 *                0 <= k <= 4096, 0 <= r <= 4096 (k = 0 or r = 0 drop the
 *                core or the correction term; the corresponding pointers
 *                may then be NULL).  Otherwise ARCHEAD_ESHAPE.
 * A5 .. sD       HOST pointers in the canonical layout above, borrowed for
 *                the duration of the call only (the caller keeps ownership
 *                and may free them on return).  NULL where required ->
 *                ARCHEAD_EINVAL.  An A5 value outside [-16, 15] ->
 *                ARCHEAD_ERANGE.
 * hip_stream     stream used for the host-to-device copies; the call waits
 *                for them before returning.
 * out            receives the handle; set to NULL on failure.  The handle
 *                owns all device memory it allocates (packed fields in the
 *                device layout plus a workspace) until archead_free.
 */
archead_status archead_pack_load(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g,
                                 const int8_t *A5, const uint16_t *sA,
                                 const int8_t *B8, const uint16_t *sB,
                                 const uint8_t *R4, const uint16_t *sR,
                                 const int8_t *C8, const uint16_t *sC,
                                 const int8_t *D8, const uint16_t *sD,
                                 void *hip_stream, archead_t *out);

/*
 * archead_reserve -- size the handle's device workspace for up to M_max
 * hidden states per call, so that later forward calls with M <= M_max never
 * allocate.  The call waits until the new workspace is ready.
 * A forward call with a larger M grows the workspace itself, in stream
 * order and without waiting: the new buffer is allocated and zeroed on the
 * call's stream (hipMallocAsync), and the old one is released on that
 * stream behind the work already enqueued there (hipFreeAsync).  A forward
 * call that would grow the workspace while its stream is being captured
 * into a HIP graph fails with ARCHEAD_EINVAL before enqueuing anything:
 * reserve before capturing.
 * M_max < 0 -> ARCHEAD_EINVAL; M_max > 2^20 -> ARCHEAD_ESHAPE.
 */
archead_status archead_reserve(archead_t h, int64_t M_max, void *hip_stream);

/*
 * archead_forward -- logits = X W_hat^T, evaluated factored as in eq 7
 * (ARCHead paper section 3.2): the dense V x d head is never formed.
 *
 * M        number of hidden states, 0 <= M <= 2^20 (M = 0 is a no-op that
 *          succeeds whatever X and logits are).
 * X        DEVICE pointer, bf16, M x d row-major, 16-byte aligned.
 * logits   DEVICE pointer, fp32, M x V row-major, written in full.
 * X and logits are caller-owned and must stay valid until the stream has
 * passed this call.  Work is enqueued on hip_stream and not waited for.
 * Numerics: integer fields are used exactly; accumulation is fp32; the
 * large-M path rounds the product sR*R4 once to fp16 (see archead_path).
 */
archead_status archead_forward(archead_t h, int64_t M, const void *X, float *logits,
                               void *hip_stream);

/*
 * archead_forward_argmax -- as archead_forward, plus the per-token top-1
 * index: argmax[m] = min{ v : logits[m,v] = max_u logits[m,u] } (the top-1
 * token whose agreement with the dense head the ARCHead pages report).
 *
 * logits   DEVICE fp32 M x V, or NULL to skip writing the logits.
 * argmax   DEVICE int32 M, written in full.  NaN logits make the index of
 *          that row unspecified (but within [0, V)).
 */
archead_status archead_forward_argmax(archead_t h, int64_t M, const void *X, float *logits,
                                      int32_t *argmax, void *hip_stream);

/*
 * archead_forward_argmax_noalloc -- archead_forward_argmax for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It never allocates or frees
 * anything: the kernels' workspace is a fixed device array of 8 MiB per GPU
 * inside the library, kept until the process ends.  Its address is looked
 * up once per device, on the first call there.
 *
 * Arguments, results, numerics and stream behaviour are those of
 * archead_forward_argmax (automatic path); the results are identical.
 * A call whose workspace would exceed 8 MiB -> ARCHEAD_ESHAPE (for the
 * 151936 x 4096 head with k = 256, r = 64 that is every M below 128; the
 * large-M path needs more).
 * Every call on a GPU, from any handle, shares that GPU's array, which keeps
 * the last call's contents: each call first clears (with a small kernel on
 * hip_stream) what must start at zero.  Calls that overlap on one GPU
 * (different streams with no ordering between them) race and give
 * undefined results; order them on one stream or with events.
 */
archead_status archead_forward_argmax_noalloc(archead_t h, int64_t M, const void *X, float *logits,
                                              int32_t *argmax, void *hip_stream);

/*
 * archead_forward_path -- archead_forward_argmax with the vocabulary-tile
 * kernel family forced (archead_path).  logits and argmax may each be NULL
 * (not both).  An unknown path -> ARCHEAD_EINVAL.  Every path computes the
 * same function to within the documented rounding.
 */
archead_status archead_forward_path(archead_t h, int64_t M, const void *X, float *logits,
                                     int32_t *argmax, int path, void *hip_stream);

/*
 * archead_forward_timed -- archead_forward_path that also records two HIP
 * events on hip_stream immediately before and after the vocabulary-tile
 * kernel (the step that streams the packed fields), so that a caller can
 * time that kernel alone.  ev_before / ev_after are hipEvent_t values (as
 * void*) created by the caller on the current device; NULL -> ARCHEAD_EINVAL.
 * For benchmarking and profiling; the results are those of
 * archead_forward_path.
 */
archead_status archead_forward_timed(archead_t h, int64_t M, const void *X, float *logits,
                                     int32_t *argmax, int path, void *hip_stream,
                                     void *ev_before, void *ev_after);

/*
 * archead_forward_ce -- the forward plus the softmax log-normaliser and
 * the cross-entropy of each hidden state's logits, reduced inside the
 * vocabulary-tile pass (the logits need not be written).  The ARCHead
 * pages (abstract and section 1) note that the head's logits go straight
 * into the softmax and judge the head by the cross-entropy it adds and by
 * relative perplexity = exp(mean cross-entropy); in natural logarithms:
 *   lse[m] = log sum_v exp(logits[m, v])
 *   nll[m] = lse[m] - logits[m, targets[m]]
 *
 * targets  DEVICE int32 M, the target row of each hidden state, or NULL
 *          (then nll must be NULL too).  A target outside [0, V) gives
 *          nll[m] = NaN; it is not an error.
 * logits   DEVICE fp32 M x V, or NULL to skip writing the logits.
 * argmax   DEVICE int32 M (as archead_forward_argmax), or NULL.
 * lse      DEVICE fp32 M, written in full; NULL -> ARCHEAD_EINVAL.
 * nll      DEVICE fp32 M, written in full, or NULL (with targets NULL).
 *          targets and nll not both given or both NULL -> ARCHEAD_EINVAL.
 * Other arguments, ownership and stream behaviour as archead_forward.
 * Numerics: lse and nll are taken from the same fp32 logits the forward
 * writes; exponentials and sums run in fp32 against each tile's maximum
 * (no overflow for any finite logits), so lse equals the log-normaliser of
 * those logits up to fp32 rounding of the exponentials and their sums.
 * NaN or infinite logits make lse and nll of that row unspecified.
 */
archead_status archead_forward_ce(archead_t h, int64_t M, const void *X, const int32_t *targets,
                                  float *logits, int32_t *argmax, float *lse, float *nll,
                                  void *hip_stream);

/* archead_forward_ce_path -- archead_forward_ce with the vocabulary-tile
 * kernel family forced (archead_path); an unknown path -> ARCHEAD_EINVAL. */
archead_status archead_forward_ce_path(archead_t h, int64_t M, const void *X, const int32_t *targets,
                                       float *logits, int32_t *argmax, float *lse, float *nll,
                                       int path, void *hip_stream);

/*
 * archead_forward_topk -- the forward (logits written) plus the K largest
 * logits of every hidden state, in order: values[m, 0] is the largest,
 * equal values by lower vocabulary index (so indices[m, 0] is the argmax of
 * archead_forward_argmax).  The pages report how often the packed head keeps
 * the dense head's top-1 token (ARCHead paper section 1, results); the same
 * ordering over K candidates is what top-k sampling draws from.
 *
 * K        1 <= K <= min(16, V); otherwise ARCHEAD_EINVAL.
 * logits   DEVICE fp32 M x V, written in full (required: the selection
 *          reads them back after the vocabulary-tile pass).
 * values   DEVICE fp32 M x K, row-major: values[m, j] = logits[m, indices[m, j]].
 * indices  DEVICE int32 M x K, row-major.
 * Other arguments, ownership and stream behaviour as archead_forward.
 * NaN logits make the order of that row unspecified.
 */
archead_status archead_forward_topk(archead_t h, int64_t M, const void *X, int32_t K, float *logits,
                                    float *values, int32_t *indices, void *hip_stream);

/* archead_forward_topk_path -- archead_forward_topk with the vocabulary-tile
 * kernel family forced (archead_path); an unknown path -> ARCHEAD_EINVAL. */
archead_status archead_forward_topk_path(archead_t h, int64_t M, const void *X, int32_t K, float *logits,
                                         float *values, int32_t *indices, int path, void *hip_stream);

/*
 * archead_forward_sample -- archead_forward_topk plus one draw per hidden
 * state from its K candidates at temperature tau (top-k sampling): candidate
 * j weighs exp((values[m, j] - values[m, 0]) / tau), and the draw is the
 * first j whose running sum of weights exceeds u[m] times their total;
 * samples[m] = indices[m, j].  The weights and sums are fp32.
 *
 * temperature  tau > 0 and finite, with log2(e) / tau finite in fp32 (so no
 *              subnormal tau), else ARCHEAD_EINVAL.
 * u            DEVICE fp32 M, uniform numbers in [0, 1) drawn by the caller
 *              (a value outside [0, 1) picks the first or the last candidate).
 * samples      DEVICE int32 M.
 * K, logits, values, indices as archead_forward_topk (all required).
 */
archead_status archead_forward_sample(archead_t h, int64_t M, const void *X, int32_t K, float temperature,
                                      const float *u, float *logits, float *values, int32_t *indices,
                                      int32_t *samples, void *hip_stream);

/*
 * archead_build -- construct a packed head on the GPU from a dense head W
 * and calibration hidden states H (ARCHead paper section 3.4, the
 * construction algorithm with inputs W, H, r_c, r_r, g, p, lambda; its steps
 * are equations 2-5 and the INT8 text after eq 7):
 *   C = H^T H / N, C_lambda = C + lambda mean(diag C) I, T_p = C_lambda^p (eq 2);
 *   rank-k core A_c B_c of W by randomized SVD, sqrt(S) to each side;
 *   A5 = Q5(A_c), B8 = Q8(B_c) (row scales); R4 = SC4(W - A_c B_c) with
 *   (row, g-group) scales (eq 3); E = W - W_d;
 *   randomized rank-r SVD of E T_p: A_w = U_r S_r, B_w = V_r^T T_p^-1 (eqs 4-5);
 *   C8 = Q8(A_w) (row scales), D8 = Q8(B_w) ((row, g-group) scales).
 * Every quantiser is symmetric: s = fp16(absmax / qmax) rounded to nearest
 * even directly from fp64, q = clamp(rint(x / s)); a zero group gets s = 0,
 * q = 0.  Arithmetic is fp64 throughout (matrix-core GEMMs).
 *
 * V, d, k, r, g  as archead_pack_load (d a multiple of 128 up to 65536;
 *                k, r <= min(V, d, 1008)).  Otherwise ARCHEAD_ESHAPE.
 * N              calibration rows, N >= 1.
 * W, H           DEVICE fp64, V x d and N x d row-major (borrowed).
 * p              the metric power: one of 1/4, 1/2, 3/4, 1 (the powers the
 *                Newton-Schulz square roots reach); else ARCHEAD_EINVAL.
 * lambda         damping, > 0.
 * power_iters    power iterations of both randomized SVDs (0..16).
 * oversample     extra columns of their Gaussian test matrices (0..64, with
 *                max(k, r) + oversample <= 1024: the sketch's eigenproblem
 *                runs in one workgroup); else ARCHEAD_EINVAL.
 * seed           seed of the test matrices (Philox4x32-10 counters).
 * A5 .. sD       DEVICE outputs in the canonical host layout of
 *                archead_pack_load (caller-allocated; the k- and r-term
 *                fields may be NULL when k = 0 / r = 0).
 * The call allocates its own working memory and waits for the stream before
 * returning (construction is not a hot path).  HIP failures -> ARCHEAD_EHIP.
 */
archead_status archead_build(int64_t V, int64_t d, int64_t k, int64_t r, int64_t g, int64_t N,
                             const double *W, const double *H, double p, double lambda,
                             int power_iters, int oversample, uint64_t seed,
                             int8_t *A5, uint16_t *sA, int8_t *B8, uint16_t *sB,
                             uint8_t *R4, uint16_t *sR, int8_t *C8, uint16_t *sC,
                             int8_t *D8, uint16_t *sD, void *hip_stream);

/*
 * archead_quantize -- the symmetric quantiser of archead_build alone
 * (ARCHead paper eq 3's Q_b; the INT8 factors after eq 7): x is DEVICE fp64
 * rows x cols row-major; each row's consecutive groups of `group` columns get
 * one fp16 scale s = fp16(absmax / (2^(bits-1) - 1)) and codes
 * q = clamp(rint(x / s), -2^(bits-1), 2^(bits-1) - 1) (s = 0, q = 0 for an
 * all-zero group).  q: DEVICE int8 rows x cols; s: DEVICE uint16 (fp16 bits)
 * rows x cols/group.  2 <= bits <= 8 and group dividing cols, else
 * ARCHEAD_EINVAL.  Enqueued on hip_stream, not waited for.
 */
archead_status archead_quantize(const double *x, int64_t rows, int64_t cols, int bits, int64_t group,
                                int8_t *q, uint16_t *s, void *hip_stream);

/*
 * archead_packed_bytes -- eq 10 of the ARCHead paper: the sum over the
 * registered packed buffers of numel x element size (A5 counted at 5 bits,
 * R4 at 4 bits, int8 fields at 8, scales at 16; each buffer rounded up to a
 * byte).  Device padding and the workspace are excluded.
 */
archead_status archead_packed_bytes(archead_t h, uint64_t *bytes);

/* archead_device_bytes -- device memory the handle holds right now
 * (packed fields with their tile padding, plus the workspace). */
archead_status archead_device_bytes(archead_t h, uint64_t *bytes);

/* archead_free -- release the handle and all its device memory (waits for the
 * device first).  NULL is accepted (no-op).  Using h afterwards is an error
 * the library detects while the memory has not been reused (ARCHEAD_EINVAL). */
archead_status archead_free(archead_t h);

/* Static text for a status code. */
const char *archead_status_string(archead_status s);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char *archead_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ARCHEAD_H */

/*
 * int8mm.h -- C ABI of the LLM.int8() mixed-precision decomposed matmul on
 * AMD Instinct MI355X (gfx950).
 *
 *     Y = X_O . W_O  (fp16 operands, fp32 accumulation)
 *       + dequant( int8(X_R) . int8(W_R) )
 *
 * O is the set of input-feature columns of X whose largest |x| over the rows
 * of this call exceeds the threshold, R the rest ("LLM.int8() notes"
 * (zwxr.cn), section 2.3, decomposition formula and threshold).  W is
 * quantized once per output channel with absmax/127 scales ("PyTorch 2.9
 * supports LLM.int8()" (yongjin360.com), section 1); X is quantized on every
 * call, one absmax/127 scale per row taken over the R columns (same page,
 * section 2, dynamic activation quantization).  Codes round half to even and
 * clamp to [-127, 127].  The int8 product accumulates exactly in int32, is
 * rescaled by a_x[m] * a_w[n] / 127^2 and the outlier product is added
 * (same page, section 3: the two parts are merged).  W_O is the dequantized
 * int8 weight fp16(fp32(Wq * a_w) / 127): the prepared weight holds no fp16
 * copy of W.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device.
 *     The caller owns all memory; the library allocates nothing, never
 *     synchronises the host and enqueues all work on `stream` (0 = the null
 *     stream).
 *   - float16 data is passed as IEEE binary16 bit patterns (int8mm_half).
 *     Every element pointer must be aligned to its element size (2 bytes
 *     for float16, 4 for float and int32; INT8MM_EINVAL otherwise).
 *   - All argument checks run on the host before anything is enqueued; a
 *     failed check returns a negative status and enqueues nothing.
 *   - HIP launch failures return INT8MM_EHIP; the error text is available
 *     from int8mm_last_hip_error() on the calling thread.
 *   - No global mutable state (the one exception is the static workspace of
 *     int8_matmul_noalloc, see there): calls on different streams with
 *     different workspaces may run concurrently.  Two calls that share a
 *     workspace must be ordered (e.g. on one stream).
 *   - A call can be captured in a HIP graph and replayed: it records only
 *     kernel launches (fills are done by kernels, never by hipMemsetAsync),
 *     and every workspace region a kernel reads was written by an earlier
 *     kernel of the same call (no counters are kept between calls).
 *   - X and Y are row-major.  The int8 operands and the fp16 outlier slices
 *     (the prepared weight Wq, and the stage outputs Xq, X_O, W_O) use the
 *     library's panel-tiled layout, built for gfx950's memory path: rows are
 *     padded to Rp = 256*ceil(R/256), each row is `row_bytes` long (ldk bytes
 *     for int8, 2*ldk bytes for fp16, ldk = int8_weight_ld(K) = K rounded up
 *     to 64), and byte b of row r sits at
 *         ((r/256)*(row_bytes/64) + b/64)*16384 + (r%256)*64 + b%64,
 *     i.e. 256-row x 64-byte blocks of 16 KiB, contiguous.  Padding columns
 *     of Wq and Xq hold zeros.  These buffers are read and written with
 *     16-byte accesses: each must be 16-byte aligned (INT8MM_EINVAL
 *     otherwise).
 */
#ifndef INT8MM_H
#define INT8MM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 bit pattern. */
typedef uint16_t int8mm_half;

/* Exported entry points (the library is built with hidden visibility). */
#define INT8MM_API __attribute__((visibility("default")))

/* Status codes (returned; nothing throws across the ABI). */
#define INT8MM_OK 0
#define INT8MM_EINVAL (-1)     /* null pointer, NaN or negative threshold   */
#define INT8MM_ESHAPE (-2)     /* negative dimension or K > INT8MM_MAX_K     */
#define INT8MM_EWORKSPACE (-3) /* workspace null, too small or misaligned    */
#define INT8MM_EHIP (-4)       /* a HIP launch failed                        */
#define INT8MM_ESCRATCH (-5)   /* int8_matmul_noalloc: shape needs more
                                  workspace than its static buffer holds     */

/* Largest K for which every int32 accumulator |sum_k q_x q_w| <= 127*127*K
 * fits in int32 (127*127*133144 = 2147479576 < 2^31). */
#define INT8MM_MAX_K 133144

/* Rows of X up to which int8_matmul takes the memory-bound decode kernel
 * (one pass over the int8 weight); larger M takes the MFMA tile GEMM. */
#define INT8MM_DECODE_MAX_M 16

/* Row length, in elements, of every [.][ldk] buffer: K rounded up to 64.
 * Returns -1 for K < 0. */
INT8MM_API int64_t int8_weight_ld(int64_t K);

/* Bytes of a prepared weight: 256*ceil(N/256) * ldk.  -1 for an invalid
 * shape. */
INT8MM_API int64_t int8_weight_bytes(int64_t N, int64_t K);

/*
 * int8_prepare_weight -- one-time per-output-channel quantization of W.
 * ("PyTorch 2.9 supports LLM.int8()", section 1: scale[n] = max|W[n,:]|/127,
 * int8 weight = round(W / scale); run once, the page's "first inference is
 * slower" one-time quantization.)
 *
 *   W        [N][K]   float16, row-major (nn.Linear [out_features][in_features]).
 *   Wq       int8_weight_bytes(N, K) bytes out, panel-tiled [Np][ldk]:
 *                     Wq[n][k] = clamp(rne(fp32(127*W[n][k]) / a_w[n]), -127, 127),
 *                     0 where a_w[n] == 0; padding rows and columns are 0.
 *   w_scale  [N]      float out: a_w[n] = max_k |W[n][k]| (the absmax itself,
 *                     not divided by 127).
 * N == 0 or K == 0 is a valid no-op (returns INT8MM_OK, nothing enqueued,
 * except that with K == 0 and N > 0 the scales are set to 0).
 * Errors: EINVAL (null pointer with N > 0), ESHAPE (N < 0, K < 0, K > MAX_K),
 * EHIP.
 */
INT8MM_API int int8_prepare_weight(const int8mm_half* W, int64_t N, int64_t K,
                        int8_t* Wq, float* w_scale, hipStream_t stream);

/*
 * int8_pack_weight -- an already-quantized weight into the prepared form.
 * ("PyTorch 2.9 supports LLM.int8()", section 1: the stored 8-bit weight is
 * its int8 codes with one scale per output channel.)  For callers that hold
 * the codes and scales of an absmax/127 per-channel quantization instead of
 * the float16 W.
 *
 *   Wq_rowmajor [N][K] int8 codes, row-major (row n = output channel n).
 *                      Codes are read as the method's range [-127, 127]; a
 *                      code of -128 is stored as -127 (the int32 bound of
 *                      INT8MM_MAX_K assumes |code| <= 127).
 *   Wq          int8_weight_bytes(N, K) bytes out, panel-tiled [Np][ldk] as
 *                      from int8_prepare_weight; padding rows and columns 0.
 * The scales are not touched: pass them to int8_matmul as w_scale, as the
 * channel absmax a_w[n] (so that W ~ Wq * a_w / 127).  For codes produced by
 * int8_prepare_weight (unpacked) the output is byte-identical to its Wq.
 * N == 0 or K == 0: nothing to do.  Errors: EINVAL (null pointer, Wq not
 * 16-byte aligned), ESHAPE, EHIP.
 */
INT8MM_API int int8_pack_weight(const int8_t* Wq_rowmajor, int64_t N, int64_t K,
                     int8_t* Wq, hipStream_t stream);

/*
 * Bytes of device workspace int8_matmul / int8_matmul_stages need for this
 * shape (sized for the worst case |O| = K).  Returns 0 for an invalid shape.
 * The workspace must be 256-byte aligned.  Its contents on entry do not
 * matter; on return they are unspecified.
 */
INT8MM_API size_t int8_matmul_workspace_size(int64_t M, int64_t K, int64_t N);

/*
 * int8_matmul -- Y = decomposed int8 matmul of X with the prepared weight.
 *
 *   X         [M][K]   float16 activations (row-major, row stride K).
 *   Wq        prepared weight (panel-tiled), w_scale [N] float: from
 *                      int8_prepare_weight.
 *   threshold          outlier threshold t >= 0 (+inf allowed): column k is an
 *                      outlier when max_m |X[m][k]| > t (strict).  t = 0 sends
 *                      every non-zero column to the fp16 path; t = +inf none.
 *   Y         [M][N]   float16 out.
 *   workspace          >= int8_matmul_workspace_size(M, K, N) bytes.
 * M == 0 or N == 0: nothing to do, returns INT8MM_OK.  K == 0: Y is zeroed.
 * Errors: EINVAL (null pointer, NaN or negative threshold), ESHAPE,
 * EWORKSPACE, EHIP.
 */
INT8MM_API int int8_matmul(const int8mm_half* X, int64_t M, int64_t K,
                const int8_t* Wq, const float* w_scale, int64_t N,
                float threshold, int8mm_half* Y,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * int8_linear -- the forward of an 8-bit linear layer with a bias
 * ("PyTorch 2.9 supports LLM.int8()", the Linear8bitLt replacement example:
 * an nn.Linear, bias included, swapped for an 8-bit layer that keeps no fp16
 * weight):
 *
 *     Y[m][n] = fp16( dequant(C)[m][n] + (X_O . W_O)[m][n] + bias[n] )
 *
 * the bias added in fp32 before the single rounding to fp16.  Same kernels,
 * arguments, workspace and errors as int8_matmul, plus:
 *   bias      [N]      float16, or NULL (then the call is int8_matmul).
 * K == 0: Y[m][n] = bias[n] (0 without a bias).
 */
INT8MM_API int int8_linear(const int8mm_half* X, int64_t M, int64_t K,
                const int8_t* Wq, const float* w_scale, int64_t N,
                const int8mm_half* bias, float threshold, int8mm_half* Y,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * int8_column_absmax -- the column maxima the outlier test compares with the
 * threshold: colmax[k] = max_m |X[m][k]| (0 when M == 0), exact, as float16.
 * The statistic behind choosing the threshold ("LLM.int8() notes", section
 * 5.1: look at the activation maxima before setting it; a column is an
 * outlier column for every t < colmax[k]).  Same kernels as the outlier
 * detection of int8_matmul.
 *
 *   X         [M][K]   float16 activations (row-major).
 *   colmax    [K]      float16 out.
 *   workspace          >= int8_matmul_workspace_size(M, K, 0) bytes, 256-byte
 *                      aligned (contents on entry do not matter).
 * K == 0: nothing to do.  Errors: EINVAL (null X with M, K > 0; null colmax
 * with K > 0), ESHAPE, EWORKSPACE, EHIP.
 */
INT8MM_API int int8_column_absmax(const int8mm_half* X, int64_t M, int64_t K,
                       int8mm_half* colmax, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * int8_outlier_counts -- |O| at several thresholds from the column maxima:
 * counts[i] = number of columns k < K with colmax[k] > thresholds[i], the
 * strict comparison of the outlier test (binary16 maximum widened to fp32).
 * What each candidate threshold would send to the fp16 path ("LLM.int8()
 * notes", section 5.1: set the threshold from the activations' statistics;
 * section 2.3: a low threshold moves many columns to fp16, a high one
 * quantizes the outliers).
 *
 *   colmax      [K]            float16 device pointer (e.g. from
 *                              int8_column_absmax); may be NULL when K == 0.
 *   thresholds  [n_thresholds] float HOST pointer, each >= 0 (+inf allowed),
 *                              copied into the launch (the caller may reuse
 *                              the array as soon as the call returns).
 *   n_thresholds               1 .. INT8MM_MAX_COUNT_THRESHOLDS.
 *   counts      [n_thresholds] int32 device pointer, out.
 * K == 0: every count is 0.  Errors: EINVAL (null thresholds or counts; null
 * colmax with K > 0; n_thresholds out of range; a NaN or negative
 * threshold; misaligned colmax or counts), ESHAPE (K < 0 or > INT8MM_MAX_K),
 * EHIP.  All checks run before anything is enqueued.
 */
#define INT8MM_MAX_COUNT_THRESHOLDS 64

INT8MM_API int int8_outlier_counts(const int8mm_half* colmax, int64_t K, const float* thresholds,
                                   int n_thresholds, int32_t* counts, hipStream_t stream);

/*
 * int8_matmul_stages -- the same kernels as int8_matmul for this shape, with
 * every intermediate of the method exposed (for verification).  Every output
 * pointer is optional (NULL = not wanted).  When C is given the matmul kernel
 * runs in its int32-output mode and Y is not produced; Y is produced only
 * when C is NULL and Y is not.
 *
 *   mask        [K]      uint8 out: 1 where column k is an outlier.
 *   n_outliers  [1]      int32 out: |O|.
 *   outlier_idx [K]      int32 out: O in ascending order (first |O| valid).
 *   Xq          [Mp][ldk] int8 out, panel-tiled: quantized X, 0 in outlier and
 *                        pad columns (rows M..Mp-1 unspecified).
 *   x_scale     [M]      float out: a_x[m] = max over R of |X[m][k]| (0 if none).
 *   X_O         [Mp][ldk] float16 out, panel-tiled (rows of 2*ldk bytes):
 *                        X_O[m][j] = X[m][O_j] for j < |O|, then zeros up to
 *                        the next multiple of 64 columns (rest unspecified).
 *   W_O         [Np][ldk] float16 out, panel-tiled: W_O[n][j] =
 *                        fp16(fp32(Wq[n][O_j]*a_w[n])/127) for j < |O|, then
 *                        zeros up to the next multiple of 64 columns.
 *   C           [M][N]   int32 out: C[m][n] = sum_k Xq[m][k] * Wq[n][k].
 *   Y           [M][N]   float16 out.
 * Errors as int8_matmul.
 */
INT8MM_API int int8_matmul_stages(const int8mm_half* X, int64_t M, int64_t K,
                       const int8_t* Wq, const float* w_scale, int64_t N,
                       float threshold,
                       uint8_t* mask, int32_t* n_outliers, int32_t* outlier_idx,
                       int8_t* Xq, float* x_scale, int8mm_half* X_O,
                       int8mm_half* W_O, int32_t* C, int8mm_half* Y,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * int8_matmul_profiled -- int8_matmul, plus two caller-created HIP events
 * that the dispatch of the matmul kernel (the tile GEMM, or the decode
 * kernel for M <= 16) stamps with its own start and end times, so that the
 * kernel's duration can be read with hipEventElapsedTime.  Either event may
 * be NULL.  Same computation, arguments and errors as int8_matmul.
 */
INT8MM_API int int8_matmul_profiled(const int8mm_half* X, int64_t M, int64_t K,
                const int8_t* Wq, const float* w_scale, int64_t N,
                float threshold, int8mm_half* Y,
                void* workspace, size_t workspace_bytes, hipStream_t stream,
                hipEvent_t matmul_start, hipEvent_t matmul_stop);

/*
 * int8_matmul_noalloc -- int8_matmul for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, with no workspace
 * argument.  The workspace is a static device buffer of the library,
 * INT8MM_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, reserved when the library's
 * device code is loaded on that GPU and held until the process ends; the
 * call allocates nothing (no hipMalloc, no allocating library routine).
 *
 *   Arguments, layouts, results and errors as int8_matmul, plus:
 *   INT8MM_ESCRATCH  the shape needs more than the buffer holds, i.e.
 *                    int8_matmul_workspace_size(M, K, N) >
 *                    int8_matmul_noalloc_max_workspace() (checked on the host
 *                    before anything is enqueued; decode shapes, M <= 16, fit
 *                    for every K; prefill shapes fit up to about 40 MiB of
 *                    X + outlier slices).
 * Every call on one GPU uses that GPU's single buffer, which keeps the last
 * call's contents: calls that overlap on one GPU (concurrent streams, or
 * host threads) race and must be ordered by the caller.  Every part of it
 * that a kernel reads was written by an earlier kernel of the same call.
 */
#define INT8MM_NOALLOC_SCRATCH_BYTES (64u << 20)

INT8MM_API int int8_matmul_noalloc(const int8mm_half* X, int64_t M, int64_t K,
                const int8_t* Wq, const float* w_scale, int64_t N,
                float threshold, int8mm_half* Y, hipStream_t stream);

/* Bytes of int8_matmul_noalloc's static workspace (the largest
 * int8_matmul_workspace_size it accepts). */
INT8MM_API size_t int8_matmul_noalloc_max_workspace(void);

/* Static text for a status code. */
INT8MM_API const char* int8mm_strerror(int status);

/* Text of the last HIP error seen by this library on the calling thread
 * ("" if none). */
INT8MM_API const char* int8mm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INT8MM_H */

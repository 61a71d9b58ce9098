/*
 * i8mp.h - C ABI of libi8mp.so, the LLM.int8() vector-wise mixed-precision
 * linear for AMD Instinct MI355X (gfx950).
 *
 * The method (transformers PR "`bitsandbytes` - `Linear8bitLt` integration
 * into `transformers` models", section "About the mixed quantization method in
 * few words"): the matmul over outlier feature columns runs in fp16, the rest
 * in int8.  The ops follow the names of the bitsandbytes PR "LLM.int8()
 * Refactoring: Part 1" (sections "Enhancements", "Deprecations", "Next steps"):
 * int8_vectorwise_quant, extract_outliers, int8_linear_matmul, int8_mm_dequant
 * and the sparse decomposition, on row-major data only, on an explicit stream,
 * with NULL allowed for optional arguments, for any shape, and capturable in a
 * graph.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device, except
 *    where a comment says "host".  fp16 tensors are IEEE binary16 bit patterns
 *    passed as void*.  Matrices are row-major with an explicit leading
 *    dimension in elements (ld >= number of columns).
 *  - The caller owns every buffer.  The library allocates nothing, never
 *    synchronizes, never reads device memory back to the host and keeps no
 *    state besides loaded code and a per-device architecture check.  All work
 *    is enqueued on `stream` (0 = the null stream), so every call can be
 *    captured into a HIP graph.
 *  - Errors are returned, never thrown or aborted on.  Arguments are checked
 *    before anything is enqueued; on a non-OK status nothing was enqueued,
 *    except for I8MP_ELAUNCH (a launch failed; earlier kernels of the same call
 *    may have been enqueued).
 *  - Sizes: m, n >= 0, k >= 1; k <= I8MP_MAX_K so that int32 accumulation of
 *    int8 products is exact.  m == 0 or n == 0 is a valid empty call.
 *    Leading dimensions of the GEMM operands and outputs (lda, ldb, ldw, ldc,
 *    ldout), of the linear's input (ldx) and the outlier capacity are at most
 *    I8MP_MAX_LD elements.
 *  - Calls that share a workspace or outputs and overlap in time race; calls
 *    on one stream are ordered.
 *
 * Numerics (the readings of the pages; the pages print no formula):
 *  - outlier columns O = { j : |x[i,j]| >= threshold for some row i }, with
 *    threshold <= 0 meaning "no outlier handling" (pure int8; also used to
 *    quantize weights);
 *  - absmax[i] = max over j not in O of |x[i,j]| (fp32, exact), 0 if none;
 *  - q[i,j] = clamp(rne(fl32(x[i,j] * fl32(127 / absmax[i]))), -127, 127), all in
 *    IEEE binary32; 0 in outlier columns and in rows with absmax 0;
 *  - out[i,n] = fp16( (w_absmax[n]/127) * (C[i,n] * absmax[i]/127 + P[i,n]) + bias[n] )
 *    with C = q . w_q^T exact in int32 and P[i,n] = sum_{j in O} x[i,j] * w_q[n,j]
 *    (the int8 weights, widened exactly), computed in fp32.
 */
#ifndef I8MP_H
#define I8MP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t i8mp_status;

#define I8MP_OK 0
#define I8MP_EINVAL -1     /* NULL required pointer, bad size, ld too small, bad cap */
#define I8MP_ERANGE -2     /* k > I8MP_MAX_K: int32 accumulation could overflow   */
#define I8MP_EWORKSPACE -3 /* workspace NULL or smaller than the query returned   */
#define I8MP_EDEVICE -4    /* current device is not gfx950, or no device          */
#define I8MP_ELAUNCH -5    /* a kernel launch failed (hipGetLastError)            */
#define I8MP_ESCRATCH -6   /* the call needs more than the fixed scratch array    */

/* floor((2^31 - 1) / 127^2): largest k whose worst-case int8 dot product fits int32. */
#define I8MP_MAX_K 133144

/* Largest leading dimension (elements) of the GEMM operands and outputs, and
 * largest outlier capacity: the kernels address a tile of up to 256 rows with
 * 32-bit byte offsets.  Larger values are I8MP_EINVAL. */
#define I8MP_MAX_LD 1048576

/* Host.  Static English text for a status code (never NULL). */
const char* i8mp_status_string(i8mp_status s);

/* Host.  ABI version of this header: (major << 16) | minor. */
int32_t i8mp_abi_version(void);


/* ------------------------------------------------------------------------- */
/* int8_vectorwise_quant: outlier-column detection + row-scale calibration +
 * int8 quantization in one op (bitsandbytes PR "LLM.int8() Refactoring:
 * Part 1", "Enhancements": fused activation scale calibration and
 * quantization; the outlier columns of the sparse decomposition).
 *
 *   x            fp16 [m x k], leading dimension ldx >= k (elements)
 *   threshold    outlier magnitude; <= 0 disables outlier handling
 *   q            int8 [m x ldq] output codes, ldq >= k; only columns [0, k) are written
 *   absmax       fp32 [m] output row absmax over non-outlier columns
 *   outlier_bitmap  optional uint32 [ceil(k/32)] output, bit (j % 32) of word
 *                j / 32 set iff column j is an outlier; may be NULL
 *   workspace    device scratch of at least i8mp_quant_workspace_bytes(m, k)
 *                bytes (the per-row-block partial outlier bitmaps of the
 *                detection); contents on entry are ignored; may be NULL iff
 *                that query returns 0 or threshold <= 0
 *
 * Weight quantization is this op with threshold <= 0 on the fp16 weight
 * [n x k]: q is the int8 weight state and absmax its per-row statistics.
 */
size_t i8mp_quant_workspace_bytes(int64_t m, int64_t k);

i8mp_status i8mp_int8_vectorwise_quant(const void* x, int64_t m, int64_t k, int64_t ldx,
                                       float threshold, int8_t* q, int64_t ldq, float* absmax,
                                       uint32_t* outlier_bitmap, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* extract_outliers: the fp16 columns X[:, O] and the sorted outlier index list
 * (bitsandbytes PR "LLM.int8() Refactoring: Part 1", "Deprecations":
 * extract_outliers; the index list the autograd function keeps for the
 * outlier columns).
 *
 *   x               fp16 [m x k], ldx >= k
 *   outlier_bitmap  uint32 [ceil(k/32)] as written by i8mp_int8_vectorwise_quant
 *   cap             capacity (>= 0) of idx and of the columns of x_out
 *   idx             int32 [cap] output: ascending outlier columns, -1 past the count
 *   count           int32 [1] output: the number of outlier columns.  It may
 *                   exceed cap: then only the first cap columns are listed and
 *                   gathered, and a caller building the linear from the
 *                   separate ops must extract again with cap >= count (cap = k
 *                   always suffices) for the method's result
 *   x_out           optional fp16 [m x ldo] output, ldo >= cap: x_out[i, s] =
 *                   x[i, idx[s]] for s < min(count, cap), 0 for the other s < cap
 */
i8mp_status i8mp_outlier_extract(const void* x, int64_t m, int64_t k, int64_t ldx,
                                 const uint32_t* outlier_bitmap, int32_t cap, int32_t* idx,
                                 int32_t* count, void* x_out, int64_t ldo, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* int8_linear_matmul (replacement of igemmlt in the bitsandbytes PR,
 * "Deprecations"): C = A . B^T exactly, int32.
 *
 *   a  int8 [m x lda], lda >= k      (activations, row-major, K contiguous)
 *   b  int8 [n x ldb], ldb >= k      (weights, nn.Linear orientation)
 *   c  int32 [m x ldc] output, ldc >= n
 * Any m, n >= 0 and 1 <= k <= I8MP_MAX_K.
 */
i8mp_status i8mp_int8_linear_matmul(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                                    int64_t m, int64_t n, int64_t k, int32_t* c, int64_t ldc,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* int8_mm_dequant with the sparse-decomposition term (bitsandbytes PR,
 * "Deprecations": mm_dequant and vectorwise_mm_dequant replaced by
 * int8_mm_dequant; "Next steps": sparse decomposition):
 *
 *   out[i,n] = fp16( (col_absmax[n]/127) * (C[i,n]*row_absmax[i]/127 + P[i,n]) + bias[n] )
 *   P[i,n]   = sum_{s < min(count, cap)} x_out[i,s] * b[n, idx[s]]   (fp32)
 *
 *   c           int32 [m x ldc], ldc >= n
 *   row_absmax  fp32 [m];  col_absmax fp32 [n]
 *   bias        optional fp16 [n] (NULL = no bias)
 *   x_out, idx, count, b   optional outlier term (all NULL, or all non-NULL):
 *               x_out fp16 [m x ldo] and idx int32 [cap] / count int32 [1] as
 *               written by i8mp_outlier_extract; b int8 [n x ldb] the int8
 *               weight with k columns (idx entries must be < k)
 *   out         fp16 [m x ldout] output, ldout >= n
 */
i8mp_status i8mp_int8_mm_dequant(const int32_t* c, int64_t ldc, const float* row_absmax,
                                 const float* col_absmax, const void* bias, int64_t m, int64_t n,
                                 const void* x_out, int64_t ldo, const int32_t* idx,
                                 const int32_t* count, int32_t cap, const int8_t* b, int64_t ldb,
                                 int64_t k, void* out, int64_t ldout, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* int8 vectorwise dequantize (bitsandbytes PR "LLM.int8() Refactoring: Part 1",
 * "Next steps": an int8 dequantize op), the inverse of the row-wise
 * quantization up to the codes' rounding:
 *
 *   out[i,j] = q[i,j] * fl32(absmax[i] / 127)   (fp32 arithmetic: IEEE quotient,
 *              one fp32 product), stored as fp16 (round to nearest even) or fp32
 *
 *   q          int8 [m x ldq], ldq >= k (e.g. codes and absmax from
 *              i8mp_int8_vectorwise_quant, or int8 weights and their w_absmax)
 *   absmax     fp32 [m], the rows' absmax
 *   out_dtype  I8MP_DTYPE_F16 or I8MP_DTYPE_F32
 *   out        fp16 or fp32 [m x ldout], ldout >= k
 *   m == 0 or k == 0 is a no-op; leading dimensions above I8MP_MAX_LD, or an
 *   unknown out_dtype, return I8MP_EINVAL.
 */
#define I8MP_DTYPE_F16 0
#define I8MP_DTYPE_F32 1
i8mp_status i8mp_int8_vectorwise_dequant(const int8_t* q, int64_t ldq, int64_t m, int64_t k,
                                         const float* absmax, int32_t out_dtype, void* out, int64_t ldout,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* The whole mixed-precision linear, fused: quantize + detect, extract, int8
 * MFMA GEMM with the dequant, outlier sub-matmul and bias in its epilogue.
 *
 *   x          fp16 [m x k], ldx >= k (ldx at most I8MP_MAX_LD)
 *   w_q        int8 [n x ldw], ldw >= k   (from i8mp_int8_vectorwise_quant, threshold <= 0)
 *   w_absmax   fp32 [n]
 *   bias       optional fp16 [n]
 *   threshold  outlier threshold (<= 0: pure int8)
 *   cap        capacity (>= 0) of the gathered outlier columns X_O in the
 *              workspace.  Every outlier column takes the fp16 path whatever
 *              the count: the epilogue reads the x values of the first cap
 *              outlier columns from X_O and those of any further column from x
 *              through the index list (slower).  The index list always holds
 *              every outlier column and the count is exact.
 *   out        fp16 [m x ldout] output, ldout >= n
 *   workspace  at least i8mp_linear_workspace(...).bytes bytes; contents on entry
 *              are ignored; after the call it holds the intermediates at the
 *              offsets the layout query reports.
 */
typedef struct i8mp_linear_workspace {
    size_t bytes;          /* total size needed                                   */
    size_t q_offset;       /* int8 codes [m x ldq], zero-padded to ldq            */
    int64_t ldq;           /* leading dimension of the codes                      */
    size_t absmax_offset;  /* fp32 [m] row absmax                                 */
    size_t bitmap_offset;  /* uint32 [ceil(k/32)] outlier bitmap                  */
    size_t idx_offset;     /* int32 [idx_len] outlier columns, ascending, -1 past
                              the count                                           */
    size_t count_offset;   /* int32 [1] outlier count                             */
    size_t xo_offset;      /* fp16 [m x cap_pad]: x of the first min(count, cap)
                              outlier columns, zero past them                     */
    int32_t cap_pad;       /* cap rounded up to the fp16 MFMA depth               */
    size_t scratch_offset; /* private: partial outlier bitmaps of the detection   */
    size_t scratch_bytes;
    int64_t idx_len;       /* entries of the index list: k rounded up to 32       */
} i8mp_linear_workspace;

i8mp_status i8mp_linear_workspace_query(int64_t m, int64_t n, int64_t k, int32_t cap,
                                        i8mp_linear_workspace* layout /* host */);

/* The two halves of i8mp_linear_forward, for callers that schedule them
 * separately (e.g. to quantize the next layer's input while this one's GEMM
 * runs on another stream, or to time the GEMM alone).  Calling
 * i8mp_linear_quantize then i8mp_linear_matmul_dequant on one stream with the
 * same workspace is exactly i8mp_linear_forward.
 *
 * i8mp_linear_quantize: outlier detection, row calibration, quantization and
 * outlier extraction of x into the workspace (arguments as for the forward).
 * i8mp_linear_matmul_dequant: the int8 MFMA GEMM of the workspace codes with
 * w_q and the fused epilogue (row/column absmax, outlier sub-matmul, bias);
 * x, m, k and cap must be those of the i8mp_linear_quantize call that filled
 * the workspace (x is read for outlier columns past cap). */
i8mp_status i8mp_linear_quantize(const void* x, int64_t m, int64_t k, int64_t ldx, float threshold,
                                 int32_t cap, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

i8mp_status i8mp_linear_matmul_dequant(const void* x, int64_t ldx, const void* workspace,
                                       size_t workspace_bytes, int64_t m, int64_t k, int32_t cap,
                                       const int8_t* w_q, int64_t ldw, const float* w_absmax, int64_t n,
                                       const void* bias, void* out, int64_t ldout, hipStream_t stream);

i8mp_status i8mp_linear_forward(const void* x, int64_t m, int64_t k, int64_t ldx,
                                const int8_t* w_q, int64_t ldw, const float* w_absmax, int64_t n,
                                const void* bias, float threshold, int32_t cap, void* out,
                                int64_t ldout, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): i8mp_linear_forward
 * with the same arguments except the workspace, which is a fixed device array
 * inside the library of I8MP_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * acquired on the first call on that GPU and held until the process ends.
 * The call allocates nothing.  A shape whose workspace (the layout query's
 * bytes for m, k and cap) exceeds the array returns I8MP_ESCRATCH and
 * enqueues nothing.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race, and the
 * intermediates of a call are overwritten by the next one. */
#define I8MP_NOALLOC_SCRATCH_BYTES (32u << 20)
i8mp_status i8mp_linear_forward_noalloc(const void* x, int64_t m, int64_t k, int64_t ldx,
                                        const int8_t* w_q, int64_t ldw, const float* w_absmax, int64_t n,
                                        const void* bias, float threshold, int32_t cap, void* out,
                                        int64_t ldout, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Backward pass through the int8 linear (training with the fp16 weight kept).
 * The bitsandbytes PR "LLM.int8() Refactoring: Part 1", in its review of
 * bitsandbytes/autograd/_functions.py, keeps a transposed int8 copy of the
 * layer input (CAt) whose outlier columns, listed by the forward's saved index,
 * are zeroed; the transformers PR page ("`bitsandbytes` - `Linear8bitLt`
 * integration into `transformers` models") notes that fine-tuning through the
 * layers works while the fp16 weights are kept.  No formula is printed; the
 * readings, in the forward's int8/fp16 split:
 *
 *  - column-wise quantization of A [r x c]: column scale s[j] = max_i |A[i,j]|
 *    (fp32, exact), code = clamp(rne(fl32(A[i,j] * fl32(127 / s[j]))), -127, 127)
 *    (0 if s[j] == 0), handed over transposed: qt[j, i] (K-contiguous);
 *  - grad_x[i,j] = fp16( (s_wt[j]/127) * (C[i,j] * s_g[i]/127) ),
 *    C = g_q . wt_q^T exact (contraction over n): g = dL/dy quantized row-wise,
 *    the weight W quantized column-wise; no outlier term;
 *  - grad_w[n,j] = fp16( (s_xt[j]/127) * (C[n,j] * s_gt[n]/127) ) for j not an
 *    outlier column, C = gt_q . xt_q^T exact (contraction over the m rows), g
 *    and x quantized column-wise with x's outlier columns zeroed;
 *    grad_w[n,j] = fp16( sum_i g[i,n] * x[i,j] ) (fp32) for the outlier columns.
 */

/* Column-wise ("transposed") int8 quantization:
 *
 *   a            fp16 [rows x lda], lda >= cols
 *   zero_idx     optional int32 [cap] columns whose codes are all 0 (their scale
 *                is still reported); only the first min(*zero_count, cap) are
 *                used (device values, e.g. the idx / count of a forward)
 *   zero_count   int32 [1], required with zero_idx
 *   qt           int8 [cols x ldqt] output, ldqt >= rows: qt[j, i] = code of
 *                a[i, j]; qt[j, i] = 0 for rows <= i < ldqt
 *   col_absmax   fp32 [cols] output
 *   workspace    at least i8mp_colwise_quant_workspace_bytes(rows, cols) bytes
 * rows >= 0, cols >= 1; ldqt at most I8MP_MAX_LD.  cols == 0 is a no-op.
 */
size_t i8mp_colwise_quant_workspace_bytes(int64_t rows, int64_t cols);
i8mp_status i8mp_int8_colwise_quant(const void* a, int64_t rows, int64_t cols, int64_t lda,
                                    const int32_t* zero_idx, const int32_t* zero_count, int32_t cap,
                                    int8_t* qt, int64_t ldqt, float* col_absmax, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Workspace of i8mp_linear_backward; after a call it holds the operands of both
 * gradient GEMMs at these offsets. */
typedef struct i8mp_backward_workspace {
    size_t bytes;          /* total size needed                                   */
    int64_t ld_n;          /* round_up(n, 128): row length of g_q and wt_q        */
    int64_t ld_m;          /* round_up(m, 128): row length of gt_q and xt_q       */
    size_t gq_offset;      /* int8 [m x ld_n] row-wise codes of g, zero-padded    */
    size_t gs_offset;      /* fp32 [m] row absmax of g                            */
    size_t wtq_offset;     /* int8 [k x ld_n] column-wise codes of W (CBt)        */
    size_t wts_offset;     /* fp32 [k] column absmax of W                         */
    size_t gtq_offset;     /* int8 [n x ld_m] column-wise codes of g              */
    size_t gts_offset;     /* fp32 [n] column absmax of g                         */
    size_t xtq_offset;     /* int8 [k x ld_m] column-wise codes of x, outlier
                              columns zeroed (CAt)                                */
    size_t xts_offset;     /* fp32 [k] column absmax of x                         */
    size_t scratch_offset; /* private: column maxima, outlier-gradient sums       */
    size_t scratch_bytes;
} i8mp_backward_workspace;

i8mp_status i8mp_linear_backward_workspace_query(int64_t m, int64_t n, int64_t k, int32_t cap,
                                                 i8mp_backward_workspace* layout /* host */);

/* Both gradients of out = x . W^T (+ bias) for grad_out = dL/dout:
 *
 *   grad_out   fp16 [m x ldg], ldg >= n
 *   x          fp16 [m x ldx], ldx >= k   (the forward's input)
 *   w          fp16 [n x ldw], ldw >= k   (the weight kept in fp16 for training;
 *              required when grad_x is requested)
 *   cap, fwd_workspace   the forward's outlier capacity and its workspace (from
 *              i8mp_linear_forward or i8mp_linear_quantize on this x with this
 *              m, k and cap), read for its outlier bitmap, index list, count
 *              and gathered outlier columns; NULL = no outlier columns.  As in
 *              the forward, every outlier column takes the fp16 path; those
 *              past cap are summed from grad_out and x directly (slower).
 *   grad_x     optional fp16 [m x ldgx] output, ldgx >= k (NULL: not computed)
 *   grad_w     optional fp16 [n x ldgw] output, ldgw >= k (NULL: not computed)
 *   workspace  at least the query's bytes
 * m, n >= 0, k >= 1; m and n at most I8MP_MAX_K (they are contraction lengths),
 * leading dimensions at most I8MP_MAX_LD.  The bias gradient is the column sum
 * of grad_out and is not part of this call.
 */
i8mp_status i8mp_linear_backward(const void* grad_out, int64_t ldg, const void* x, int64_t ldx,
                                 const void* w, int64_t ldw, int64_t m, int64_t n, int64_t k,
                                 int32_t cap, const void* fwd_workspace, size_t fwd_workspace_bytes,
                                 void* grad_x, int64_t ldgx, void* grad_w, int64_t ldgw,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Blockwise 4-bit weights (the page "Loading an LLM in 4 bits using
 * bitsandbytes", sections "Normalized Float" and "Double Quantization"): fp4
 * with 1 sign bit, 2 exponent bits and 1 mantissa bit (E2M1: magnitudes 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6), blocks of 64 weights with an fp32 scale each, and
 * double quantization of those scales to 8 bits in groups of 256.  Readings:
 *  - a block is 64 consecutive weights of a row of W [n x k], k a multiple of
 *    64; its scale A = max |w| over the block (fp32, exact);
 *  - code = sign bit of w (bit 3) | magnitude code (bits 0..2) of the E2M1
 *    value nearest to fl32(|w| * fl32(6 / A)) (ties to the even mantissa bit,
 *    saturating at 6); two codes per byte, element 2j in the low nibble of
 *    byte j of the row;
 *  - double quantization over the flattened block scales, groups of 256 (the
 *    last may be shorter): s2 = group max, c8 = clamp(rne(fl32(A * fl32(255 / s2))),
 *    0, 255); the scale used is then fl32(c8 * fl32(s2 / 255));
 *  - w' = fl32(E2M1 value * fl32(A / 6)).
 * The nf4 type has no value table on the pages and is not provided.
 */

/* codes uint8 [n x ldc], ldc >= k/2; absmax fp32 [n * k/64] (row-major blocks).
 * k must be a positive multiple of 64 (else I8MP_EINVAL); n == 0 is a no-op. */
i8mp_status i8mp_fp4_quantize(const void* w, int64_t n, int64_t k, int64_t ldw, uint8_t* codes, int64_t ldc,
                              float* absmax, hipStream_t stream);

/* c8 uint8 [nb], s2 fp32 [ceil(nb / 256)] from the block scales absmax fp32 [nb]. */
i8mp_status i8mp_fp4_double_quant(const float* absmax, int64_t nb, uint8_t* c8, float* s2, hipStream_t stream);

/* out [n x ldout], ldout >= k: w' as fp16 (I8MP_DTYPE_F16, rounded once from
 * the fp32 w') or fp32.  Scales: absmax (non-NULL, c8 and s2 NULL) or the
 * double-quantized c8 / s2 (absmax NULL). */
i8mp_status i8mp_fp4_dequantize(const uint8_t* codes, int64_t ldc, int64_t n, int64_t k, const float* absmax,
                                const uint8_t* c8, const float* s2, int32_t out_dtype, void* out, int64_t ldout,
                                hipStream_t stream);

/* The 4-bit linear for decode-sized batches:
 *   out[i, r] = fp16( sum_j x[i, j] * w'[r, j] + bias[r] )   (fp32 sums)
 * where each half block's fp32 sum of x times the E2M1 values is scaled once by
 * the block's A / 6, computed from the raw scales within a few ulp of the
 * dequantized weight's scale (far inside the sums' rounding).
 * x fp16 [m x ldx] 16-byte aligned with ldx a multiple of 8; codes 16-byte
 * aligned with ldc a multiple of 16; scales as for the dequantize; bias
 * optional fp16 [n]; out fp16 [m x ldout], ldout >= n.  Any m >= 0: every four
 * rows of x read the weights once. */
i8mp_status i8mp_fp4_linear(const void* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* codes, int64_t ldc,
                            const float* absmax, const uint8_t* c8, const float* s2, int64_t n, const void* bias,
                            void* out, int64_t ldout, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* I8MP_H */

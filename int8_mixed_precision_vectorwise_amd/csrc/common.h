// Internal definitions shared by the libi8mp translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "i8mp.h"

namespace i8mp {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint16_t half_bits;

// IEEE binary16 bits <-> fp32 (exact widening; round to nearest even when narrowing)
__device__ inline float h2f(half_bits h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ inline half_bits f2h(float f) { return __builtin_bit_cast(half_bits, (_Float16)f); }

// ---- outlier detection and quantization -------------------------------------
constexpr int kQuantThreads = 256;
constexpr int kMaxRowBlocks = 8;      // partial bitmaps written by the detect pass

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Scratch of the quantizer: kMaxRowBlocks partial outlier bitmaps of
// ceil(k/32) words each.
inline size_t quant_scratch_bytes(int64_t k) {
    return (size_t)round_up(kMaxRowBlocks * ceil_div(k, 32) * 4, 256);
}

struct QuantArgs {
    const half_bits* x;
    int64_t m, k, ldx;
    float threshold;            // > 0: outliers on
    uint32_t* partial;          // [kMaxRowBlocks x words] partial bitmaps written by detect
    const uint32_t* bitmap_in;  // row kernel: bitmaps to OR ([row_blocks x words]), null: no outliers
    int64_t row_blocks;
    int64_t words;              // ceil(k / 32)
    int8_t* q;                  // nullable: no codes
    int64_t ldq;
    int64_t kpad;               // codes in [k, kpad) are written as 0
    float* absmax;              // nullable iff q is null
    uint32_t* bitmap_out;       // nullable
    int32_t* idx_out;           // nullable
    int32_t* count_out;         // nullable
    int32_t cap;                // capacity of idx_out / x_out columns
    int32_t idx_len;            // idx entries written (>= cap, -1 padded)
    half_bits* x_out;           // nullable
    int64_t ldo;
    int32_t xo_cols;            // x_out columns written per row (>= cap, zero padded)
    int64_t rows_per_block;     // set by the launchers
};

// Detection (threshold > 0) + calibration + quantization + extraction of x.
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// The row kernel alone, with a.bitmap_in the bitmap(s) to OR (or null).
hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t stream);

struct GemmArgs {
    const int8_t* a; int64_t lda;
    const int8_t* b; int64_t ldb;
    int64_t m, n, k;
    bool a_zero_padded;                  // A rows hold zeros from k to a multiple of 128
    int32_t* c; int64_t ldc;             // int32 output (unfused)
    // fused epilogue
    const float* row_absmax;
    const float* col_absmax;
    const half_bits* bias;               // nullable
    const half_bits* x_out; int64_t ldo; // nullable: no outlier term
    const int32_t* idx;
    const int32_t* count;
    int32_t cap;
    half_bits* out; int64_t ldout;
};

hipError_t launch_gemm_i32(const GemmArgs& g, hipStream_t stream);
// m <= 16, 16-byte aligned operands, A covering whole 128-byte K chunks
hipError_t launch_decode(const GemmArgs& g, bool fused, hipStream_t stream);
hipError_t launch_gemm_fused(const GemmArgs& g, hipStream_t stream);
// The whole forward of one to four rows in one launch (quantization inside the
// GEMV's workgroups); qa / g as for launch_quantize / launch_gemm_fused with the
// same workspace.  Only where decode_forward_fits.
bool decode_forward_fits(const QuantArgs& qa, const GemmArgs& g);
hipError_t launch_decode_forward(const QuantArgs& qa, const GemmArgs& g, hipStream_t stream);

// ---- backward: column-wise quantization and the outlier weight gradient ----
// The fp16 outlier columns of grad_w: sum_i g[i, n] * x_out[i, s], summed
// per 512-row block by the column-maximum pass over g (part), then over the
// blocks into grad_w[n, idx[s]] for s < min(count, cap).
struct FixArgs {
    const half_bits* x_out;      // nullable: off.  The forward's gathered outlier columns [m x ldo],
    int64_t ldo;                 // zero past the count; ldo >= round_up(cap, 8), a multiple of 8
    const int32_t* idx;          // [cap] outlier columns
    const int32_t* count;        // [1]
    int32_t cap;
    float* part;                 // [row blocks x cap x cols_pad] fp32 block sums
    half_bits* grad_w;           // [n x ldgw]
    int64_t ldgw;
};

struct ColQuantArgs {
    const half_bits* x;          // [rows x lda]
    int64_t rows, cols, lda;
    const int32_t* zero_idx;     // nullable: columns whose codes are zeroed
    const int32_t* zero_count;   // [1], used with zero_idx
    int32_t cap;                 // entries of zero_idx considered: min(count, cap)
    int8_t* qt;                  // [cols x ldqt] transposed codes, rows .. ldqt - 1 written as 0
    int64_t ldqt;
    float* col_absmax;           // [cols]
    float* partial;              // [row blocks x cols_pad] column maxima of 512-row blocks
    FixArgs fix;                 // x = g: also the block sums of the outlier columns of grad_w
    int64_t cols_pad;            // set by the launcher
    int64_t row_blocks;          // set by the launcher
};

int64_t colquant_row_blocks(int64_t rows);
// bytes of ColQuantArgs::partial for a rows x cols input
inline size_t colquant_scratch_bytes(int64_t rows, int64_t cols) {
    return (size_t)colquant_row_blocks(rows) * (size_t)round_up(cols > 0 ? cols : 1, 64) * 4;
}
// bytes of FixArgs::part for g [m x n] and capacity cap
inline size_t fix_part_bytes(int64_t m, int64_t n, int32_t cap) {
    return (size_t)colquant_row_blocks(m) * (size_t)(cap > 0 ? cap : 1) * (size_t)round_up(n > 0 ? n : 1, 64) * 4;
}
hipError_t launch_colwise_quant(const ColQuantArgs& a, hipStream_t stream);
// grad_w[n, idx[s]] = fp16(sum of the block sums) for s < min(count, cap), once
// the column pass over g [m x n] has written them
hipError_t launch_outlier_store(const FixArgs& f, int64_t m, int64_t n, hipStream_t stream);
// out[i, j] = +0 for an fp16 rows x cols matrix (an empty contraction)
hipError_t launch_fill_f16(half_bits* out, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream);

// ---- blockwise 4-bit (FP4 E2M1) weights ------------------------------------
struct Fp4Args {
    const half_bits* w; int64_t ldw;     // quantize: fp16 weights [n x ldw]
    uint8_t* codes_out;                  // quantize: packed codes [n x ldc]
    float* absmax_out;                   // quantize: fp32 block absmax [n * k / 64]
    const uint8_t* codes; int64_t ldc;   // packed codes, element 2j in the low nibble of byte j
    const float* absmax;                 // block scales, or null with c8 / s2 (double-quantized)
    const uint8_t* c8;                   // [n * k / 64]
    const float* s2;                     // [ceil(n * k / 64 / 256)]
    const half_bits* x; int64_t ldx, m;  // linear: x [m x ldx]
    const half_bits* bias;               // linear: nullable
    void* out; int64_t ldout;
    bool half_out;                       // dequantize: fp16 (else fp32)
    int64_t n, k;                        // k a multiple of 64
};
hipError_t launch_fp4_quantize(const Fp4Args& a, hipStream_t stream);
hipError_t launch_fp4_double_quant(const float* absmax, int64_t nb, uint8_t* c8, float* s2, hipStream_t stream);
hipError_t launch_fp4_dequantize(const Fp4Args& a, hipStream_t stream);
// x 16-byte aligned with ldx a multiple of 8, codes rows 16-byte aligned (ldc a multiple of 16)
hipError_t launch_fp4_linear(const Fp4Args& a, hipStream_t stream);

struct DequantArgs {
    const int32_t* c; int64_t ldc;
    const float* row_absmax;
    const float* col_absmax;
    const half_bits* bias;
    int64_t m, n;
    const half_bits* x_out; int64_t ldo;
    const int32_t* idx;
    const int32_t* count;
    int32_t cap;
    const int8_t* b; int64_t ldb;
    half_bits* out; int64_t ldout;
};

hipError_t launch_dequant(const DequantArgs& d, hipStream_t stream);

struct VecDequantArgs {
    const int8_t* q; int64_t ldq;
    int64_t m, k;
    const float* absmax;
    void* out; int64_t ldout;
    bool half_out;                       // fp16 output, else fp32
};

hipError_t launch_vectorwise_dequant(const VecDequantArgs& d, hipStream_t stream);

}  // namespace i8mp

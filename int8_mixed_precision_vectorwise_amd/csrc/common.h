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

// ---- outlier detection / quantization plan ---------------------------------
constexpr int kQuantThreads = 256;
constexpr int kDetectCols = 256;      // columns per detect workgroup (32 lanes x 8 fp16)

struct QuantPlan {
    int64_t words;        // ceil(k / 32)
    int64_t detect_gx;    // column blocks of the detect grid
    int64_t row_blocks;   // R: row blocks of the detect grid (= partial bitmaps)
    int64_t rows_per_detect_block;
    int64_t rows_per_quant_block;
    size_t partial_bytes;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

inline QuantPlan make_quant_plan(int64_t m, int64_t k, bool detect) {
    QuantPlan p{};
    p.words = ceil_div(k, 32);
    p.detect_gx = ceil_div(k, kDetectCols);
    // rows per quant workgroup: 4 waves, one row per wave at a time; enough
    // workgroups to cover the CUs twice before giving a wave more rows
    auto quant_rows = [&](int64_t r) {
        int64_t rpb = 4 * ceil_div(r, 8);            // amortize the partial-bitmap OR
        if (rpb < 4) rpb = 4;
        while (rpb > 4 && ceil_div(m, rpb) < 512) rpb -= 4;
        return rpb;
    };
    if (!detect || m <= 0) {
        p.row_blocks = 0;
        p.rows_per_detect_block = 0;
        p.rows_per_quant_block = quant_rows(0);
        p.partial_bytes = 0;
        return p;
    }
    // row blocks of the detect grid: about 1024 workgroups, at least 8 rows each,
    // at most 32 partials (the OR every quant workgroup does is R words per word)
    int64_t r = ceil_div(1024, p.detect_gx);
    if (r > 32) r = 32;
    const int64_t r_rows = ceil_div(m, 8);
    if (r > r_rows) r = r_rows;
    if (r < 1) r = 1;
    const int64_t rb = round_up(ceil_div(m, r), 8);
    r = ceil_div(m, rb);
    p.row_blocks = r;
    p.rows_per_detect_block = rb;
    p.rows_per_quant_block = quant_rows(r);
    p.partial_bytes = (size_t)(r * p.words) * sizeof(uint32_t);
    return p;
}

// ---- kernel launchers (defined in the .hip files) ---------------------------
struct QuantArgs {
    const half_bits* x;
    int64_t m, k, ldx;
    float threshold;            // > 0: outliers on
    const uint32_t* partial;    // [row_blocks x words] partial bitmaps (or the final bitmap, row_blocks = 1)
    int64_t row_blocks;
    int64_t words;
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
    int64_t rows_per_block;
};

hipError_t launch_detect(const half_bits* x, int64_t m, int64_t k, int64_t ldx, float threshold,
                         const QuantPlan& plan, uint32_t* partial, hipStream_t stream);
hipError_t launch_quant(const QuantArgs& a, hipStream_t stream);

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

}  // namespace i8mp

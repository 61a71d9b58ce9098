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
    int32_t* idx_out;           // nullable: the outlier columns, ascending
    int32_t* count_out;         // nullable
    int32_t cap;                // x_out holds the values of the first cap outlier columns
    int32_t idx_len;            // idx entries written: the first idx_len columns, -1 past the count
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
    // outlier sub-matmul, on iff count is non-null: slot s < count has column
    // idx[s] (idx holds idx_len >= count entries); its x values come from
    // x_out[:, s] for s < cap (zero from the count to ldo), from x[:, idx[s]]
    // past cap
    const int32_t* count;
    const int32_t* idx; int32_t idx_len;
    const half_bits* x_out; int64_t ldo; // nullable iff cap == 0
    int32_t cap;
    const half_bits* x; int64_t ldx;     // the layer input
    half_bits* out; int64_t ldout;
};

// x value of outlier slot s of activation row r (see GemmArgs)
__device__ inline float outlier_x(const GemmArgs& g, int64_t r, int s) {
    return h2f(s < g.cap ? g.x_out[r * g.ldo + s] : g.x[r * g.ldx + g.idx[s]]);
}
// number of outlier slots of the fused epilogue: the device count, bounded by
// the index list it is read from
__device__ inline int outlier_count(const GemmArgs& g, int c) {
    return c < 0 ? 0 : (c > g.idx_len ? g.idx_len : c);
}

hipError_t launch_gemm_i32(const GemmArgs& g, hipStream_t stream);
// m <= 16, 16-byte aligned operands, A covering whole 128-byte K chunks
hipError_t launch_decode(const GemmArgs& g, bool fused, hipStream_t stream);
hipError_t launch_gemm_fused(const GemmArgs& g, hipStream_t stream);
// The whole forward of one or two rows in one launch (quantization inside the
// GEMV's workgroups); qa / g as for launch_quantize / launch_gemm_fused with the
// same workspace.  Only where decode_forward_fits.
bool decode_forward_fits(const QuantArgs& qa, const GemmArgs& g);
hipError_t launch_decode_forward(const QuantArgs& qa, const GemmArgs& g, hipStream_t stream);

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

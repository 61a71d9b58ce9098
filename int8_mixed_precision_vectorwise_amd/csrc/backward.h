// Internal declarations of the backward (column-wise quantization, outlier weight gradient) kernels (gfx950 only).
#pragma once

#include "common.h"

namespace i8mp {

// ---- backward: column-wise quantization and the outlier weight gradient ----
// The fp16 outlier columns of grad_w, grad_w[n, idx[s]] = sum_i g[i, n] * x[i, idx[s]]
// for every slot s < count: for s < cap summed per 512-row block by the
// column-maximum pass over g from the forward's gathered columns (part), then
// over the blocks; past cap summed over the rows of g and x directly.
struct FixArgs {
    const half_bits* x_out;      // nullable (cap == 0).  The forward's gathered outlier columns [m x ldo],
    int64_t ldo;                 // zero past the count; ldo >= round_up(cap, 8), a multiple of 8
    const int32_t* idx;          // nullable: off.  [idx_len] outlier columns, ascending
    int32_t idx_len;
    const int32_t* count;        // [1]
    int32_t cap;
    float* part;                 // [row blocks x cap x cols_pad] fp32 block sums
    half_bits* grad_w;           // [n x ldgw]
    int64_t ldgw;
    const half_bits* g; int64_t ldg;   // [m x ldg] upstream gradient (slots past cap)
    const half_bits* x; int64_t ldx;   // [m x ldx] layer input (slots past cap)
};

struct ColQuantArgs {
    const half_bits* x;          // [rows x lda]
    int64_t rows, cols, lda;
    const int32_t* zero_idx;     // nullable: columns whose codes are zeroed
    const int32_t* zero_count;   // [1], used with zero_idx
    int32_t cap;                 // entries of zero_idx considered: min(count, cap)
    const uint32_t* zero_bitmap; // nullable: columns whose bit is set get zero codes too
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
// grad_w[n, idx[s]] for every outlier slot s, once the column pass over g
// [m x n] has written the block sums of the slots below cap
hipError_t launch_outlier_store(const FixArgs& f, int64_t m, int64_t n, hipStream_t stream);
// out[i, j] = +0 for an fp16 rows x cols matrix (an empty contraction)
hipError_t launch_fill_f16(half_bits* out, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream);

}  // namespace i8mp

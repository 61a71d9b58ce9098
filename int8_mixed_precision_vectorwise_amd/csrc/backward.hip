// Kernels of the backward pass through the int8 linear:
//  - column-wise ("transposed") int8 quantization: a column-maximum pass and a
//    code pass that writes the codes transposed (the K-contiguous operand
//    layout of the int8 GEMM), with listed columns zeroed (the CAt of the
//    bitsandbytes PR "LLM.int8() Refactoring: Part 1", its review of
//    bitsandbytes/autograd/_functions.py);
//  - the fp16 outlier columns of the weight gradient, sum_i g[i, n] * x[i, j]
//    for j in the forward's outlier list.
// The two gradient GEMMs themselves are the forward's int8 GEMM with its
// dequant epilogue (gemm.hip), called from api.hip.
#include "common.h"
#include "backward.h"
#include "quant_util.h"

namespace i8mp {

namespace {

// A workgroup of 4 waves covers 64 columns x 512 rows; lane l of a wave takes
// the 8 columns (l & 7) * 8 .. + 8 of 16 consecutive rows, so one lane's codes
// of one column are 16 consecutive bytes of a transposed row.
constexpr int kStripCols = 64;
constexpr int kLaneRows = 16;
constexpr int kWaveRows = 8 * kLaneRows;        // 128
constexpr int kBlockRows = 4 * kWaveRows;       // 512

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// per-half maximum of two words of fp16 magnitudes (non-negative fp16 bit
// patterns order like unsigned integers)
__device__ inline uint32_t umax16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

__device__ inline uint4 umax16x8(const uint4& a, const uint4& b) {
    return make_uint4(umax16x2(a.x, b.x), umax16x2(a.y, b.y), umax16x2(a.z, b.z), umax16x2(a.w, b.w));
}

__device__ inline uint4 shfl_xor4(const uint4& v, int off) {
    return make_uint4(__shfl_xor(v.x, off, 64), __shfl_xor(v.y, off, 64), __shfl_xor(v.z, off, 64),
                      __shfl_xor(v.w, off, 64));
}

// The 16 row chunks of one lane: rows r0 .. r0 + 15, columns c .. c + 7 of x
// (rows >= rows and columns >= cols read as 0).  kVec: 16-byte loads (cols and
// lda multiples of 8, 16-byte aligned base), so a chunk is all in or all out.
template <bool kVec>
__device__ inline void load_lane_rows(const ColQuantArgs& a, int64_t r0, int64_t c, uint4 (&v)[kLaneRows]) {
#pragma unroll
    for (int j = 0; j < kLaneRows; ++j) {
        const int64_t r = r0 + j;
        v[j] = (r < a.rows && c < a.cols) ? load8<kVec>(a.x + r * a.lda, c, a.cols) : make_uint4(0, 0, 0, 0);
    }
}

// Block sums of the fp16 outlier columns of grad_w while g's rows are in
// registers: part[blockIdx.y][s][col] = sum over the block's rows r of
// g[r, col] * x_out[r, s] in fp32, in a fixed order: each lane takes its 16
// rows in pairs with v_dot2_f32_f16 (two exact fp16 products added into an
// fp32 accumulator), lane pairs one row-lane apart are added (DPP), then the
// 16 row groups of the workgroup in order.  Slots go 8 at a time.
__device__ inline float dpp_ror8(float v) {  // lane i <- lane (i + 8) mod 16 of its row: lane i ^ 8
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf,
                                                                 false));
}

__device__ inline void fix_block_sums(const ColQuantArgs& a, const uint4 (&v)[kLaneRows], int64_t r0, int cc,
                                      int rl, int wave, int tid) {
    const FixArgs& f = a.fix;
    int32_t cnt = *f.count;
    if (cnt > f.cap) cnt = f.cap;
    __shared__ float red[16][8][kStripCols];  // [row group][slot][column of the strip]
    for (int32_t s0 = 0; s0 < cnt; s0 += 8) {
        float acc[8][8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[s][e] = 0.0f;
#pragma unroll
        for (int jp = 0; jp < kLaneRows / 2; ++jp) {
            uint32_t xw[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t r = r0 + 2 * jp + h;
                // x_out has ldo >= round_up(cap, 8) columns, zero past the count
                const uint4 xv = r < a.rows ? *reinterpret_cast<const uint4*>(f.x_out + r * f.ldo + s0)
                                            : make_uint4(0, 0, 0, 0);
                xw[h][0] = xv.x; xw[h][1] = xv.y; xw[h][2] = xv.z; xw[h][3] = xv.w;
            }
            const uint4 g0 = v[2 * jp], g1 = v[2 * jp + 1];
            const uint32_t gw[2][4] = {{g0.x, g0.y, g0.z, g0.w}, {g1.x, g1.y, g1.z, g1.w}};
            // (value of row 2jp, value of row 2jp + 1) per slot and per column
            h2_t xp[8], gp[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                xp[2 * w] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(xw[1][w], xw[0][w], 0x05040100u));
                xp[2 * w + 1] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(xw[1][w], xw[0][w], 0x07060302u));
                gp[2 * w] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(gw[1][w], gw[0][w], 0x05040100u));
                gp[2 * w + 1] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(gw[1][w], gw[0][w], 0x07060302u));
            }
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[s][e] = __builtin_amdgcn_fdot2(gp[e], xp[s], acc[s][e], false);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[s][e] += dpp_ror8(acc[s][e]);
        if ((rl & 1) == 0) {
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) red[wave * 4 + (rl >> 1)][s][cc * 8 + e] = acc[s][e];
        }
        __syncthreads();
        for (int o = tid; o < 8 * kStripCols; o += 256) {
            const int s = o / kStripCols, ci = o % kStripCols;
            float t = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) t += red[q][s][ci];
            const int64_t col = (int64_t)blockIdx.x * kStripCols + ci;
            if (s0 + s < cnt && col < a.cols)
                f.part[((int64_t)blockIdx.y * f.cap + s0 + s) * a.cols_pad + col] = t;
        }
        __syncthreads();
    }
}

// Pass 1: maxima of |x| per column over each 512-row block,
// partial[blockIdx.y][col] (fp32, exact); kFix: also the block sums above.
template <bool kVec, bool kFix>
__global__ __launch_bounds__(256) void colmax_kernel(ColQuantArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cc = lane & 7, rl = lane >> 3;
    const int64_t c = (int64_t)blockIdx.x * kStripCols + cc * 8;
    const int64_t r0 = (int64_t)blockIdx.y * kBlockRows + wave * kWaveRows + rl * kLaneRows;
    uint4 v[kLaneRows];
    load_lane_rows<kVec>(a, r0, c, v);
    const uint4 mag = make_uint4(0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu);
    uint4 mx = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kLaneRows; ++j)
        mx = umax16x8(mx, make_uint4(v[j].x & mag.x, v[j].y & mag.y, v[j].z & mag.z, v[j].w & mag.w));
    // the 8 row lanes of a column chunk differ in lane bits 3..5
    mx = umax16x8(mx, shfl_xor4(mx, 8));
    mx = umax16x8(mx, shfl_xor4(mx, 16));
    mx = umax16x8(mx, shfl_xor4(mx, 32));
    __shared__ uint4 red[4][8];
    if (rl == 0) red[wave][cc] = mx;
    __syncthreads();
    if (tid < kStripCols) {
        const int q = tid >> 3, e = tid & 7;
        uint4 m = umax16x8(umax16x8(red[0][q], red[1][q]), umax16x8(red[2][q], red[3][q]));
        const int64_t col = (int64_t)blockIdx.x * kStripCols + tid;
        if (col < a.cols) a.partial[(int64_t)blockIdx.y * a.cols_pad + col] = h2f(half_at(m, e));
    }
    if constexpr (kFix) fix_block_sums(a, v, r0, cc, rl, wave, tid);
}

// Pass 2: codes of x^T.  Column scale s = max over the partial maxima, inv =
// fl32(127 / s) (0 for a zero column or a listed one), code = rne(fl32(x * inv))
// as in the row quantizer (|x| <= s keeps the product in [-127, 127]).  Rows
// rows .. ldqt - 1 of the transposed codes are written as 0.
template <bool kVecIn, bool kVecOut>
__global__ __launch_bounds__(256) void colquant_kernel(ColQuantArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cc = lane & 7, rl = lane >> 3;
    const int64_t c = (int64_t)blockIdx.x * kStripCols + cc * 8;
    const int64_t r0 = (int64_t)blockIdx.y * kBlockRows + wave * kWaveRows + rl * kLaneRows;
    if (c >= a.cols) return;  // no barrier below
    // the rows first (their latency hides behind the scale computation); a
    // lane past ldqt loads nothing but may still write the column scales
    const bool live = r0 < a.ldqt;
    uint4 v[kLaneRows];
    if (live) load_lane_rows<kVecIn>(a, r0, c, v);

    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0f;
    for (int64_t rb = 0; rb < a.row_blocks; ++rb) {
        const float4* p = reinterpret_cast<const float4*>(a.partial + rb * a.cols_pad + c);
        const float4 p0 = p[0], p1 = p[1];
        s[0] = fmaxf(s[0], p0.x); s[1] = fmaxf(s[1], p0.y); s[2] = fmaxf(s[2], p0.z); s[3] = fmaxf(s[3], p0.w);
        s[4] = fmaxf(s[4], p1.x); s[5] = fmaxf(s[5], p1.y); s[6] = fmaxf(s[6], p1.z); s[7] = fmaxf(s[7], p1.w);
    }
    uint32_t zmask = 0;
    if (a.zero_bitmap) zmask = (a.zero_bitmap[c >> 5] >> (c & 31)) & 0xffu;  // c % 8 == 0
    if (a.zero_idx) {
        int32_t nz = *a.zero_count;
        if (nz > a.cap) nz = a.cap;
        for (int32_t t = 0; t < nz; ++t) {
            const int64_t d = (int64_t)a.zero_idx[t] - c;
            if (d >= 0 && d < 8) zmask |= 1u << d;
        }
    }
    float inv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        inv[e] = (s[e] > 0.0f && !((zmask >> e) & 1u)) ? 127.0f / s[e] : 0.0f;  // IEEE division
    if (blockIdx.y == 0 && wave == 0 && rl == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (c + e < a.cols) a.col_absmax[c + e] = s[e];
    }
    if (!live) return;

#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (c + e >= a.cols) break;
        // fl32(fl32(x * inv) + 1.5 * 2^23): the low byte is the code (two
        // roundings, no fused multiply-add)
        uint32_t b[kLaneRows];
        {
#pragma clang fp contract(off)
#pragma unroll
            for (int j = 0; j < kLaneRows; ++j) {
                const float p = h2f(half_at(v[j], e)) * inv[e];
                b[j] = __builtin_bit_cast(uint32_t, p + 12582912.0f);
            }
        }
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
            w[d] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[4 * d + 3], b[4 * d + 2], 0x0c0c0400u),
                                         __builtin_amdgcn_perm(b[4 * d + 1], b[4 * d], 0x0c0c0400u), 0x05040100u);
        int8_t* dst = a.qt + (c + e) * a.ldqt + r0;
        if (kVecOut) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
            for (int j = 0; j < kLaneRows; ++j)
                if (r0 + j < a.ldqt) dst[j] = (int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xffu);
        }
    }
}

// grad_w[col, idx[s]]: for s < cap the fp16 of the sum over the row blocks of
// the block sums, in row-block order; past cap (more outlier columns than the
// forward gathered) the fp32 sum over the rows, in row order, of g[i, col] *
// x[i, idx[s]] (exact fp16 products)
__global__ __launch_bounds__(256) void fix_store_kernel(FixArgs f, int64_t m, int64_t n, int64_t cols_pad,
                                                        int64_t row_blocks) {
    int32_t cnt = *f.count;
    cnt = cnt < 0 ? 0 : (cnt > f.idx_len ? f.idx_len : cnt);
    const int32_t kept = cnt < f.cap ? cnt : f.cap;
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= n) return;
    for (int32_t s = blockIdx.y; s < cnt; s += gridDim.y) {
        const int32_t j = f.idx[s];
        float t = 0.0f;
        if (s < kept) {
            for (int64_t rb = 0; rb < row_blocks; ++rb) t += f.part[(rb * f.cap + s) * cols_pad + col];
        } else {
            for (int64_t i = 0; i < m; ++i) t = fmaf(h2f(f.g[i * f.ldg + col]), h2f(f.x[i * f.ldx + j]), t);
        }
        f.grad_w[col * f.ldgw + j] = f2h(t);
    }
}

__global__ __launch_bounds__(256) void fill_f16_kernel(half_bits* out, int64_t rows, int64_t cols, int64_t ld) {
    const int64_t total = rows * cols;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256)
        out[(t / cols) * ld + t % cols] = 0;
}

}  // namespace

hipError_t launch_fill_f16(half_bits* out, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    int64_t blocks = ceil_div(rows * cols, 256);
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(fill_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, rows, cols, ld);
    return hipGetLastError();
}

int64_t colquant_row_blocks(int64_t rows) { return ceil_div(rows > 0 ? rows : 1, kBlockRows); }

hipError_t launch_colwise_quant(const ColQuantArgs& in, hipStream_t stream) {
    ColQuantArgs a = in;
    a.cols_pad = round_up(a.cols, kStripCols);
    a.row_blocks = colquant_row_blocks(a.rows);
    const bool vec_in = a.cols % 8 == 0 && a.lda % 8 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;
    const bool vec_out = a.ldqt % 16 == 0 && (reinterpret_cast<uintptr_t>(a.qt) & 15) == 0;
    const unsigned gx = (unsigned)ceil_div(a.cols, kStripCols);
    if (a.rows > 0) {
        const dim3 grid(gx, (unsigned)a.row_blocks);
        const bool fix = a.fix.x_out != nullptr && a.fix.cap > 0;
        if (vec_in && fix)
            hipLaunchKernelGGL((colmax_kernel<true, true>), grid, dim3(256), 0, stream, a);
        else if (vec_in)
            hipLaunchKernelGGL((colmax_kernel<true, false>), grid, dim3(256), 0, stream, a);
        else if (fix)
            hipLaunchKernelGGL((colmax_kernel<false, true>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((colmax_kernel<false, false>), grid, dim3(256), 0, stream, a);
    } else {
        // no rows: every column scale is 0 (one zero partial row)
        a.row_blocks = 0;
    }
    // at least one row block: it writes the column scales even when ldqt == 0
    const dim3 grid(gx, (unsigned)(a.ldqt > 0 ? ceil_div(a.ldqt, kBlockRows) : 1));
    if (vec_in && vec_out)
        hipLaunchKernelGGL((colquant_kernel<true, true>), grid, dim3(256), 0, stream, a);
    else if (vec_in)
        hipLaunchKernelGGL((colquant_kernel<true, false>), grid, dim3(256), 0, stream, a);
    else if (vec_out)
        hipLaunchKernelGGL((colquant_kernel<false, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((colquant_kernel<false, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_outlier_store(const FixArgs& f, int64_t m, int64_t n, hipStream_t stream) {
    if (!f.idx || m <= 0 || n <= 0) return hipSuccess;
    // the count is on the device: 32 slot strides cover any count
    const dim3 grid((unsigned)ceil_div(n, 256), 32u);
    hipLaunchKernelGGL(fix_store_kernel, grid, dim3(256), 0, stream, f, m, n, round_up(n, kStripCols),
                       colquant_row_blocks(m));
    return hipGetLastError();
}

}  // namespace i8mp

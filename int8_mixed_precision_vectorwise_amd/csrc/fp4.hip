// Blockwise 4-bit (FP4, E2M1) weights: quantization in blocks of 64 with an
// fp32 absmax per block, 8-bit double quantization of the block scales in
// groups of 256, dequantization, and the decode linear (one to four rows of
// x against 4-bit weights).  The format and the two block sizes are those of
// the page "Loading an LLM in 4 bits using bitsandbytes" (sections "Normalized
// Float" and "Double Quantization"): 1 sign bit, 2 exponent bits, 1 mantissa bit.
#include "common.h"
#include "fp4.h"
#include "quant_util.h"

namespace i8mp {

namespace {

constexpr int kBlk = 64;     // weights per block scale
constexpr int kDqGroup = 256;  // block scales per double-quantization group

typedef _Float16 hh2 __attribute__((ext_vector_type(2)));

// Magnitude code (0..7) of a non-negative fp32 value: the nearest of 0, 0.5,
// 1, 1.5, 2, 3, 4, 6, ties to the even code (the mantissa bit), saturating at
// 6.  A value exactly between two neighbours goes up only where the upper
// neighbour's code is even (0.75, 1.75, 3.5).
__device__ inline uint32_t e2m1_mag(float v) {
    return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) + (uint32_t)(v >= 1.75f) +
           (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) + (uint32_t)(v > 5.0f);
}

// fp32 value of a 4-bit code from its bits: exponent field e (bias 1), mantissa m
__device__ inline float e2m1_f32(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3f000000u : 0u);
    return __uint_as_float(mag | ((c & 8u) << 28));
}

// Block scale A of block blk (flattened): the fp32 absmax, or the double-
// quantized fl32(c8 * fl32(s2 / 255)).
__device__ inline float block_scale(const Fp4Args& a, int64_t blk) {
    if (a.absmax) return a.absmax[blk];
    const float step = a.s2[blk / kDqGroup] / 255.0f;
    return (float)a.c8[blk] * step;
}

// The factor fl32(A / 6) that the decode linear applies to a half block's fp32
// sum, from the raw scale values: the absmax sa times fl32(1 / 6), or, when
// double-quantized (A = c8 * s2 / 255, sa = s2), c8 * (s2 * fl32(1 / 1530)).
// Three roundings of relative size 2^-24 each, so within a few ulp of
// fl32(fl32(c8 * fl32(s2 / 255)) / 6), the weight the dequantize op builds: far
// inside the rounding of the fp32 sums, and a few operations per chunk instead
// of an IEEE division sequence.
template <bool kDq>
__device__ inline float fp4_factor(float sa, uint32_t c8) {
    return kDq ? (float)c8 * (sa * (1.0f / 1530.0f)) : sa * (1.0f / 6.0f);
}

// One lane per 8 weights, 8 lanes per block: absmax, codes, packed nibbles
// (element 2j in the low nibble of byte j).
template <bool kVec>
__global__ __launch_bounds__(256) void fp4_quant_kernel(Fp4Args a) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t kb = a.k / kBlk;
    const int64_t blk = t >> 3;
    const int part = (int)(t & 7);
    const bool live = blk < a.n * kb;
    const int64_t row = live ? blk / kb : 0, b = live ? blk % kb : 0;
    const int64_t col = b * kBlk + part * 8;
    const uint4 v = live ? load8<kVec>(a.w + row * a.ldw, col, a.k) : make_uint4(0, 0, 0, 0);
    float mx = chunk_absmax(v);
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));   // the 8 lanes of a block are 8 consecutive lanes
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    if (!live) return;
    const float inv = mx > 0.0f ? 6.0f / mx : 0.0f;  // IEEE division
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const half_bits h = half_at(v, e);
        const float f = fabsf(h2f(h)) * inv;
        packed |= (e2m1_mag(f) | ((uint32_t)(h >> 15) << 3)) << (4 * e);
    }
    uint8_t* dst = a.codes_out + row * a.ldc + col / 2;
    if (kVec) {
        *reinterpret_cast<uint32_t*>(dst) = packed;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = (uint8_t)(packed >> (8 * j));
    }
    if (part == 0) a.absmax_out[blk] = mx;
}

// One workgroup per group of 256 block scales.
__global__ __launch_bounds__(256) void fp4_dq_kernel(const float* absmax, int64_t nb, uint8_t* c8, float* s2) {
    const int64_t i = (int64_t)blockIdx.x * kDqGroup + threadIdx.x;
    const float v = i < nb ? absmax[i] : 0.0f;
    __shared__ float red[4];
    const float w = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
    __syncthreads();
    const float s = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float inv = s > 0.0f ? 255.0f / s : 0.0f;  // IEEE division
    if (i < nb) c8[i] = (uint8_t)fminf(fmaxf(__builtin_rintf(v * inv), 0.0f), 255.0f);
    if (threadIdx.x == 0) s2[blockIdx.x] = s;
}

// One lane per 8 weights: w' = fl32(E2M1 value * fl32(A / 6)), stored as fp32
// or rounded to fp16.
__global__ __launch_bounds__(256) void fp4_dequant_kernel(Fp4Args a) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t kb = a.k / kBlk;
    const int64_t blk = t >> 3;
    if (blk >= a.n * kb) return;
    const int64_t row = blk / kb, col = (blk % kb) * kBlk + (t & 7) * 8;
    const uint8_t* src = a.codes + row * a.ldc + col / 2;
    const uint32_t packed = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) |
                            ((uint32_t)src[3] << 24);
    const float d = block_scale(a, blk) / 6.0f;
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = e2m1_f32((packed >> (4 * e)) & 15u) * d;
    if (a.half_out) {
        half_bits* o = static_cast<half_bits*>(a.out) + row * a.ldout + col;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = f2h(w[e]);
    } else {
        float* o = static_cast<float*>(a.out) + row * a.ldout + col;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = w[e];
    }
}

// The decode linear: out[i, n] = fp16(sum_k x[i, k] * w'[n, k] + bias[n]) for
// M rows of x, where x is too long for LDS (k > 16384; shorter rows take the
// LDS-x kernels below).  A workgroup takes kRows weight rows; its 256 lanes split each
// row into 16-byte code chunks (32 weights, half a block), lane t taking chunks
// t, t + 256, ..., the same chunks of all kRows rows, so the lane's x chunk is
// read once for them.  The next chunk's codes are requested before the current
// one is used.  The hardware conversion turns a code byte into two exact fp16
// E2M1 values (scale 1); v_dot2_f32_f16 adds their products with x into an
// fp32 sum per half block, which is then scaled by fl32(A / 6).  Lane sums are
// reduced in the wave (DPP), then over the 4 waves in LDS.
// weight rows per workgroup: 4 for three or more rows of x (fewer registers,
// two waves per SIMD at four rows of x), 8 otherwise
template <int M>
constexpr int fp4_rows() { return M >= 3 ? 4 : 8; }

// Everything one chunk needs, loaded together: the codes of the kRows rows,
// the lane's x chunk, and the raw block-scale values (converted only where
// they are used, so that no load is waited for early).
template <int M, int R>
struct Fp4Chunk {
    uint4 cv[R];
    uint4 xv[M][4];
    float sa[R];          // absmax, or the group maximum s2 when double-quantized
    uint32_t c8[R];       // double-quantized scale code
};

template <int M, int R>
__device__ inline void fp4_load(const Fp4Args& a, int64_t n0, int64_t c, int64_t kb, Fp4Chunk<M, R>& t) {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) t.xv[m][q] = *reinterpret_cast<const uint4*>(a.x + m * a.ldx + c * 32 + q * 8);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool live = n0 + r < a.n;
        const int64_t blk = live ? (n0 + r) * kb + c / 2 : 0;
        t.cv[r] = live ? *reinterpret_cast<const uint4*>(a.codes + (n0 + r) * a.ldc + c * 16) : make_uint4(0, 0, 0, 0);
        if (a.absmax) {
            t.sa[r] = a.absmax[blk];
            t.c8[r] = 0;
        } else {
            t.sa[r] = a.s2[blk / kDqGroup];
            t.c8[r] = a.c8[blk];
        }
    }
}

template <int M, int R>
__device__ inline void fp4_compute(const Fp4Args& a, const Fp4Chunk<M, R>& t, int64_t n0, float (&acc)[R][M]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (n0 + r >= a.n) break;  // the same for the whole workgroup
        const float d = a.absmax ? fp4_factor<false>(t.sa[r], 0) : fp4_factor<true>(t.sa[r], t.c8[r]);
        const uint32_t cw[4] = {t.cv[r].x, t.cv[r].y, t.cv[r].z, t.cv[r].w};
        float part[M];
#pragma unroll
        for (int m = 0; m < M; ++m) part[m] = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hh2 wv[4];
            wv[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 0);
            wv[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 1);
            wv[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 2);
            wv[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 3);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint32_t xq[4] = {t.xv[m][q].x, t.xv[m][q].y, t.xv[m][q].z, t.xv[m][q].w};
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    part[m] = __builtin_amdgcn_fdot2(wv[b], __builtin_bit_cast(hh2, xq[b]), part[m], false);
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = fmaf(part[m], d, acc[r][m]);
    }
}

template <int M>
__global__ __launch_bounds__(256) void fp4_gemv_kernel(Fp4Args a) {
    constexpr int kRows = fp4_rows<M>();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t chunks = a.k / 32, kb = a.k / kBlk;
    const int64_t n0 = (int64_t)blockIdx.x * kRows;
    float acc[kRows][M];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
    int64_t c = tid;
    if (c < chunks) {
        Fp4Chunk<M, kRows> cur, nxt;
        fp4_load(a, n0, c, kb, cur);
        for (;;) {
            const int64_t cn = c + 256;
            const bool more = cn < chunks;
            if (more) fp4_load(a, n0, cn, kb, nxt);  // issued before the current chunk is used
            fp4_compute(a, cur, n0, acc);
            if (!more) break;
            cur = nxt;
            c = cn;
        }
    }
    __shared__ float red[4][kRows * M];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float s = wave_sum_f32(acc[r][m]);
            if (lane == 0) red[wave][r * M + m] = s;
        }
    __syncthreads();
    if (tid < kRows * M) {
        const int r = tid / M, m = tid % M;
        const int64_t row = n0 + r;
        if (row < a.n) {
            const float s = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
            const float b = a.bias ? h2f(a.bias[row]) : 0.0f;
            static_cast<half_bits*>(a.out)[m * a.ldout + row] = f2h(s + b);
        }
    }
}

// The decode linear with x staged in LDS, taken for one row of x: a grid of
// one or two workgroups per CU (two when x fits 64 KB), each of 8 waves.  A
// workgroup copies its M rows of x into LDS once (direct-to-LDS DMA, in 4 KB
// blocks, zero past the row); then every wave takes whole weight rows (wave v
// of the grid: rows v, v + nw, ...), so the grid sweeps a band of neighbouring
// rows at a time.  A lane takes the 16-byte code chunks lane, lane + 64, ...
// (CPL of them, the fewest that cover the row; 32 weights each, half a block)
// and reads the matching x from LDS (for its first 1 to 3 slots from registers
// loaded from there once); per row the 64 lane sums meet in a DPP
// reduction and lane 0 writes the M outputs.  As soon as a chunk of the
// current row has been converted, the same chunk of the wave's next row is
// requested into its registers, so CPL chunks are always in flight.  Each code
// byte is read once from HBM and x once per workgroup from L2 (the L2-x kernel
// above reads x again for every group of 4 or 8 weight rows).  Chunks past the
// row read zero codes through the row's buffer range, against the zeros of
// the x block's tail.
constexpr int kFp4Waves = 8;
typedef unsigned v4u_l __attribute__((ext_vector_type(4)));

// the buffer ranges of one weight row's codes and block scales (empty past n)
struct Fp4RowSrc {
    __amdgpu_buffer_rsrc_t codes, scales, s2;
    int64_t b0;   // first block of the row
    uint32_t g0;  // the same, as the 32-bit base of the group index: the launcher
                  // takes the kernels that use it only where n k / 64 < 2^32
};

template <bool kDq>
__device__ inline Fp4RowSrc fp4_row_src(const Fp4Args& a, int64_t row, int64_t chunks, int64_t kb) {
    const bool live = row < a.n;
    Fp4RowSrc r;
    r.b0 = live ? row * kb : 0;
    r.g0 = (uint32_t)r.b0;
    r.codes = buf_rsrc(a.codes + (live ? row * a.ldc : 0), live ? chunks * 16 : 0);
    if constexpr (kDq) {
        r.scales = buf_rsrc(a.c8 + r.b0, live ? kb : 0);
        r.s2 = buf_rsrc(a.s2, ((a.n * kb + kDqGroup - 1) / kDqGroup) * 4);
    } else {
        r.scales = buf_rsrc(a.absmax + r.b0, live ? kb * 4 : 0);
        r.s2 = r.scales;
    }
    return r;
}

// chunk c of a row: its codes, and its raw block scale (the absmax, or the
// code c8 and the group maximum s2)
template <bool kDq>
__device__ inline void fp4_chunk_load(const Fp4RowSrc& r, int c, uint4& cv, float& sa, uint32_t& c8) {
    // each code byte is read once: the non-temporal (nt) cache policy
    cv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.codes, c * 16, 0, 2));
    if constexpr (kDq) {
        c8 = __builtin_amdgcn_raw_buffer_load_b8(r.scales, c >> 1, 0, 0);
        sa = __builtin_bit_cast(float,
                                __builtin_amdgcn_raw_buffer_load_b32(r.s2, (int)(((r.g0 + (uint32_t)(c >> 1)) / kDqGroup) * 4), 0, 0));
    } else {
        sa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r.scales, (c >> 1) * 4, 0, 0));
        c8 = 0;
    }
}

template <int M, int CPL, bool kDq>
__global__ __launch_bounds__(64 * kFp4Waves) void fp4_rows_kernel(Fp4Args a) {
    __shared__ __attribute__((aligned(1024))) uint8_t xs[CPL * M * 4096];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t chunks = a.k / 32, kb = a.k / kBlk;
    const int64_t nw = (int64_t)gridDim.x * kFp4Waves;
    int64_t row = (int64_t)blockIdx.x * kFp4Waves + wave;

    // x -> LDS in 4 KB blocks: block (j, m) holds bytes [4096 j, 4096 j + 4096)
    // of row m (the x of chunks 64 j .. 64 j + 63, 64 bytes each), zeros past
    // the row.  1 KB per wave instruction, instruction q by wave q % 8.
    for (int q = wave; q < CPL * M * 4; q += kFp4Waves) {
        const int blk = q >> 2, part = q & 3;
        const int j = blk / M, m = blk % M;
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(a.x + m * a.ldx, a.k * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void*)(xs + q * 1024), 16, j * 4096 + part * 1024 + lane * 16, 0,
            0, 0);
    }
    uint4 cv[CPL];
    float sa[CPL];
    uint32_t c8[CPL];
    {
        const Fp4RowSrc r = fp4_row_src<kDq>(a, row, chunks, kb);
#pragma unroll
        for (int j = 0; j < CPL; ++j) fp4_chunk_load<kDq>(r, lane + 64 * j, cv[j], sa[j], c8[j]);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's copies (and its first row) landed
    __syncthreads();                      // ... and every wave's
    // one row of x: the lane's x chunks of the first kXS slots stay in
    // registers across the weight rows (16 per slot, within 128 VGPRs)
    constexpr int kXS = M != 1 ? 0 : CPL <= 3 ? CPL : CPL <= 5 ? 3 : CPL <= 7 ? 2 : 1;
    uint32_t xr[kXS > 0 ? kXS : 1][16];
    if constexpr (kXS > 0) {
#pragma unroll
        for (int j = 0; j < kXS; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4u_l xv = *reinterpret_cast<const __attribute__((address_space(3))) v4u_l*>(
                    (const __attribute__((address_space(3))) uint8_t*)xs + lane * 64 + j * 4096 + q * 16);
                xr[j][4 * q] = xv.x;
                xr[j][4 * q + 1] = xv.y;
                xr[j][4 * q + 2] = xv.z;
                xr[j][4 * q + 3] = xv.w;
            }
    }

    for (; row < a.n; row += nw) {
        const Fp4RowSrc rn = fp4_row_src<kDq>(a, row + nw, chunks, kb);   // past n: nothing is read
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            const float d = fp4_factor<kDq>(sa[j], c8[j]);
            const uint32_t cw[4] = {cv[j].x, cv[j].y, cv[j].z, cv[j].w};
            hh2 wv[4][4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wv[q][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 0);
                wv[q][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 1);
                wv[q][2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 2);
                wv[q][3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 3);
            }
            // the chunk's registers are free: request the same chunk of the next row
            fp4_chunk_load<kDq>(rn, c, cv[j], sa[j], c8[j]);
            // this chunk's x: 64 bytes per row at lane * 64 of blocks (j, m),
            // the same for every weight row (for the first kXS slots held in
            // registers above; the others read from LDS here, with more rows
            // of x through a base made opaque per chunk so that the reads stay
            // here)
            uint32_t xb = (uint32_t)lane * 64u;
            if constexpr (M > 1) asm volatile("" : "+v"(xb));
            const __attribute__((address_space(3))) uint8_t* const xl =
                (const __attribute__((address_space(3))) uint8_t*)xs + xb + j * M * 4096;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float part = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t xq[4];
                    if (j < kXS) {   // resolved at compile time: j is unrolled
#pragma unroll
                        for (int b = 0; b < 4; ++b) xq[b] = xr[j < kXS ? j : 0][4 * q + b];
                    } else {
                        const v4u_l xv =
                            *reinterpret_cast<const __attribute__((address_space(3))) v4u_l*>(xl + m * 4096 + q * 16);
                        xq[0] = xv.x;
                        xq[1] = xv.y;
                        xq[2] = xv.z;
                        xq[3] = xv.w;
                    }
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        part = __builtin_amdgcn_fdot2(wv[q][b], __builtin_bit_cast(hh2, xq[b]), part, false);
                }
                acc[m] = fmaf(part, d, acc[m]);
            }
            // (without this barrier the compiler keeps the lane's x chunks in
            // registers across the rows: 229 registers, half the waves, and 5 %
            // slower on 13B m = 1)
            __builtin_amdgcn_sched_barrier(0);
        }
        // the bias through a range that is empty without one (no branch here,
        // which would let the chunks' arithmetic sink past their barriers)
        const __amdgpu_buffer_rsrc_t rbias = buf_rsrc(a.bias, a.bias ? a.n * 2 : 0);
        const float bias =
            h2f((half_bits)__builtin_amdgcn_raw_buffer_load_b16(rbias, (int)row * 2, 0, 0));
        // lane 0 stores the M outputs; the other lanes' offsets are out of
        // range (a branch here would also let the arithmetic sink)
        const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.out, ((M - 1) * a.ldout + a.n) * 2);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float s = wave_sum_f32(acc[m]);
            const int off = lane == 0 ? (int)(m * a.ldout + row) * 2 : (int)0x80000000;
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f2h(s + bias), ro, off, 0, 0);
        }
    }
}

// Two to four rows of x: the same staging of x in LDS, but a wave takes
// groups of four weight rows (group v of the grid's nw waves: rows 4v .. 4v +
// 3, then group v + nw, ...), and a lane the same code chunk of all four, so
// each chunk of x read from LDS (64 bytes per row of x) serves four weight
// rows.  A row's chunks go in segments of 256 (S = 4 per lane); a lane keeps
// the current segment's codes of the four rows in registers and, as each
// chunk slot is used, requests that slot of the next segment (of the same
// group, or the first of its next group).
template <int M, int NSEG, bool kDq>
__global__ __launch_bounds__(64 * kFp4Waves) void fp4_rows4_kernel(Fp4Args a) {
    constexpr int R = 4, S = 4;
    __shared__ __attribute__((aligned(1024))) uint8_t xs[NSEG * S * M * 4096];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t chunks = a.k / 32, kb = a.k / kBlk;
    const int nseg = (int)((chunks + 255) / 256);
    const int64_t groups = (a.n + R - 1) / R;
    const int64_t nw = (int64_t)gridDim.x * kFp4Waves;
    int64_t g = (int64_t)blockIdx.x * kFp4Waves + wave;
    int sg = 0;

    // x -> LDS in 4 KB blocks: block (J, m) holds bytes [4096 J, 4096 J + 4096)
    // of row m (the x of chunks 64 J .. 64 J + 63), zeros past the row
    for (int q = wave; q < NSEG * S * M * 4; q += kFp4Waves) {
        const int blk = q >> 2, part = q & 3;
        const int J = blk / M, m = blk % M;
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(a.x + m * a.ldx, a.k * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void*)(xs + q * 1024), 16, J * 4096 + part * 1024 + lane * 16, 0,
            0, 0);
    }
    uint4 cv[R][S];
    float sa[R][S];
    uint32_t c8[R][S];
    {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const Fp4RowSrc src = fp4_row_src<kDq>(a, g * R + r, chunks, kb);
#pragma unroll
            for (int j = 0; j < S; ++j) fp4_chunk_load<kDq>(src, lane + 64 * j, cv[r][j], sa[r][j], c8[r][j]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's copies (and its first segment) landed
    __syncthreads();                      // ... and every wave's

    const __amdgpu_buffer_rsrc_t rbias = buf_rsrc(a.bias, a.bias ? a.n * 2 : 0);
    const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.out, ((M - 1) * a.ldout + a.n) * 2);
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
    while (g < groups) {
        int64_t gn = g;
        int sn = sg + 1;
        if (sn == nseg) {
            sn = 0;
            gn = g + nw;
        }
        Fp4RowSrc nsrc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) nsrc[r] = fp4_row_src<kDq>(a, gn * R + r, chunks, kb);   // past n: nothing
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int c = sg * 256 + lane + 64 * j;
            // this chunk's x, 64 bytes per row of x, read once for the four
            // weight rows (the base is made opaque so that the reads stay here)
            uint32_t xb = (uint32_t)lane * 64u;
            asm volatile("" : "+v"(xb));
            const __attribute__((address_space(3))) uint8_t* const xl =
                (const __attribute__((address_space(3))) uint8_t*)xs + xb + (sg * S + j) * M * 4096;
            uint32_t xq[M][16];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4u_l v = *reinterpret_cast<const __attribute__((address_space(3))) v4u_l*>(xl + m * 4096 + q * 16);
                    xq[m][4 * q] = v.x;
                    xq[m][4 * q + 1] = v.y;
                    xq[m][4 * q + 2] = v.z;
                    xq[m][4 * q + 3] = v.w;
                }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float d = fp4_factor<kDq>(sa[r][j], c8[r][j]);
                const uint32_t cw[4] = {cv[r][j].x, cv[r][j].y, cv[r][j].z, cv[r][j].w};
                hh2 wv[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    wv[4 * q] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 0);
                    wv[4 * q + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 1);
                    wv[4 * q + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 2);
                    wv[4 * q + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 3);
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float part = 0.0f;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        part = __builtin_amdgcn_fdot2(wv[e], __builtin_bit_cast(hh2, xq[m][e]), part, false);
                    acc[r][m] = fmaf(part, d, acc[r][m]);
                }
            }
            // the slot's registers are free: request it for the next segment
#pragma unroll
            for (int r = 0; r < R; ++r)
                fp4_chunk_load<kDq>(nsrc[r], sn * 256 + lane + 64 * j, cv[r][j], sa[r][j], c8[r][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (sn == 0) {
            // group g done: its 4 x M sums, lane 0 stores (other lanes' offsets
            // are out of range)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = g * R + r;
                const float bias =
                    h2f((half_bits)__builtin_amdgcn_raw_buffer_load_b16(rbias, (int)row * 2, 0, 0));
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const float sum = wave_sum_f32(acc[r][m]);
                    const int off = lane == 0 && row < a.n ? (int)(m * a.ldout + row) * 2 : (int)0x80000000;
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f2h(sum + bias), ro, off, 0, 0);
                    acc[r][m] = 0.0f;
                }
            }
        }
        g = gn;
        sg = sn;
    }
}

// Two to four rows of x on the matrix cores.  Every workgroup takes the same
// number of weight rows, R = ceil(n / grid) (held as T tiles of 16 rows, rows
// past R masked), so every CU streams the same bytes; its 8 waves split the
// chunks of 128 weights (wave w: chunks w, w + 8, ...) and meet in LDS at the
// end, summed in wave order.  x sits in LDS as for the kernels above, in 4 KB
// blocks, and so do the workgroup's block scale factors fl32(A / 6), read once.
//
// A chunk is two blocks of 64.  Lane (n, g) (n = lane % 16, g = lane / 16)
// holds 16 code bytes of weight row n of the tile: weights 128 c + 32 g .. +
// 31, so a load is 64 bytes of each of 16 rows.  Step s of
// v_mfma_f32_16x16x32_f16 takes weights 128 c + 32 g + 8 s .. + 7 of both
// operands (the same relabelling of k in x and in the weights, so the dot
// product is unchanged).  Lanes g = 0, 1 then carry block 2 c and lanes g = 2,
// 3 block 2 c + 1.  The x operand puts x row r in MFMA row r for block 2 c's
// lanes and in MFMA row 4 + r for block 2 c + 1's (zeros elsewhere), so one
// step yields both blocks' sums apart: output rows 0-3 (lanes 0-15) hold
// block 2 c's, rows 4-7 (lanes 16-31) block 2 c + 1's, and each lane scales
// its sums by its block's factor: acc += fl32(A / 6) * P.  At the end lanes
// 0-15 add lanes 16-31: the outputs of rows 0-3 of x.
typedef float v4f_16 __attribute__((ext_vector_type(4)));
constexpr int kFp4MfmaJ = 7;          // 4 KB x blocks per row of x: k <= 14336
constexpr int kFp4MfmaScales = 8192;  // block scales per workgroup: rows_per_wg * k / 64 + 2

template <int M, int T, bool kDq>
__global__ __launch_bounds__(64 * kFp4Waves) void fp4_mfma16_kernel(Fp4Args a, int64_t rows_per_wg) {
    // chunks per wave in flight: 4 KB of codes (8 KB measured 2 % slower,
    // 12 KB 9 %, 16 KB 10 %; 2 KB 2 %)
    constexpr int W = kFp4Waves, D = T <= 2 ? 2 : 1;
    __shared__ __attribute__((aligned(1024))) uint8_t xs[kFp4MfmaJ * M * 4096];
    // the workgroup's block scale factors fl32(A / 6) (read here once, with
    // whole-line loads: in the loop each load would touch 16 rows' scales)
    __shared__ float sd[kFp4MfmaScales];
    __shared__ float red[W][T][4][16];
    // zeros: the x operand of the lanes a pass leaves out
    __shared__ __attribute__((aligned(16))) uint32_t xz[16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t kb = a.k / kBlk, kc = (a.k + 127) / 128;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    int64_t valid = a.n - r0;
    if (valid > rows_per_wg) valid = rows_per_wg;

    // x -> LDS: block (J, m) at (J M + m) * 4096, only the blocks x reaches
    const int jx = (int)((a.k * 2 + 4095) / 4096);
    for (int q = wave; q < jx * M * 4; q += W) {
        const int blk = q >> 2, part = q & 3;
        const int J = blk / M, m = blk % M;
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(a.x + m * a.ldx, a.k * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void*)(xs + q * 1024), 16, J * 4096 + part * 1024 + lane * 16, 0,
            0, 0);
    }
    const int l16 = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t rc = buf_rsrc(a.codes + r0 * a.ldc, (valid - 1) * a.ldc + a.k / 2);
    uint4 cv[D][T];
    const int lane_off = (int)(l16 * a.ldc) + 16 * g;   // this lane's row and 16 bytes in a chunk
    auto load = [&](int u, int64_t c) {   // chunk c into ring slot u (past the row: zeros)
        const bool live = 2 * c + (g >> 1) < kb;
        const int base = (int)(64 * c) + lane_off;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int co = live ? base + (int)(16 * t * a.ldc) : (int)0x80000000;
            cv[u][t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 2));
        }
    };
    // the scale factors fl32(A / 6) of rows r0 .. r0 + rows_per_wg, the whole
    // area (zeros past the valid rows): every load goes out before the first
    // is used (the factor as in the kernels above).
    // The first D chunks are requested after these loads, and only the
    // copies and the scales are waited for (loads complete in order).
    constexpr int kFill = kFp4MfmaScales / (64 * W);
    {
        float v[kFill];        // absmax, or s2 when double-quantized
        uint32_t cq[kFill];    // c8 when double-quantized
        if constexpr (kDq) {
            const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.c8 + r0 * kb, valid * kb);
            const __amdgpu_buffer_rsrc_t r2 = buf_rsrc(a.s2, ((a.n * kb + kDqGroup - 1) / kDqGroup) * 4);
#pragma unroll
            for (int it = 0; it < kFill; ++it) {
                const int i = tid + 64 * W * it;
                cq[it] = __builtin_amdgcn_raw_buffer_load_b8(rs, i, 0, 0);
                v[it] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(r2, (int)((r0 * kb + i) / kDqGroup) * 4, 0, 0));
            }
        } else {
            const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.absmax + r0 * kb, valid * kb * 4);
#pragma unroll
            for (int it = 0; it < kFill; ++it) {
                v[it] = __builtin_bit_cast(float,
                                           __builtin_amdgcn_raw_buffer_load_b32(rs, (tid + 64 * W * it) * 4, 0, 0));
                cq[it] = 0;
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // the scale loads go out before the chunks'
#pragma unroll
        for (int u = 0; u < D; ++u) load(u, wave + (int64_t)W * u);
        __builtin_amdgcn_sched_barrier(0);
        static_assert(D * T <= 15, "the wait below counts the chunk loads in four bits");
        __builtin_amdgcn_s_waitcnt(0x0f70 | (D * T));   // vmcnt(D T): the copies and the scales landed
#pragma unroll
        for (int it = 0; it < kFill; ++it) sd[tid + 64 * W * it] = fp4_factor<kDq>(v[it], cq[it]);
    }
    if (tid < 16) xz[tid] = 0u;
    __syncthreads();   // every wave's copies and factors are in LDS

    // MFMA row l16 of this lane's x operand: x row l16 (block 2c's lanes, g < 2)
    // or l16 - 4 (block 2c + 1's), else zeros
    const bool x_ok = g < 2 ? l16 < M : (l16 >= 4 && l16 < 4 + M);
    const int xrow = x_ok ? (l16 & 3) : 0;
    float acc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;
    for (int64_t c0 = wave; c0 < kc; c0 += (int64_t)W * D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int64_t c = c0 + (int64_t)W * u;
            if (c < kc) {
                // x of chunk c: bytes 256 c + 64 g + 16 s of row xrow, in block J = c / 16;
                // the lanes outside the x rows read the zero area
                uint32_t xo = (uint32_t)(((c >> 4) * M + xrow) * 4096 + 256 * (c & 15) + 64 * g);
                asm volatile("" : "+v"(xo));
                typedef const __attribute__((address_space(3))) uint8_t lu8;
                typedef const __attribute__((address_space(3))) v4u_l lv4u;
                lu8* const px = x_ok ? (lu8*)xs + xo : (lu8*)xz;
                v8h ax[4];
#pragma unroll
                for (int st = 0; st < 4; ++st) ax[st] = __builtin_bit_cast(v8h, *reinterpret_cast<lv4u*>(px + 16 * st));
                // the factor of the block whose sums this lane holds (2c + g for
                // g < 2; lanes g >= 2 hold zeros) for its weight row (a row past
                // the share reads row 0's: its codes are zero), read before the MFMAs
                float d[T];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int rr = 16 * t + l16;
                    d[t] = sd[(rr < valid ? rr : 0) * kb + 2 * c + (g & 1)];
                }
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const uint32_t cw[4] = {cv[u][t].x, cv[u][t].y, cv[u][t].z, cv[u][t].w};
                    v4f_16 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const hh2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[st], 1.0f, 0);
                        const hh2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[st], 1.0f, 1);
                        const hh2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[st], 1.0f, 2);
                        const hh2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[st], 1.0f, 3);
                        const v8h wb = {w0.x, w0.y, w1.x, w1.y, w2.x, w2.y, w3.x, w3.y};
                        p = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax[st], wb, p, 0, 0, 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(p[r], d[t], acc[t][r]);
                }
            }
            load(u, c + (int64_t)W * D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
    // lanes 0-15: block 2c's sums plus block 2c + 1's from lanes 16-31
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] += __shfl_down(acc[t][r], 16, 64);
    if (lane < 16) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][t][r][l16] = acc[t][r];
    }
    __syncthreads();
    if (wave == 0 && lane < 16) {
        const __amdgpu_buffer_rsrc_t rbias = buf_rsrc(a.bias, a.bias ? a.n * 2 : 0);
        const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.out, ((M - 1) * a.ldout + a.n) * 2);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int rr = 16 * t + l16;
            const int64_t row = r0 + rr;
            const float bias = h2f((half_bits)__builtin_amdgcn_raw_buffer_load_b16(rbias, (int)row * 2, 0, 0));
#pragma unroll
            for (int r = 0; r < M; ++r) {
                float sum = 0.0f;
#pragma unroll
                for (int w = 0; w < W; ++w) sum += red[w][t][r][l16];
                const int off = rr < valid ? (int)(r * a.ldout + row) * 2 : (int)0x80000000;
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f2h(sum + bias), ro, off, 0, 0);
            }
        }
    }
}

template <int M, int T>
hipError_t launch_mfma16_t(const Fp4Args& a, int64_t grid, int64_t rows, hipStream_t stream) {
    if (a.absmax)
        hipLaunchKernelGGL((fp4_mfma16_kernel<M, T, false>), dim3((unsigned)grid), dim3(64 * kFp4Waves), 0, stream,
                           a, rows);
    else
        hipLaunchKernelGGL((fp4_mfma16_kernel<M, T, true>), dim3((unsigned)grid), dim3(64 * kFp4Waves), 0, stream,
                           a, rows);
    return hipGetLastError();
}

// two to four rows of x, k <= 14336, n <= 256 * 64: the MFMA kernel (false:
// not taken)
template <int M>
bool launch_mfma_m(const Fp4Args& a, hipStream_t stream, hipError_t* err) {
    if (a.k > kFp4MfmaJ * 2048 || a.n > 256 * 64) return false;
    const int64_t rows = (a.n + 255) / 256;          // weight rows per workgroup
    if (rows * (a.k / kBlk) + 2 > kFp4MfmaScales) return false;
    const int64_t grid = (a.n + rows - 1) / rows;    // every workgroup has at least one row
    *err = rows <= 32 ? launch_mfma16_t<M, 2>(a, grid, rows, stream) : launch_mfma16_t<M, 4>(a, grid, rows, stream);
    return true;
}

template <int M, int NSEG>
hipError_t launch_rows4_seg(const Fp4Args& a, hipStream_t stream) {
    const int64_t groups = (a.n + 3) / 4;
    int64_t grid = 256;
    const int64_t need = (groups + kFp4Waves - 1) / kFp4Waves;
    if (need < grid) grid = need;
    if (a.absmax)
        hipLaunchKernelGGL((fp4_rows4_kernel<M, NSEG, false>), dim3((unsigned)grid), dim3(64 * kFp4Waves), 0, stream, a);
    else
        hipLaunchKernelGGL((fp4_rows4_kernel<M, NSEG, true>), dim3((unsigned)grid), dim3(64 * kFp4Waves), 0, stream, a);
    return hipGetLastError();
}

// two to four rows of x, k <= 16384
template <int M>
hipError_t launch_rows4_m(const Fp4Args& a, hipStream_t stream) {
    return a.k / 32 <= 256 ? launch_rows4_seg<M, 1>(a, stream) : launch_rows4_seg<M, 2>(a, stream);
}

template <int M, int CPL>
hipError_t launch_rows_cpl(const Fp4Args& a, hipStream_t stream) {
    constexpr int kLds = CPL * M * 4096;
    const int64_t per_cu = kLds <= 64 * 1024 ? 2 : 1;   // one per CU measured 7 % slower (13B m = 1)
    int64_t grid = 256 * per_cu;
    const int64_t need = (a.n + kFp4Waves - 1) / kFp4Waves;
    if (need < grid) grid = need;
    if (a.absmax)
        hipLaunchKernelGGL((fp4_rows_kernel<M, CPL, false>), dim3((unsigned)grid), dim3(64 * kFp4Waves), 0, stream, a);
    else
        hipLaunchKernelGGL((fp4_rows_kernel<M, CPL, true>), dim3((unsigned)grid), dim3(64 * kFp4Waves), 0, stream, a);
    return hipGetLastError();
}

// k <= 16384 (at most 8 chunks per lane): the LDS-x kernel with the fewest
// chunk slots per lane that cover a row (at least 2): a slot past the row
// reads nothing but still costs its conversions and dot products
template <int M>
hipError_t launch_rows_m(const Fp4Args& a, hipStream_t stream) {
    switch ((a.k / 32 + 63) / 64) {
        case 0:
        case 1:
        case 2: return launch_rows_cpl<M, 2>(a, stream);
        case 3: return launch_rows_cpl<M, 3>(a, stream);
        case 4: return launch_rows_cpl<M, 4>(a, stream);
        case 5: return launch_rows_cpl<M, 5>(a, stream);
        case 6: return launch_rows_cpl<M, 6>(a, stream);
        case 7: return launch_rows_cpl<M, 7>(a, stream);
        default: return launch_rows_cpl<M, 8>(a, stream);
    }
}
constexpr int64_t kFp4LdsMaxK = 16384;

template <int M>
hipError_t launch_gemv_m(const Fp4Args& a, hipStream_t stream) {
    hipLaunchKernelGGL((fp4_gemv_kernel<M>), dim3((unsigned)ceil_div(a.n, fp4_rows<M>())), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp4_quantize(const Fp4Args& a, hipStream_t stream) {
    const int64_t lanes = a.n * (a.k / kBlk) * 8;
    if (lanes == 0) return hipSuccess;
    const bool vec = a.ldw % 8 == 0 && (reinterpret_cast<uintptr_t>(a.w) & 15) == 0 && a.ldc % 4 == 0 &&
                     (reinterpret_cast<uintptr_t>(a.codes_out) & 3) == 0;
    const dim3 grid((unsigned)ceil_div(lanes, 256));
    if (vec)
        hipLaunchKernelGGL(fp4_quant_kernel<true>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(fp4_quant_kernel<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fp4_double_quant(const float* absmax, int64_t nb, uint8_t* c8, float* s2, hipStream_t stream) {
    if (nb <= 0) return hipSuccess;
    hipLaunchKernelGGL(fp4_dq_kernel, dim3((unsigned)ceil_div(nb, kDqGroup)), dim3(256), 0, stream, absmax, nb, c8,
                       s2);
    return hipGetLastError();
}

hipError_t launch_fp4_dequantize(const Fp4Args& a, hipStream_t stream) {
    const int64_t lanes = a.n * (a.k / kBlk) * 8;
    if (lanes == 0) return hipSuccess;
    hipLaunchKernelGGL(fp4_dequant_kernel, dim3((unsigned)ceil_div(lanes, 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fp4_linear(const Fp4Args& in, hipStream_t stream) {
    // groups of at most four rows of x, each a launch over all the weights
    for (int64_t i0 = 0; i0 < in.m; i0 += 4) {
        Fp4Args a = in;
        a.x = in.x + i0 * in.ldx;
        a.out = static_cast<half_bits*>(in.out) + i0 * in.ldout;
        const int64_t mm = in.m - i0 < 4 ? in.m - i0 : 4;
        // one row of x with k <= 16384: the LDS-x kernel (13B m = 1: 2657 ->
        // 2986 GB/s); two to four rows: the MFMA kernel where it applies
        // (13B m = 4: 1604 -> 1752 GB/s against the four-row LDS-x kernel,
        // 1491 with the x-from-L2 kernel), else the four-row LDS-x kernel
        // (and only while the block count n k / 64 fits the 32-bit group index
        // of their double-quantized scales; past it the L2-x kernel)
        const bool lds = a.k <= kFp4LdsMaxK && a.n * (a.k / kBlk) < ((int64_t)1 << 32);
        if (mm >= 2) {
            hipError_t em = hipSuccess;
            const bool took = mm == 2 ? launch_mfma_m<2>(a, stream, &em)
                            : mm == 3 ? launch_mfma_m<3>(a, stream, &em)
                                      : launch_mfma_m<4>(a, stream, &em);
            if (took) {
                if (em != hipSuccess) return em;
                continue;
            }
        }
        const hipError_t e = mm == 1 ? (lds ? launch_rows_m<1>(a, stream) : launch_gemv_m<1>(a, stream))
                           : mm == 2 ? (lds ? launch_rows4_m<2>(a, stream) : launch_gemv_m<2>(a, stream))
                           : mm == 3 ? (lds ? launch_rows4_m<3>(a, stream) : launch_gemv_m<3>(a, stream))
                                     : (lds ? launch_rows4_m<4>(a, stream) : launch_gemv_m<4>(a, stream));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace i8mp

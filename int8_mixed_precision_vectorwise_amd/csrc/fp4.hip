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
// M rows of x.  A workgroup takes kRows weight rows; its 256 lanes split each
// row into 16-byte code chunks (32 weights, half a block), lane t taking chunks
// t, t + 256, ..., the same chunks of all kRows rows, so the lane's x chunk is
// read once for them.  The next chunk's codes are requested before the current
// one is used.  The hardware conversion turns a code byte into two exact fp16
// E2M1 values (scale 1); v_dot2_f32_f16 adds their products with x into an
// fp32 sum per half block, which is then scaled by fl32(A / 6).  Lane sums are
// reduced in the wave (DPP), then over the 4 waves in LDS.
// weight rows per workgroup: 4 for three or more rows of x (fewer registers,
// two waves per SIMD at four rows of x), 8 otherwise
template <int M, bool kOne>
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
        // block scale A (the absmax, or fl32(c8 * fl32(s2 / 255))), then A / 6 as
        // A * fl32(1 / 6): within one ulp of the IEEE quotient the dequantize op
        // uses, far inside the fp32 sums' rounding, and one multiply instead of a
        // division sequence per row and chunk
        const float A = a.absmax ? t.sa[r] : (float)t.c8[r] * (t.sa[r] / 255.0f);
        const float d = A * (1.0f / 6.0f);
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

// kOne: every lane has at most one chunk (k <= 8192): no next-chunk buffer,
// fewer registers, more workgroups resident.  Taken for two or more rows of x
// (13B up layer, m = 4: 40.7 -> 30.6 us); for one row the pipelined form
// measured faster (14.0 against 16.6 us).
template <int M, bool kOne>
__global__ __launch_bounds__(256) void fp4_gemv_kernel(Fp4Args a) {
    constexpr int kRows = fp4_rows<M, kOne>();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t chunks = a.k / 32, kb = a.k / kBlk;
    const int64_t n0 = (int64_t)blockIdx.x * kRows;
    float acc[kRows][M];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
    int64_t c = tid;
    if (kOne) {
        if (c < chunks) {
            Fp4Chunk<M, kRows> cur;
            fp4_load(a, n0, c, kb, cur);
            fp4_compute(a, cur, n0, acc);
        }
    } else if (c < chunks) {
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

template <int M>
hipError_t launch_gemv_m(const Fp4Args& a, hipStream_t stream) {
    if (M > 1 && a.k / 32 <= 256)
        hipLaunchKernelGGL((fp4_gemv_kernel<M, true>), dim3((unsigned)ceil_div(a.n, fp4_rows<M, true>())),
                           dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((fp4_gemv_kernel<M, false>), dim3((unsigned)ceil_div(a.n, fp4_rows<M, false>())),
                           dim3(256), 0, stream, a);
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
        hipError_t e = mm == 1 ? launch_gemv_m<1>(a, stream)
                     : mm == 2 ? launch_gemv_m<2>(a, stream)
                     : mm == 3 ? launch_gemv_m<3>(a, stream)
                               : launch_gemv_m<4>(a, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace i8mp

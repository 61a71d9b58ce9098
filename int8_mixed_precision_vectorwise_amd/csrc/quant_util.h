// Device helpers of the activation quantizer (outlier bits, masked chunk
// maximum, the IEEE code rounding, bitmap prefix), shared by the quantization
// kernels and the fused decode forward so that both compute the same codes.
#pragma once

#include "common.h"

namespace i8mp {

// bit e of the result: |x_e| >= tau for the 8 fp16 values of v
__device__ inline uint32_t outlier_bits8(const uint4& v, float tau) {
    uint32_t m = 0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = h2f((half_bits)(w[i] & 0x7fffu));
        const float hi = h2f((half_bits)((w[i] >> 16) & 0x7fffu));
        m |= (lo >= tau ? 1u : 0u) << (2 * i);
        m |= (hi >= tau ? 1u : 0u) << (2 * i + 1);
    }
    return m;
}

// 8 fp16 values starting at column col of a row.  kVec: one 16-byte load
// (the caller guarantees col + 8 <= k and 16-byte aligned rows: k and ldx
// multiples of 8; no per-element path, so the compiler keeps several such
// loads in flight).  Otherwise element by element, columns >= k as 0.
template <bool kVec>
__device__ inline uint4 load8(const half_bits* __restrict__ row, int64_t col, int64_t k) {
    if (kVec) return *reinterpret_cast<const uint4*>(row + col);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (col + e < k) w[e >> 1] |= (uint32_t)row[col + e] << (16 * (e & 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Buffer resource over bytes [base, base + bytes): loads past the end return
// 0 and stores past it are dropped, so loops over chunks need no branch per
// access (which would make the compiler's vmcnt waits conservative; on gfx9
// vmcnt also counts stores).
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    if (bytes < 0) bytes = 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline half_bits half_at(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (half_bits)((w >> (16 * (e & 1))) & 0xffffu);
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ inline uint32_t code_byte(float x, float inv, bool zero) {
    float q = __builtin_rintf(x * inv);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    const int iq = zero ? 0 : (int)q;
    return (uint32_t)iq & 0xffu;
}

// largest |x| of the chunk over the columns whose outlier bit is clear
__device__ inline float chunk_max(const uint4& v, uint32_t obits) {
    float t = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float f = fabsf(h2f(half_at(v, e)));
        t = ((obits >> e) & 1u) ? t : fmaxf(t, f);
    }
    return t;
}

// Exclusive prefix of the per-word popcounts of bm into pre (slot of each
// outlier column in the index list); returns the total (all threads call).
__device__ inline int32_t bitmap_prefix(const uint32_t* bm, int32_t* pre, int64_t words, int32_t* wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int64_t per = (words + blockDim.x - 1) / blockDim.x;
    const int64_t w0 = (int64_t)tid * per;
    int64_t w1 = w0 + per;
    if (w1 > words) w1 = words;
    int32_t s = 0;
    for (int64_t w = w0; w < w1; ++w) s += __popc(bm[w]);
    int32_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t off = 0, total = 0;
    for (int i = 0; i < nwaves; ++i) {
        if (i < wave) off += wave_tot[i];
        total += wave_tot[i];
    }
    int32_t run = off + incl - s;
    for (int64_t w = w0; w < w1; ++w) {
        pre[w] = run;
        run += __popc(bm[w]);
    }
    __syncthreads();
    return total;
}


// Workgroup 0 publishes the bitmap, the count and the ascending index list
// (its first idx_len entries, -1 past the count).
__device__ inline void publish(const QuantArgs& a, const uint32_t* bm, const int32_t* pre, int32_t total,
                               bool outl) {
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    if (a.bitmap_out)
        for (int64_t w = tid; w < a.words; w += nt) a.bitmap_out[w] = outl ? bm[w] : 0u;
    if (a.count_out && tid == 0) *a.count_out = total;
    if (a.idx_out) {
        for (int32_t s = tid; s < a.idx_len; s += nt)
            if (s >= total) a.idx_out[s] = -1;
        if (outl) {
            for (int64_t w = tid; w < a.words; w += nt) {
                uint32_t v = bm[w];
                int32_t slot = pre[w];
                while (v) {
                    const int b = __ffs(v) - 1;
                    if (slot < a.idx_len) a.idx_out[slot] = (int32_t)(w * 32 + b);
                    ++slot;
                    v &= v - 1u;
                }
            }
        }
    }
}

// Codes of the 8 columns starting at col of row r, and the row's outlier
// values among them gathered into x_out at their slots.
__device__ inline void emit8(const QuantArgs& a, const uint4& v, uint32_t obits, int64_t r, int64_t col,
                             float inv, bool zero_row, bool vec_q, const uint32_t* bm, const int32_t* pre) {
    if (a.q) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b = code_byte(h2f(half_at(v, e)), inv, zero_row || ((obits >> e) & 1u));
            if (e < 4) lo |= b << (8 * e);
            else hi |= b << (8 * (e - 4));
        }
        int8_t* qr = a.q + r * a.ldq + col;
        if (vec_q && col + 8 <= a.k) {
            *reinterpret_cast<uint2*>(qr) = make_uint2(lo, hi);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (col + e < a.k) qr[e] = (int8_t)(((e < 4 ? lo : hi) >> (8 * (e & 3))) & 0xffu);
        }
    }
    if (a.x_out && obits) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((obits >> e) & 1u) {
                const int64_t j = col + e;
                const int64_t w = j >> 5;
                const uint32_t below = bm[w] & ((1u << (j & 31)) - 1u);
                const int32_t slot = pre[w] + __popc(below);
                if (slot < a.cap) a.x_out[r * a.ldo + slot] = half_at(v, e);
            }
        }
    }
}

// Sums over the 64 lanes, returned wave-uniform: DPP adds within each row of
// 16 lanes (quad swaps, half-row and row mirrors), then the four row totals
// read out with v_readlane.  No LDS traffic, unlike a shuffle ladder.
template <int kCtrl>
__device__ inline int32_t dpp_i32(int32_t v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false);
}
constexpr int kDppQuadSwap1 = 0xb1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4e;  // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ inline int32_t wave_sum_i32(int32_t v) {
    v += dpp_i32<kDppQuadSwap1>(v);
    v += dpp_i32<kDppQuadSwap2>(v);
    v += dpp_i32<kDppHalfMirror>(v);
    v += dpp_i32<kDppRowMirror>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
           __builtin_amdgcn_readlane(v, 48);
}

__device__ inline float wave_sum_f32(float v) {
    v += __int_as_float(dpp_i32<kDppQuadSwap1>(__float_as_int(v)));
    v += __int_as_float(dpp_i32<kDppQuadSwap2>(__float_as_int(v)));
    v += __int_as_float(dpp_i32<kDppHalfMirror>(__float_as_int(v)));
    v += __int_as_float(dpp_i32<kDppRowMirror>(__float_as_int(v)));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Largest value over the 64 lanes (values >= 0), wave-uniform, as wave_sum_f32.
__device__ inline float wave_max_uniform(float v) {
    v = fmaxf(v, __int_as_float(dpp_i32<kDppQuadSwap1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppQuadSwap2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppHalfMirror>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<kDppRowMirror>(__float_as_int(v))));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// largest |x| of the 8 fp16 values (packed fp16 maxima of the magnitudes: exact)
__device__ inline float chunk_absmax(const uint4& v) {
    const uint32_t mag = 0x7fff7fffu;
    const h2_t a = __builtin_bit_cast(h2_t, v.x & mag), b = __builtin_bit_cast(h2_t, v.y & mag);
    const h2_t c = __builtin_bit_cast(h2_t, v.z & mag), d = __builtin_bit_cast(h2_t, v.w & mag);
    const h2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return fmaxf((float)m.x, (float)m.y);
}

// The 8 fp16 values with those whose bit is set in ob replaced by +0.
__device__ inline uint4 mask_outliers(const uint4& v, uint32_t ob) {
    auto keep = [&](uint32_t w, int d) {
        const uint32_t lo = (uint32_t)((int32_t)(ob << (31 - 2 * d)) >> 31);      // all ones if bit 2d
        const uint32_t hi = (uint32_t)((int32_t)(ob << (30 - 2 * d)) >> 31);      // all ones if bit 2d + 1
        return w & ~((lo & 0x0000ffffu) | (hi & 0xffff0000u));
    };
    return make_uint4(keep(v.x, 0), keep(v.y, 1), keep(v.z, 2), keep(v.w, 3));
}

// Codes of a chunk with no outlier column: rne(x * inv) in fp32.  Every |x|
// of the chunk is at most the row absmax s and inv = fl32(127 / s), so the
// product rounds into [-127, 127] and the clamp of the code definition never
// acts; inv = 0 (a zero row) gives 0.
__device__ inline uint2 codes8_plain(const uint4& v, float inv) {
    // p = fl32(x * inv) has |p| <= 127, so fl32(p + 1.5 * 2^23) is p rounded
    // to the nearest integer, ties to even (the ulp there is 1), held in the
    // low mantissa bits: the low byte is the code.  The multiply and the add
    // must stay two roundings (no fused multiply-add).
#pragma clang fp contract(off)
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = h2f(half_at(v, e)) * inv;
        b[e] = __builtin_bit_cast(uint32_t, p + 12582912.0f);
    }
    // byte selects: low bytes of (b1, b0) to bytes 1, 0; then two such halves
    const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
    const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u), 0x05040100u);
    return make_uint2(lo, hi);
}

}  // namespace i8mp

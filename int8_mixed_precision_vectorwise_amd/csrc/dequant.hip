// Standalone int8_mm_dequant with the sparse-decomposition term, and the
// int8 vectorwise dequantize op (gfx950).
//
// out[i,n] = fp16( (col_absmax[n]/127) * (C[i,n]*row_absmax[i]/127 + P[i,n]) + bias[n] )
// P[i,n]   = sum over the kept outlier slots s of x_out[i,s] * b[n, idx[s]]
// (bitsandbytes PR "LLM.int8() Refactoring: Part 1": int8_mm_dequant replacing
// mm_dequant / vectorwise_mm_dequant; sparse decomposition under "Next steps").
//
// The unfused path: it reads the int32 C back from HBM, so it is bound by
// 4 bytes in + 2 bytes out per element.  One thread per output column, a
// workgroup walks rows_per_block rows so that the column's outlier weights
// (a strided gather) are fetched once into registers and reused.
#include "common.h"

namespace i8mp {

namespace {
constexpr int kRegSlots = 32;
}  // namespace

__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs d, int64_t rows_per_block) {
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    int64_t r1 = r0 + rows_per_block;
    if (r1 > d.m) r1 = d.m;
    if (col >= d.n) return;  // no barriers below
    const float r127 = 1.0f / 127.0f;
    int cnt = 0;
    if (d.x_out) {
        cnt = *d.count;
        if (cnt > d.cap) cnt = d.cap;
    }
    const float sw = d.col_absmax[col] * r127;
    const float bj = d.bias ? h2f(d.bias[col]) : 0.0f;
    float wo[kRegSlots];
#pragma unroll
    for (int s = 0; s < kRegSlots; ++s)
        wo[s] = s < cnt ? (float)d.b[col * d.ldb + d.idx[s]] : 0.0f;
    for (int64_t r = r0; r < r1; ++r) {
        float p = 0.0f;
        if (cnt) {
            const half_bits* xo = d.x_out + r * d.ldo;
#pragma unroll
            for (int s = 0; s < kRegSlots; ++s)
                if (s < cnt) p = fmaf(h2f(xo[s]), wo[s], p);
            for (int s = kRegSlots; s < cnt; ++s)
                p = fmaf(h2f(xo[s]), (float)d.b[col * d.ldb + d.idx[s]], p);
        }
        const float y = sw * ((float)d.c[r * d.ldc + col] * (d.row_absmax[r] * r127) + p) + bj;
        d.out[r * d.ldout + col] = f2h(y);
    }
}

hipError_t launch_dequant(const DequantArgs& d, hipStream_t stream) {
    const int64_t rpb = 16;
    dim3 grid((unsigned)ceil_div(d.n, 256), (unsigned)ceil_div(d.m, rpb));
    hipLaunchKernelGGL(dequant_kernel, grid, dim3(256), 0, stream, d, rpb);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// int8 vectorwise dequantize (bitsandbytes PR "LLM.int8() Refactoring: Part
// 1", "Next steps": add an int8 dequantize op):
//   out[i, j] = q[i, j] * fl32(absmax[i] / 127)   in fp32 (IEEE quotient and
//   product), stored as fp16 (round to nearest even) or fp32.
// The inverse of the row-wise quantization up to the code's rounding.  A
// stream of 16-code chunks: one thread per chunk, a row per grid row (rows
// past gridDim.y loop), 16-byte loads and stores where the rows allow them.
template <bool kHalf, bool kVec>
__global__ __launch_bounds__(256) void vectorwise_dequant_kernel(VecDequantArgs d) {
    const int64_t col = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
    if (col >= d.k) return;  // no barriers here
    for (int64_t r = blockIdx.y; r < d.m; r += gridDim.y) {
        const float sc = d.absmax[r] / 127.0f;  // IEEE division
        const int8_t* qr = d.q + r * d.ldq + col;
        float v[16];
        if (kVec && col + 16 <= d.k) {
            const v4i w = *reinterpret_cast<const v4i*>(qr);
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = (float)(int8_t)(((uint32_t)w[e >> 2] >> (8 * (e & 3))) & 0xffu) * sc;
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = col + e < d.k ? (float)qr[e] * sc : 0.0f;
        }
        if constexpr (kHalf) {
            half_bits* o = static_cast<half_bits*>(d.out) + r * d.ldout + col;
            if (kVec && col + 16 <= d.k) {
                v8h h0, h1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    h0[e] = (_Float16)v[e];
                    h1[e] = (_Float16)v[8 + e];
                }
                *reinterpret_cast<v8h*>(o) = h0;
                *reinterpret_cast<v8h*>(o + 8) = h1;
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (col + e < d.k) o[e] = f2h(v[e]);
            }
        } else {
            float* o = static_cast<float*>(d.out) + r * d.ldout + col;
            if (kVec && col + 16 <= d.k) {
#pragma unroll
                for (int t = 0; t < 4; ++t) *reinterpret_cast<v4f*>(o + 4 * t) = v4f{v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]};
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (col + e < d.k) o[e] = v[e];
            }
        }
    }
}

hipError_t launch_vectorwise_dequant(const VecDequantArgs& d, hipStream_t stream) {
    const int64_t esz = d.half_out ? 2 : 4;
    // 16-byte codes and 16-byte output pieces at every full chunk
    const bool vec = (d.ldq & 15) == 0 && (reinterpret_cast<uintptr_t>(d.q) & 15) == 0 &&
                     ((d.ldout * esz) & 15) == 0 && (reinterpret_cast<uintptr_t>(d.out) & 15) == 0;
    const dim3 grid((unsigned)ceil_div(ceil_div(d.k, 16), 256), (unsigned)(d.m < 65535 ? d.m : 65535));
    if (d.half_out) {
        if (vec) hipLaunchKernelGGL((vectorwise_dequant_kernel<true, true>), grid, dim3(256), 0, stream, d);
        else hipLaunchKernelGGL((vectorwise_dequant_kernel<true, false>), grid, dim3(256), 0, stream, d);
    } else {
        if (vec) hipLaunchKernelGGL((vectorwise_dequant_kernel<false, true>), grid, dim3(256), 0, stream, d);
        else hipLaunchKernelGGL((vectorwise_dequant_kernel<false, false>), grid, dim3(256), 0, stream, d);
    }
    return hipGetLastError();
}

}  // namespace i8mp

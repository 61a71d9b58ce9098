// Standalone int8_mm_dequant with the sparse-decomposition term (gfx950).
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

}  // namespace i8mp

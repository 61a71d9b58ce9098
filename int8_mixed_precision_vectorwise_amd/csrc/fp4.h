// Internal declarations of the blockwise 4-bit weight kernels (gfx950 only).
#pragma once

#include "common.h"

namespace i8mp {

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

}  // namespace i8mp

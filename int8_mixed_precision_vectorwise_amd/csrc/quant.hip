// Outlier-column detection and fused row calibration + int8 quantization +
// outlier extraction for gfx950.
//
// The method keeps outlier feature columns in fp16 and quantizes the rest of
// each row to int8 with its own absmax (transformers PR "`bitsandbytes` -
// `Linear8bitLt` integration into `transformers` models", "About the mixed
// quantization method in few words"; bitsandbytes PR "LLM.int8() Refactoring:
// Part 1", "Enhancements": calibration and quantization fused in one op).
//
// Because a row's scale excludes every outlier column, and the outlier set is
// a property of all rows, the work is split at the one point that needs a
// global view:
//   detect_kernel  one pass over X: per (row block, 256-column block) a word
//                  of the partial outlier bitmap (no atomics, no zeroing: every
//                  word of every partial is written);
//   quant_kernel   ORs the partial bitmaps into LDS, then one row per
//                  wavefront: coalesced 16-byte loads, wavefront-shuffle absmax
//                  over the non-outlier columns, IEEE fp32 quantization, 8-byte
//                  code stores, gather of the outlier values into the compact
//                  fp16 matrix.  Workgroup 0 also writes the bitmap, the ascending
//                  index list and the count.
#include "common.h"

namespace i8mp {

namespace {

__device__ inline float h2f(half_bits h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ inline uint32_t outlier_bits8(const uint4& v, float tau) {
    uint32_t m = 0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float lo = h2f((half_bits)(w[i] & 0x7fffu));
        float hi = h2f((half_bits)((w[i] >> 16) & 0x7fffu));
        m |= (lo >= tau ? 1u : 0u) << (2 * i);
        m |= (hi >= tau ? 1u : 0u) << (2 * i + 1);
    }
    return m;
}

// 8 fp16 values starting at column col of a row; columns >= k read as 0.
template <bool kVec>
__device__ inline uint4 load8(const half_bits* __restrict__ row, int64_t col, int64_t k) {
    if (kVec && col + 8 <= k) return *reinterpret_cast<const uint4*>(row + col);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (col + e < k) w[e >> 1] |= (uint32_t)row[col + e] << (16 * (e & 1));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
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

// One int8 code per the method's reading: 0 for outlier columns and for rows
// without a non-outlier magnitude, else clamp(rne(fl32(x * inv)), -127, 127).
__device__ inline uint32_t code_byte(float x, float inv, bool zero) {
    float q = __builtin_rintf(x * inv);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    int iq = zero ? 0 : (int)q;
    return (uint32_t)iq & 0xffu;
}

}  // namespace

template <bool kVec>
__global__ __launch_bounds__(256) void detect_kernel(const half_bits* __restrict__ x, int64_t m,
                                                     int64_t k, int64_t ldx, float tau,
                                                     int64_t rows_per_block, int64_t words,
                                                     uint32_t* __restrict__ partial) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cg = tid & 31;  // group of 8 columns
    const int rsub = tid >> 5;
    const int64_t col0 = (int64_t)blockIdx.x * kDetectCols + cg * 8;
    const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
    int64_t r_end = r_begin + rows_per_block;
    if (r_end > m) r_end = m;

    uint32_t mask = 0;
    if (col0 < k) {
        if (kVec && col0 + 8 <= k) {
#pragma unroll 8
            for (int64_t r = r_begin + rsub; r < r_end; r += 8) {
                uint4 v = *reinterpret_cast<const uint4*>(x + r * ldx + col0);
                mask |= outlier_bits8(v, tau);
            }
        } else {
            for (int64_t r = r_begin + rsub; r < r_end; r += 8) {
                uint4 v = load8<false>(x + r * ldx, col0, k);
                mask |= outlier_bits8(v, tau);
            }
        }
    }
    mask |= __shfl_xor(mask, 32, 64);  // lanes l and l^32 hold the same columns
    __shared__ uint32_t red[4][32];
    if (lane < 32) red[wave][lane] = mask;
    __syncthreads();
    if (tid < 8) {
        uint32_t word = 0;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int g = tid * 4 + q4;
            const uint32_t mm = red[0][g] | red[1][g] | red[2][g] | red[3][g];
            word |= (mm & 0xffu) << (8 * q4);
        }
        const int64_t w = (int64_t)blockIdx.x * 8 + tid;
        if (w < words) partial[(int64_t)blockIdx.y * words + w] = word;
    }
}

// Rows are processed one per wavefront (no workgroup barrier inside the row
// loop), in batches of kBatch 16-byte loads per lane that are all in flight
// together.  A row of at most one batch (k <= 4096) stays in registers; a
// longer row is read twice, the second time from L2 / the infinity cache.
constexpr int kBatch = 8;

// kBlockRow: the whole workgroup quantizes one row at a time (few rows: every
// row's loads go out in one batch across 256 threads); otherwise one row per
// wavefront.
template <bool kVec, bool kBlockRow>
__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a) {
    extern __shared__ uint32_t smem[];
    uint32_t* bm = smem;                                       // [words]
    int32_t* pre = reinterpret_cast<int32_t*>(smem + a.words);  // [words]
    __shared__ int32_t wave_tot[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool outl = a.partial != nullptr;
    const bool need_prefix = outl && (a.x_out || a.idx_out || a.count_out);

    // The first row's first batch of loads goes out now, so that its latency
    // overlaps the bitmap and prefix work below.
    constexpr int P = kBlockRow ? 256 : 64;  // threads sharing a row
    const int pid = kBlockRow ? tid : lane;
    const int64_t rr0 = kBlockRow ? 0 : wave;
    const int64_t r_first = (int64_t)blockIdx.x * a.rows_per_block + rr0;
    const bool preload = rr0 < a.rows_per_block && r_first < a.m;
    uint4 v[kBatch];
    auto load_batch = [&](const half_bits* __restrict__ xr, int64_t b) {
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int64_t col = (b * P * kBatch + (int64_t)pid + P * c) * 8;
            v[c] = col < a.k ? load8<kVec>(xr, col, a.k) : make_uint4(0, 0, 0, 0);
        }
    };
    if (preload) load_batch(a.x + r_first * a.ldx, 0);

    // 1. the final outlier bitmap: OR of the per-row-block partials.  The
    // partial words are independent loads; 8 are kept in flight per thread and
    // folded into LDS with ds_or.
    if (outl) {
        for (int64_t w = tid; w < a.words; w += 256) bm[w] = 0u;
        __syncthreads();
        const int64_t total_words = a.row_blocks * a.words;
        for (int64_t f0 = tid; f0 < total_words; f0 += 256 * 8) {
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t f = f0 + 256 * u;
                v[u] = f < total_words ? a.partial[f] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t f = f0 + 256 * u;
                if (v[u]) atomicOr(&bm[f % a.words], v[u]);
            }
        }
        __syncthreads();
        if (tid == 0 && (a.k & 31)) bm[a.words - 1] &= (1u << (a.k & 31)) - 1u;
    }
    __syncthreads();

    // 2. exclusive prefix of the per-word popcounts (slot of each outlier column)
    int32_t total = 0;
    if (need_prefix) {
        const int64_t per = (a.words + 255) / 256;
        const int64_t w0 = (int64_t)tid * per;
        int64_t w1 = w0 + per;
        if (w1 > a.words) w1 = a.words;
        int32_t s = 0;
        for (int64_t w = w0; w < w1; ++w) s += __popc(bm[w]);
        int32_t incl = s;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int32_t t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        int32_t off = 0;
        for (int i = 0; i < 4; ++i) {
            if (i < wave) off += wave_tot[i];
            total += wave_tot[i];
        }
        int32_t run = off + incl - s;
        for (int64_t w = w0; w < w1; ++w) {
            pre[w] = run;
            run += __popc(bm[w]);
        }
        __syncthreads();
    }
    const int32_t kept = total < a.cap ? total : a.cap;

    // 3. workgroup 0 publishes the bitmap, the index list and the count
    if (blockIdx.x == 0) {
        if (a.bitmap_out)
            for (int64_t w = tid; w < a.words; w += 256) a.bitmap_out[w] = outl ? bm[w] : 0u;
        if (a.count_out && tid == 0) *a.count_out = total;
        if (a.idx_out) {
            for (int32_t s = tid; s < a.idx_len; s += 256)
                if (s >= kept) a.idx_out[s] = -1;
            if (outl) {
                for (int64_t w = tid; w < a.words; w += 256) {
                    uint32_t v = bm[w];
                    int32_t slot = pre[w];
                    while (v) {
                        const int b = __ffs(v) - 1;
                        if (slot < a.cap) a.idx_out[slot] = (int32_t)(w * 32 + b);
                        ++slot;
                        v &= v - 1u;
                    }
                }
            }
        }
    }

    // 4. rows, one per wavefront
    const int64_t nchunks = (a.k + 7) / 8;
    const int64_t nbatch = (nchunks + (kBlockRow ? 256 : 64) * kBatch - 1) / ((kBlockRow ? 256 : 64) * kBatch);
    const bool vec_q = a.q && ((a.ldq & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.q) & 7) == 0);
    auto obyte = [&](int64_t col) -> uint32_t {
        return outl ? (bm[col >> 5] >> (col & 31)) & 0xffu : 0u;
    };
    auto chunk_max = [&](const uint4& vv, uint32_t obits) {
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = fabsf(h2f(half_at(vv, e)));
            t = ((obits >> e) & 1u) ? t : fmaxf(t, f);
        }
        return t;
    };
    __shared__ float rmax[4];
    for (int64_t rr = rr0; rr < a.rows_per_block; rr += kBlockRow ? 1 : 4) {
        const int64_t r = (int64_t)blockIdx.x * a.rows_per_block + rr;
        if (r >= a.m) break;
        const half_bits* __restrict__ xr = a.x + r * a.ldx;

        // 4a. absmax over the non-outlier columns
        float mx = 0.0f;
        for (int64_t b = 0; b < nbatch; ++b) {
            if (b > 0 || rr != rr0) load_batch(xr, b);  // batch 0 of the first row is in v
#pragma unroll
            for (int c = 0; c < kBatch; ++c) {
                const int64_t col = (b * P * kBatch + (int64_t)pid + P * c) * 8;
                if (col < a.k) mx = fmaxf(mx, chunk_max(v[c], obyte(col)));
            }
        }
        float s = wave_max(mx);
        if constexpr (kBlockRow) {
            if (lane == 0) rmax[wave] = s;
            __syncthreads();
            s = fmaxf(fmaxf(rmax[0], rmax[1]), fmaxf(rmax[2], rmax[3]));
            __syncthreads();
        }

        // 4b. codes, 4c. outlier gather
        const float inv = s > 0.0f ? 127.0f / s : 0.0f;  // IEEE division
        const bool zero_row = !(s > 0.0f);
        auto emit = [&](const uint4& vv, uint32_t obits, int64_t col) {
            if (a.q) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t b =
                        code_byte(h2f(half_at(vv, e)), inv, zero_row || ((obits >> e) & 1u));
                    if (e < 4) lo |= b << (8 * e);
                    else hi |= b << (8 * (e - 4));
                }
                int8_t* qr = a.q + r * a.ldq + col;
                if (vec_q && col + 8 <= a.k) {
                    *reinterpret_cast<uint2*>(qr) = make_uint2(lo, hi);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e < a.k)
                            qr[e] = (int8_t)(((e < 4 ? lo : hi) >> (8 * (e & 3))) & 0xffu);
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
                        if (slot < a.cap) a.x_out[r * a.ldo + slot] = half_at(vv, e);
                    }
                }
            }
        };
        for (int64_t b = 0; b < nbatch; ++b) {
            if (nbatch > 1) load_batch(xr, b);  // one batch: still in registers
#pragma unroll
            for (int c = 0; c < kBatch; ++c) {
                const int64_t col = (b * P * kBatch + (int64_t)pid + P * c) * 8;
                if (col < a.k) emit(v[c], obyte(col), col);
            }
        }
        if (a.q) {
            for (int64_t j = a.k + pid; j < a.kpad; j += P) a.q[r * a.ldq + j] = 0;
            if (pid == 0) a.absmax[r] = s;
        }
        if (a.x_out)
            for (int32_t t = kept + pid; t < a.xo_cols; t += P) a.x_out[r * a.ldo + t] = 0;
    }
}

hipError_t launch_detect(const half_bits* x, int64_t m, int64_t k, int64_t ldx, float threshold,
                         const QuantPlan& plan, uint32_t* partial, hipStream_t stream) {
    const bool vec = ((ldx & 7) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    dim3 grid((unsigned)plan.detect_gx, (unsigned)plan.row_blocks);
    if (vec)
        hipLaunchKernelGGL(detect_kernel<true>, grid, dim3(256), 0, stream, x, m, k, ldx, threshold,
                           plan.rows_per_detect_block, plan.words, partial);
    else
        hipLaunchKernelGGL(detect_kernel<false>, grid, dim3(256), 0, stream, x, m, k, ldx,
                           threshold, plan.rows_per_detect_block, plan.words, partial);
    return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs& a, hipStream_t stream) {
    const bool vec = ((a.ldx & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
    const size_t lds = (size_t)a.words * 2 * sizeof(uint32_t);
    // few rows: one workgroup per row, all of its threads on that row
    if (a.m <= 64) {
        QuantArgs b = a;
        b.rows_per_block = 1;
        dim3 grid((unsigned)(a.m > 0 ? a.m : 1));
        if (vec)
            hipLaunchKernelGGL((quant_kernel<true, true>), grid, dim3(256), lds, stream, b);
        else
            hipLaunchKernelGGL((quant_kernel<false, true>), grid, dim3(256), lds, stream, b);
        return hipGetLastError();
    }
    const int64_t blocks = ceil_div(a.m, a.rows_per_block);
    dim3 grid((unsigned)blocks);
    if (vec)
        hipLaunchKernelGGL((quant_kernel<true, false>), grid, dim3(256), lds, stream, a);
    else
        hipLaunchKernelGGL((quant_kernel<false, false>), grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

}  // namespace i8mp

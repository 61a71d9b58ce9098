// Outlier-column detection, row calibration, int8 quantization and outlier
// extraction for gfx950.
//
// The method keeps outlier feature columns in fp16 and quantizes the rest of
// each row to int8 with its own absmax (transformers PR "`bitsandbytes` -
// `Linear8bitLt` integration into `transformers` models", "About the mixed
// quantization method in few words"; bitsandbytes PR "LLM.int8() Refactoring:
// Part 1", "Enhancements": calibration and quantization fused in one op).
//
// A row's scale excludes every outlier column and the outlier set is a
// property of all rows, so every row waits for one global view of the outlier
// columns; the work is split at that point:
//   detect_kernel  one pass over x: per (row block, 256 or 64 columns) workgroup, a
//                  word per 32 columns of the row block's partial bitmap
//                  (every word written, no atomics, at most 8 row blocks);
//   quant_kernel   ORs the partial bitmaps into LDS, then quantizes one row per
//                  wavefront (short rows) or per workgroup (long rows), in one
//                  batch of 16-byte loads per row up to 32768 columns:
//                  wavefront-shuffle absmax over the non-outlier columns, IEEE
//                  fp32 quantization, 8-byte code stores, gather of the outlier
//                  values into the compact fp16 matrix.  Workgroup 0 also
//                  writes the bitmap, the ascending index list and the count.
//
// One or two rows of at most 65536 columns (decode) take quant_small_kernel:
// one workgroup of 1024 threads holds all of x in registers and does every
// step in one launch.
//
// (A single kernel with a grid-wide meeting point instead of the second
// launch measured slower on MI355X: the device-scope release / acquire round
// trips it needs cost more than the launch they replace.)
//
// Codes: fl32(127 / absmax) by IEEE division, x * that in fp32, round half to
// even, clamp to [-127, 127]; 0 in outlier columns and in rows whose absmax
// is 0.
#include "common.h"
#include "quant_util.h"

namespace i8mp {

namespace {
// whole 16-byte chunks of x: k and ldx multiples of 8, x 16-byte aligned
bool vector_rows(const QuantArgs& a) {
    return ((a.k & 7) == 0) && ((a.ldx & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
}
}  // namespace

// ---------------------------------------------------------------------------
// detect: per (RB rows, 8 CG columns) workgroup, the OR of the rows' outlier
// bits, written to the row block's partial bitmap (every word, no atomics).
// CG lanes read one row's 16 CG-byte segment, 256 / CG rows at a time: 256
// columns (512-byte segments) where that fills the GPU, else 64 columns
// (128-byte segments, four times the workgroups).
template <bool kVec, int CG>
__global__ __launch_bounds__(256) void detect_kernel(const half_bits* __restrict__ x, int64_t m, int64_t k,
                                                     int64_t ldx, float tau, int64_t rows_per_block,
                                                     int64_t words, uint32_t* __restrict__ partial) {
    constexpr int RL = 256 / CG;         // rows read together (CG groups of 8 columns per row)
    static_assert(CG % 4 == 0 && 256 % CG == 0, "whole bitmap words per workgroup");
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rsub = tid / CG;
    const int64_t col0 = (int64_t)blockIdx.x * (8 * CG) + cg * 8;
    const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
    int64_t r_end = r_begin + rows_per_block;
    if (r_end > m) r_end = m;

    uint32_t mask = 0;
    if (col0 < k) {
        if (kVec && col0 + 8 <= k) {
#pragma unroll 8
            for (int64_t r = r_begin + rsub; r < r_end; r += RL)
                mask |= outlier_bits8(*reinterpret_cast<const uint4*>(x + r * ldx + col0), tau);
        } else {
            for (int64_t r = r_begin + rsub; r < r_end; r += RL)
                mask |= outlier_bits8(load8<false>(x + r * ldx, col0, k), tau);
        }
    }
    __shared__ uint32_t red[256];
    red[tid] = mask;
    __syncthreads();
    if (tid < CG / 4) {
        uint32_t word = 0;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int g = tid * 4 + q4;
            uint32_t mm = 0;
            for (int q = 0; q < RL; ++q) mm |= red[q * CG + g];
            word |= (mm & 0xffu) << (8 * q4);
        }
        const int64_t w = (int64_t)blockIdx.x * (CG / 4) + tid;
        if (w < words) partial[(int64_t)blockIdx.y * words + w] = word;
    }
}

// ---------------------------------------------------------------------------
// quant: the OR of the partial bitmaps into LDS (8 independent loads per
// thread in flight, folded with ds_or), then rows: one per wavefront
// (kBlockRow false) or one per workgroup (true), kBatch 16-byte loads per lane
// in flight per batch.  A row of at most one batch stays in registers; a
// longer row is read twice, the second time from L2 / the infinity cache.
template <bool kVec, bool kBlockRow, int kBatch>
__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a) {
    extern __shared__ uint32_t smem[];
    uint32_t* bm = smem;                                       // [words]
    int32_t* pre = reinterpret_cast<int32_t*>(smem + a.words);  // [words]
    __shared__ int32_t wave_tot[4];
    __shared__ float rmax[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool outl = a.bitmap_in != nullptr;

    // the first row's first batch goes out before the bitmap work
    constexpr int P = kBlockRow ? 256 : 64;  // threads sharing a row
    const int pid = kBlockRow ? tid : lane;
    const int64_t rr0 = kBlockRow ? 0 : wave;
    const int64_t r_first = (int64_t)blockIdx.x * a.rows_per_block + rr0;
    const bool preload = rr0 < a.rows_per_block && r_first < a.m;
    // chunk indices (8 columns each) fit 32 bits: k <= 133144
    const int32_t nchunks = (int32_t)((a.k + 7) / 8);
    uint4 v[kBatch];
    auto load_batch = [&](const half_bits* __restrict__ xr, int32_t b) {
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int32_t ch = b * P * kBatch + pid + P * c;
            v[c] = ch < nchunks ? load8<kVec>(xr, (int64_t)ch * 8, a.k) : make_uint4(0, 0, 0, 0);
        }
    };
    if (preload) load_batch(a.x + r_first * a.ldx, 0);

    if (outl) {
        for (int64_t w = tid; w < a.words; w += 256) bm[w] = 0u;
        __syncthreads();
        const int64_t total_words = a.row_blocks * a.words;
        for (int64_t f0 = tid; f0 < total_words; f0 += 256 * 8) {
            uint32_t pw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t f = f0 + 256 * u;
                pw[u] = f < total_words ? a.bitmap_in[f] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (pw[u]) atomicOr(&bm[(f0 + 256 * u) % a.words], pw[u]);
        }
        __syncthreads();
        if (tid == 0 && (a.k & 31)) bm[a.words - 1] &= (1u << (a.k & 31)) - 1u;
    }
    __syncthreads();
    const bool need_prefix = outl && (a.x_out || a.idx_out || a.count_out);
    const int32_t total = need_prefix ? bitmap_prefix(bm, pre, a.words, wave_tot) : 0;
    const int32_t kept = total < a.cap ? total : a.cap;
    if (blockIdx.x == 0) publish(a, bm, pre, total, outl);

    const int32_t nbatch = (nchunks + P * kBatch - 1) / (P * kBatch);
    // byte c of the bitmap: the outlier bits of chunk c (8 columns)
    const uint8_t* bmb = reinterpret_cast<const uint8_t*>(bm);
    // a batch's chunks with their outlier columns set to 0: the packed fp16
    // maximum of the rest is the row absmax over the non-outlier columns, and
    // the clamp-free codes of the rest are the codes, 0 in outlier columns
    auto mask_batch = [&](int32_t b) {
        if (!outl) return;
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int32_t ch = b * P * kBatch + pid + P * c;
            v[c] = mask_outliers(v[c], ch < nchunks ? (uint32_t)bmb[ch] : 0u);
        }
    };
    for (int64_t rr = rr0; rr < a.rows_per_block; rr += kBlockRow ? 1 : 4) {
        const int64_t r = (int64_t)blockIdx.x * a.rows_per_block + rr;
        if (r >= a.m) break;
        const half_bits* __restrict__ xr = a.x + r * a.ldx;

        float mx = 0.0f;
        for (int32_t b = 0; b < nbatch; ++b) {
            if (b > 0 || rr != rr0) load_batch(xr, b);  // batch 0 of the first row is in v
            mask_batch(b);
#pragma unroll
            for (int c = 0; c < kBatch; ++c) mx = fmaxf(mx, chunk_absmax(v[c]));  // chunks past k are 0
        }
        float s = wave_max_uniform(mx);
        if constexpr (kBlockRow) {
            if (lane == 0) rmax[wave] = s;
            __syncthreads();
            s = fmaxf(fmaxf(rmax[0], rmax[1]), fmaxf(rmax[2], rmax[3]));
            __syncthreads();
        }
        const float inv = s > 0.0f ? 127.0f / s : 0.0f;  // IEEE division; 0 for a zero row
        if (a.q) {
            int8_t* qr = a.q + r * a.ldq;
            for (int32_t b = 0; b < nbatch; ++b) {
                if (nbatch > 1) {  // one batch: still in registers, masked
                    load_batch(xr, b);
                    mask_batch(b);
                }
#pragma unroll
                for (int c = 0; c < kBatch; ++c) {
                    const int32_t ch = b * P * kBatch + pid + P * c;
                    if (ch >= nchunks) continue;
                    const int64_t col = (int64_t)ch * 8;
                    const uint2 code = codes8_plain(v[c], inv);
                    if (kVec) {  // whole chunks, 8-byte aligned code rows (checked by the launcher)
                        *reinterpret_cast<uint2*>(qr + col) = code;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (col + e < a.k) qr[col + e] = (int8_t)(((e < 4 ? code.x : code.y) >> (8 * (e & 3))) & 0xffu);
                    }
                }
            }
            for (int64_t j = a.k + pid; j < a.kpad; j += P) qr[j] = 0;
            if (pid == 0) a.absmax[r] = s;
        }
        // the row's outlier values into their slots of the compact matrix
        // (bitmap words walked in order, slot from the prefix), zeros after
        if (a.x_out) {
            if (total > 0)
                for (int64_t w = pid; w < a.words; w += P) {
                    uint32_t bits = bm[w];
                    int32_t slot = bits ? pre[w] : 0;
                    while (bits) {
                        const int64_t j = w * 32 + (__ffs(bits) - 1);
                        bits &= bits - 1u;
                        if (slot < a.cap) a.x_out[r * a.ldo + slot] = xr[j];
                        ++slot;
                    }
                }
            for (int32_t t = kept + pid; t < a.xo_cols; t += P) a.x_out[r * a.ldo + t] = 0;
        }
    }
}

// ---------------------------------------------------------------------------
// One or two rows (decode): one workgroup of 1024 threads holds all of x in
// registers and so sees the whole outlier set itself: detection, calibration,
// quantization and extraction in one launch, x read once.  Chunk f = tid +
// 1024 i of the flattened (row, 8-column chunk) range, L per thread.  (For
// more rows one workgroup's memory pipeline measured slower than the two
// kernels, which spread the rows over the CUs.)
constexpr int kSmallThreads = 1024;
constexpr int kSmallMaxL = 8;
constexpr int kSmallMaxRows = 2;

template <bool kVec, int L>
__global__ __launch_bounds__(1024) void quant_small_kernel(QuantArgs a) {
    extern __shared__ uint32_t smem[];
    uint32_t* bm = smem;                                       // [words]
    int32_t* pre = reinterpret_cast<int32_t*>(smem + a.words);  // [words]
    uint32_t* rmax = smem + 2 * a.words;                        // [m] float bits
    float* rinv = reinterpret_cast<float*>(rmax + a.m);         // [m]
    __shared__ int32_t wave_tot[kSmallThreads / 64];

    const int tid = threadIdx.x;
    const bool outl = a.threshold > 0.0f;
    const int32_t cpr = (int32_t)((a.k + 7) / 8);
    const int32_t total_chunks = (int32_t)a.m * cpr;

    uint4 v[L];
    uint32_t rc[L];  // row << 16 | chunk (rows < kSmallMaxRows, chunks < 65536)
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int32_t f = tid + kSmallThreads * i;
        const int32_t r = f / cpr, ch = f - r * cpr;
        rc[i] = ((uint32_t)r << 16) | (uint32_t)ch;
        v[i] = f < total_chunks ? load8<kVec>(a.x + r * a.ldx, (int64_t)ch * 8, a.k) : make_uint4(0, 0, 0, 0);
    }
    for (int64_t w = tid; w < a.words; w += kSmallThreads) bm[w] = 0u;
    for (int64_t r = tid; r < a.m; r += kSmallThreads) rmax[r] = 0u;
    __syncthreads();
    if (outl) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
            if (tid + kSmallThreads * i < total_chunks) {
                const uint32_t bits = outlier_bits8(v[i], a.threshold);
                const int32_t ch = (int32_t)(rc[i] & 0xffffu);
                if (bits) atomicOr(&bm[ch >> 2], bits << ((ch & 3) * 8));
            }
        }
        __syncthreads();
    }
    const bool need_prefix = outl && (a.x_out || a.idx_out || a.count_out);
    const int32_t total = need_prefix ? bitmap_prefix(bm, pre, a.words, wave_tot) : 0;
    const int32_t kept = total < a.cap ? total : a.cap;
    publish(a, bm, pre, total, outl);

    // row absmax over the non-outlier columns (float bits order as uints for x >= 0)
    auto obyte = [&](int32_t ch) -> uint32_t { return outl ? (bm[ch >> 2] >> ((ch & 3) * 8)) & 0xffu : 0u; };
#pragma unroll
    for (int i = 0; i < L; ++i) {
        if (tid + kSmallThreads * i < total_chunks) {
            const float mx = chunk_max(v[i], obyte((int32_t)(rc[i] & 0xffffu)));
            if (mx > 0.0f) atomicMax(&rmax[rc[i] >> 16], __float_as_uint(mx));
        }
    }
    __syncthreads();
    for (int64_t r = tid; r < a.m; r += kSmallThreads) {
        const float s = __uint_as_float(rmax[r]);
        rinv[r] = s > 0.0f ? 127.0f / s : 0.0f;  // IEEE division
        if (a.q) a.absmax[r] = s;
    }
    __syncthreads();

    const bool vec_q = a.q && ((a.ldq & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.q) & 7) == 0);
#pragma unroll
    for (int i = 0; i < L; ++i) {
        if (tid + kSmallThreads * i < total_chunks) {
            const int32_t r = (int32_t)(rc[i] >> 16), ch = (int32_t)(rc[i] & 0xffffu);
            const float s = __uint_as_float(rmax[r]);
            emit8(a, v[i], obyte(ch), r, (int64_t)ch * 8, rinv[r], !(s > 0.0f), vec_q, bm, pre);
        }
    }
    if (a.q && a.kpad > a.k) {
        const int64_t pad = a.kpad - a.k;
        for (int64_t f = tid; f < a.m * pad; f += kSmallThreads) a.q[(f / pad) * a.ldq + a.k + f % pad] = 0;
    }
    if (a.x_out && a.xo_cols > kept) {
        const int64_t pad = a.xo_cols - kept;
        for (int64_t f = tid; f < a.m * pad; f += kSmallThreads) a.x_out[(f / pad) * a.ldo + kept + f % pad] = 0;
    }
}

// ---------------------------------------------------------------------------

namespace {

template <bool kVec, int L>
hipError_t launch_small_l(const QuantArgs& a, size_t lds, hipStream_t stream) {
    hipLaunchKernelGGL((quant_small_kernel<kVec, L>), dim3(1), dim3(kSmallThreads), lds, stream, a);
    return hipGetLastError();
}

template <bool kVec>
hipError_t launch_small(const QuantArgs& a, int64_t per_thread, size_t lds, hipStream_t stream) {
    if (per_thread <= 1) return launch_small_l<kVec, 1>(a, lds, stream);
    if (per_thread <= 2) return launch_small_l<kVec, 2>(a, lds, stream);
    if (per_thread <= 4) return launch_small_l<kVec, 4>(a, lds, stream);
    return launch_small_l<kVec, 8>(a, lds, stream);
}

// kBatch: the 16-byte loads per lane in flight, as many as the row needs up
// to 16 (longer rows take several batches)
template <bool kVec, bool kBlockRow>
hipError_t launch_rows(const QuantArgs& a, int64_t blocks, size_t lds, hipStream_t stream) {
    constexpr int P = kBlockRow ? 256 : 64;
    const int64_t per_lane = ceil_div(ceil_div(a.k, 8), P);
    const dim3 grid((unsigned)blocks), block(256);
    if (per_lane <= 2)
        hipLaunchKernelGGL((quant_kernel<kVec, kBlockRow, 2>), grid, block, lds, stream, a);
    else if (per_lane <= 4)
        hipLaunchKernelGGL((quant_kernel<kVec, kBlockRow, 4>), grid, block, lds, stream, a);
    else if (per_lane <= 8)
        hipLaunchKernelGGL((quant_kernel<kVec, kBlockRow, 8>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((quant_kernel<kVec, kBlockRow, 16>), grid, block, lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows(const QuantArgs& in, hipStream_t stream) {
    QuantArgs a = in;
    const bool vec = vector_rows(a);
    const size_t lds = (size_t)a.words * 2 * sizeof(uint32_t);
    const int64_t cpr = (a.k + 7) / 8;
    // a workgroup per row for long rows (over 4096 columns), for few rows, and
    // for rows of 2048+ columns when there are at most 512 of them (one row per
    // workgroup spreads the per-element work over the CUs); else a wavefront
    // per row
    const bool block_row = cpr > 512 || a.m <= 64 || (cpr >= 256 && a.m <= 512);
    int64_t blocks;
    // enough rows per workgroup to amortize the OR of the partial bitmaps;
    // up to 1024 workgroups for a workgroup per row (about four per CU, whose
    // row loads overlap: 7B down and 65B up quantize 8-9 % faster than with 512)
    if (block_row) {
        a.rows_per_block = a.m > 0 ? ceil_div(a.m, 1024) : 0;
        blocks = a.m > 0 ? ceil_div(a.m, a.rows_per_block) : 1;
    } else {
        a.rows_per_block = 4 * ceil_div(a.m, 4 * 512);
        blocks = ceil_div(a.m, a.rows_per_block);
    }
    // the vector path also stores whole 8-byte code chunks
    const bool vec_codes = vec && (!a.q || (((a.ldq & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.q) & 7) == 0)));
    if (vec_codes)
        return block_row ? launch_rows<true, true>(a, blocks, lds, stream)
                         : launch_rows<true, false>(a, blocks, lds, stream);
    return block_row ? launch_rows<false, true>(a, blocks, lds, stream)
                     : launch_rows<false, false>(a, blocks, lds, stream);
}

hipError_t launch_quantize(const QuantArgs& in, hipStream_t stream) {
    QuantArgs a = in;
    const bool vec = vector_rows(a);
    a.bitmap_in = nullptr;
    const int64_t per_thread = ceil_div(a.m * ceil_div(a.k, 8), kSmallThreads);
    if (a.m > 0 && a.m <= kSmallMaxRows && per_thread <= kSmallMaxL) {
        const size_t lds = ((size_t)a.words * 2 + (size_t)a.m * 2) * sizeof(uint32_t);
        return vec ? launch_small<true>(a, per_thread, lds, stream) : launch_small<false>(a, per_thread, lds, stream);
    }
    if (a.threshold > 0.0f && a.m > 0) {
        // detect: 256 or 64 columns x RB rows per workgroup, at most
        // kMaxRowBlocks row blocks (RB >= 8), about 1024 workgroups when the
        // shape allows
        auto row_blocks = [&](int64_t gx) {
            int64_t gy = ceil_div(1024, gx);
            if (gy > kMaxRowBlocks) gy = kMaxRowBlocks;
            if (gy > ceil_div(a.m, 8)) gy = ceil_div(a.m, 8);
            return gy < 1 ? (int64_t)1 : gy;
        };
        const bool narrow = ceil_div(a.k, 256) * row_blocks(ceil_div(a.k, 256)) < 256;
        const int64_t gx = ceil_div(a.k, narrow ? 64 : 256);
        int64_t gy = row_blocks(gx);
        const int64_t rb = round_up(ceil_div(a.m, gy), 8);
        gy = ceil_div(a.m, rb);
        const dim3 grid((unsigned)gx, (unsigned)gy);
        if (vec && narrow)
            hipLaunchKernelGGL((detect_kernel<true, 8>), grid, dim3(256), 0, stream, a.x, a.m, a.k, a.ldx, a.threshold,
                               rb, a.words, a.partial);
        else if (vec)
            hipLaunchKernelGGL((detect_kernel<true, 32>), grid, dim3(256), 0, stream, a.x, a.m, a.k, a.ldx,
                               a.threshold, rb, a.words, a.partial);
        else if (narrow)
            hipLaunchKernelGGL((detect_kernel<false, 8>), grid, dim3(256), 0, stream, a.x, a.m, a.k, a.ldx,
                               a.threshold, rb, a.words, a.partial);
        else
            hipLaunchKernelGGL((detect_kernel<false, 32>), grid, dim3(256), 0, stream, a.x, a.m, a.k, a.ldx,
                               a.threshold, rb, a.words, a.partial);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        a.bitmap_in = a.partial;
        a.row_blocks = gy;
    }
    return launch_quant_rows(a, stream);
}

}  // namespace i8mp

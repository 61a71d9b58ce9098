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
// step in one launch.  Three to sixteen rows take two launches over column
// slices (cs1_kernel, cs2_kernel); from 1024 rows x is read once
// (quant1_kernel, quant2_kernel).
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

typedef unsigned v2u_q __attribute__((ext_vector_type(2)));

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
    // kVec: buffer loads (chunks past k read 0) with no branch per chunk
    auto load_batch = [&](const half_bits* __restrict__ xr, int32_t b) {
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xr, kVec ? a.k * 2 : 0);
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int32_t ch = b * P * kBatch + pid + P * c;
            if constexpr (kVec)
                v[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ch * 16, 0, 0));
            else
                v[c] = ch < nchunks ? load8<false>(xr, (int64_t)ch * 8, a.k) : make_uint4(0, 0, 0, 0);
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
            // kVec: whole 8-byte chunks (checked by the launcher) through one
            // buffer range up to kpad (chunks past it dropped), no branch per
            // chunk; the chunks past k hold zeros, so they write the padding
            const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qr, kVec ? a.kpad : 0);
            for (int32_t b = 0; b < nbatch; ++b) {
                if (nbatch > 1) {  // one batch: still in registers, masked
                    load_batch(xr, b);
                    mask_batch(b);
                }
#pragma unroll
                for (int c = 0; c < kBatch; ++c) {
                    const int32_t ch = b * P * kBatch + pid + P * c;
                    const int64_t col = (int64_t)ch * 8;
                    const uint2 code = codes8_plain(v[c], inv);
                    if constexpr (kVec) {
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u_q, code), rq, ch * 8, 0, 0);
                    } else {
                        if (ch >= nchunks) continue;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (col + e < a.k) qr[col + e] = (int8_t)(((e < 4 ? code.x : code.y) >> (8 * (e & 3))) & 0xffu);
                    }
                }
            }
            const int64_t pad0 = kVec ? (int64_t)nbatch * P * kBatch * 8 : a.k;
            for (int64_t j = pad0 + pid; j < a.kpad; j += P) qr[j] = 0;
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
// One read of x for prefill-sized inputs (threshold > 0), three launches:
//   zero_words_kernel  clears kMaxRowBlocks partial outlier bitmaps in the
//                      scratch (a kernel, not a memset node, so that the call
//                      can be captured in a graph);
//   quant1_kernel      reads each row once: the outlier bits of its elements
//                      (into the workgroup's LDS bitmap, then OR-ed into partial
//                      bitmap blockIdx % kMaxRowBlocks with atomics on the
//                      words that have any), the
//                      row maximum m over the elements below the threshold, and
//                      the codes with fl32(127 / m), 0 at elements at or above
//                      the threshold;
//   quant2_kernel      with the whole outlier set (the OR of the partials): the
//                      bitmap, index list and count;
//                      per row the gather of its outlier-column values, zero
//                      codes in the outlier columns, and the check of the row
//                      scale.  The scale is the maximum over the columns outside
//                      the set, which is m unless m is reached only inside the
//                      set: when the largest element of an outlier column below
//                      the threshold equals m, the row is quantized again from
//                      the bitmap (exact; rare: every element of a planted
//                      outlier column is above the threshold).
// The codes of such a check are the two-launch quantizer's own: the same
// masked chunk maxima, the same IEEE quotient and rounding.

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ w, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) w[i] = 0u;
}

template <bool kVec, bool kBlockRow, int kBatch>
__global__ __launch_bounds__(256) void quant1_kernel(QuantArgs a, uint32_t* __restrict__ gbm) {
    extern __shared__ uint32_t smem[];
    uint32_t* bm = smem;   // [words] this workgroup's outlier bits
    __shared__ float rmax[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int P = kBlockRow ? 256 : 64;   // threads sharing a row
    const int pid = kBlockRow ? tid : lane;
    const int64_t rr0 = kBlockRow ? 0 : wave;
    const int64_t rstep = kBlockRow ? 1 : 4;
    const int32_t nchunks = (int32_t)((a.k + 7) / 8);
    const int32_t nbatch = (nchunks + P * kBatch - 1) / (P * kBatch);
    const float tau = a.threshold;

    uint4 v[kBatch], vn[kBatch];
    // kVec: buffer loads (chunks past k read 0) with no branch per chunk
    auto load_batch = [&](uint4 (&dst)[kBatch], const half_bits* __restrict__ xr, int32_t b) {
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xr, kVec ? a.k * 2 : 0);
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int32_t ch = b * P * kBatch + pid + P * c;
            if constexpr (kVec)
                dst[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ch * 16, 0, 0));
            else
                dst[c] = ch < nchunks ? load8<false>(xr, (int64_t)ch * 8, a.k) : make_uint4(0, 0, 0, 0);
        }
    };
    // a batch's outlier bits into LDS and the elements at or above the
    // threshold set to 0; returns the maximum of the rest
    auto detect_mask = [&](int32_t b, bool record) {
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int32_t ch = b * P * kBatch + pid + P * c;
            const float cm = chunk_absmax(v[c]);   // chunks past k are 0
            if (cm >= tau) {
                const uint32_t ob = outlier_bits8(v[c], tau);
                if (record) atomicOr(&bm[ch >> 2], ob << ((ch & 3) * 8));
                v[c] = mask_outliers(v[c], ob);
                mx = fmaxf(mx, chunk_absmax(v[c]));
            } else {
                mx = fmaxf(mx, cm);
            }
        }
        return mx;
    };

    const int64_t r_first = (int64_t)blockIdx.x * a.rows_per_block + rr0;
    if (rr0 < a.rows_per_block && r_first < a.m) load_batch(v, a.x + r_first * a.ldx, 0);
    for (int64_t w = tid; w < a.words; w += 256) bm[w] = 0u;
    __syncthreads();

    for (int64_t rr = rr0; rr < a.rows_per_block; rr += rstep) {
        const int64_t r = (int64_t)blockIdx.x * a.rows_per_block + rr;
        if (r >= a.m) break;
        const half_bits* __restrict__ xr = a.x + r * a.ldx;
        const int64_t rn = r + rstep;
        const bool next = rr + rstep < a.rows_per_block && rn < a.m;
        float mx = 0.0f;
        for (int32_t b = 0; b < nbatch; ++b) {
            if (b > 0) load_batch(v, xr, b);   // batch 0 is in v
            mx = fmaxf(mx, detect_mask(b, true));
        }
        // a row of one batch: the next row's loads go out before this row's
        // reduction and codes
        if (nbatch == 1 && next) load_batch(vn, a.x + rn * a.ldx, 0);
        float s = wave_max_uniform(mx);
        if constexpr (kBlockRow) {
            if (lane == 0) rmax[wave] = s;
            __syncthreads();
            s = fmaxf(fmaxf(rmax[0], rmax[1]), fmaxf(rmax[2], rmax[3]));
            __syncthreads();
        }
        const float inv = s > 0.0f ? 127.0f / s : 0.0f;   // IEEE division; 0 for a zero row
        int8_t* qr = a.q + r * a.ldq;
        // kVec: the row's codes and its zero padding to kpad through one
        // buffer range (chunks past kpad are dropped), no branch per chunk
        const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qr, kVec ? a.kpad : 0);
        for (int32_t b = 0; b < nbatch; ++b) {
            if (nbatch > 1) {   // longer rows: read again (L2 / infinity cache)
                load_batch(v, xr, b);
                detect_mask(b, false);
            }
#pragma unroll
            for (int c = 0; c < kBatch; ++c) {
                const int32_t ch = b * P * kBatch + pid + P * c;
                const int64_t col = (int64_t)ch * 8;
                const uint2 code = codes8_plain(v[c], inv);   // chunks past k are 0: codes 0
                if constexpr (kVec) {
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u_q, code), rq, ch * 8, 0, 0);
                } else {
                    if (ch >= nchunks) continue;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e < a.k) qr[col + e] = (int8_t)(((e < 4 ? code.x : code.y) >> (8 * (e & 3))) & 0xffu);
                }
            }
        }
        // padding past the chunks written above (kVec writes whole batches)
        const int64_t pad0 = kVec ? (int64_t)nbatch * P * kBatch * 8 : a.k;
        for (int64_t j = pad0 + pid; j < a.kpad; j += P) qr[j] = 0;
        if (pid == 0) a.absmax[r] = s;
        if (nbatch == 1 && next) {
#pragma unroll
            for (int c = 0; c < kBatch; ++c) v[c] = vn[c];
        } else if (next) {
            load_batch(v, a.x + rn * a.ldx, 0);
        }
    }
    __syncthreads();
    // Every workgroup finds much the same outlier columns, and atomics on
    // one word serialize at L2: the workgroups spread over kMaxRowBlocks
    // partial bitmaps.  The atomics return nothing, so no wave waits for them
    // (a wait here would also wait for the row's code stores).
    uint32_t* part = gbm + (int64_t)(blockIdx.x % kMaxRowBlocks) * a.words;
    for (int64_t w = tid; w < a.words; w += 256) {
        const uint32_t b = bm[w];
        if (b) atomicOr(&part[w], b);
    }
}

// A wave per row.  kVec: 16-byte chunks of x and 8-byte code stores.
// outlier columns whose slot -> column list quant2_kernel keeps in LDS (more:
// each row walks the bitmap words)
constexpr int kQ2Cols = 2048;

template <bool kVec>
__global__ __launch_bounds__(256) void quant2_kernel(QuantArgs a, const uint32_t* __restrict__ gbm) {
    extern __shared__ uint32_t smem[];
    uint32_t* bm = smem;                                       // [words]
    int32_t* pre = reinterpret_cast<int32_t*>(smem + a.words);  // [words]
    int32_t* cols = pre + a.words;                             // [kQ2Cols] column of each slot
    __shared__ int32_t wave_tot[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int64_t w = tid; w < a.words; w += 256) {
        uint32_t b = 0;
#pragma unroll
        for (int p = 0; p < kMaxRowBlocks; ++p) b |= gbm[(int64_t)p * a.words + w];
        bm[w] = b;
    }
    __syncthreads();
    const int32_t total = bitmap_prefix(bm, pre, a.words, wave_tot);
    const int32_t kept = total < a.cap ? total : a.cap;
    if (blockIdx.x == 0) publish(a, bm, pre, total, true);
    const bool listed = total <= kQ2Cols;
    if (listed && total > 0) {
        for (int64_t w = tid; w < a.words; w += 256) {
            uint32_t bits = bm[w];
            int32_t slot = pre[w];
            while (bits) {
                cols[slot++] = (int32_t)(w * 32 + (__ffs(bits) - 1));
                bits &= bits - 1u;
            }
        }
        __syncthreads();
    }
    const float tau = a.threshold;
    const uint8_t* bmb = reinterpret_cast<const uint8_t*>(bm);
    const int32_t nchunks = (int32_t)((a.k + 7) / 8);
    for (int64_t rr = wave; rr < a.rows_per_block; rr += 4) {
        const int64_t r = (int64_t)blockIdx.x * a.rows_per_block + rr;
        if (r >= a.m) break;
        const half_bits* __restrict__ xr = a.x + r * a.ldx;
        // the row's outlier-column values: the gather, zero codes there, and
        // their largest magnitude below the threshold
        float t = 0.0f;
        if (listed) {
            // slots lane, lane + 64, ...: the loads of a batch go out together
            constexpr int B = 4;
            for (int32_t s0 = 0; s0 < total; s0 += 64 * B) {
                int32_t j[B];
                half_bits h[B];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int32_t slot = s0 + 64 * b + lane;
                    j[b] = slot < total ? cols[slot] : -1;
                }
#pragma unroll
                for (int b = 0; b < B; ++b) h[b] = j[b] >= 0 ? xr[j[b]] : (half_bits)0;
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    if (j[b] < 0) continue;
                    const int32_t slot = s0 + 64 * b + lane;
                    if (a.x_out && slot < a.cap) a.x_out[r * a.ldo + slot] = h[b];
                    const float f = fabsf(h2f(h[b]));
                    if (f < tau) t = fmaxf(t, f);
                    if (a.q) a.q[r * a.ldq + j[b]] = 0;
                }
            }
        } else
            for (int64_t w = lane; w < a.words; w += 64) {
                uint32_t bits = bm[w];
                int32_t slot = bits ? pre[w] : 0;
                while (bits) {
                    const int64_t j = w * 32 + (__ffs(bits) - 1);
                    bits &= bits - 1u;
                    const half_bits h = xr[j];
                    if (a.x_out && slot < a.cap) a.x_out[r * a.ldo + slot] = h;
                    const float f = fabsf(h2f(h));
                    if (f < tau) t = fmaxf(t, f);
                    if (a.q) a.q[r * a.ldq + j] = 0;
                    ++slot;
                }
            }
        if (a.x_out)
            for (int32_t s2 = kept + lane; s2 < a.xo_cols; s2 += 64) a.x_out[r * a.ldo + s2] = 0;
        t = wave_max_uniform(t);
        if (!a.q || !(t > 0.0f) || t < a.absmax[r]) continue;
        // the row maximum below the threshold sits in an outlier column:
        // the scale over the columns outside the set, and the codes again
        float mx = 0.0f;
        for (int32_t ch = lane; ch < nchunks; ch += 64) {
            const uint4 v = mask_outliers(load8<kVec>(xr, (int64_t)ch * 8, a.k), (uint32_t)bmb[ch]);
            mx = fmaxf(mx, chunk_absmax(v));
        }
        const float s = wave_max_uniform(mx);
        const float inv = s > 0.0f ? 127.0f / s : 0.0f;   // IEEE division
        int8_t* qr = a.q + r * a.ldq;
        for (int32_t ch = lane; ch < nchunks; ch += 64) {
            const int64_t col = (int64_t)ch * 8;
            const uint2 code = codes8_plain(mask_outliers(load8<kVec>(xr, col, a.k), (uint32_t)bmb[ch]), inv);
            if (kVec) {
                *reinterpret_cast<uint2*>(qr + col) = code;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < a.k) qr[col + e] = (int8_t)(((e < 4 ? code.x : code.y) >> (8 * (e & 3))) & 0xffu);
            }
        }
        if (lane == 0) a.absmax[r] = s;
    }
}

// ---------------------------------------------------------------------------
// A few rows (decode, 3 to 16 rows), two launches over 256-column slices: a
// workgroup holds every row of its slice, so what it sees of the outlier set
// (the OR over the rows of each column) is final, and so is its share of each
// row's maximum over the non-outlier columns.
//   cs1_kernel  the slice's outlier bits (scratch bitmap, and the output
//               bitmap) and per row the maximum |x| over its non-outlier
//               columns (scratch, [slice x m]);
//   cs2_kernel  per row the absmax (the maximum over the slices), the codes of
//               the slice, and its outlier columns' slots (popcounts of the
//               words before it): index list entries and the gathered values.
//               Workgroup 0 writes the count, absmax, the index list's -1
//               tail and the zero padding of the gathered values.
// Thread t holds chunk t % 32 (8 columns) of rows t / 32 and t / 32 + 8.
constexpr int kCsRows = 16;
constexpr int kCsCols = 256;
constexpr int kCsBatch = 8;   // slices per lane whose scratch loads cs2 issues together

template <bool kVec>
__device__ inline void cs_load(const QuantArgs& a, uint4 (&v)[2], int rl, int64_t col) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t r = rl + 8 * h;
        v[h] = (r < a.m && col < a.k) ? load8<kVec>(a.x + r * a.ldx, col, a.k) : make_uint4(0, 0, 0, 0);
    }
}

template <bool kVec>
__global__ __launch_bounds__(256) void cs1_kernel(QuantArgs a, uint32_t* __restrict__ sbits,
                                                  float* __restrict__ spart) {
    const int tid = threadIdx.x, c = tid & 31, rl = tid >> 5;
    const int64_t col = (int64_t)blockIdx.x * kCsCols + c * 8;
    uint4 v[2];
    cs_load<kVec>(a, v, rl, col);
    __shared__ uint32_t red[256];
    red[tid] = outlier_bits8(v[0], a.threshold) | outlier_bits8(v[1], a.threshold);
    __syncthreads();
    uint32_t cb = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) cb |= red[q * 32 + c];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float mx = chunk_absmax(mask_outliers(v[h], cb));
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));   // the 32 chunks
        const int64_t r = rl + 8 * h;
        if (c == 0 && r < a.m) spart[(int64_t)blockIdx.x * a.m + r] = mx;
    }
    if (tid < kCsCols / 32) {
        uint32_t word = 0;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t mm = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) mm |= red[q * 32 + tid * 4 + q4];
            word |= (mm & 0xffu) << (8 * q4);
        }
        const int64_t w = (int64_t)blockIdx.x * (kCsCols / 32) + tid;
        if (w < a.words) {
            sbits[w] = word;
            if (a.bitmap_out) a.bitmap_out[w] = word;
        }
    }
}

template <bool kVec>
__global__ __launch_bounds__(256) void cs2_kernel(QuantArgs a, const uint32_t* __restrict__ sbits,
                                                  const float* __restrict__ spart, int64_t nslices) {
    const int tid = threadIdx.x, c = tid & 31, rl = tid >> 5, lane = tid & 63, wave = tid >> 6;
    const int64_t col = (int64_t)blockIdx.x * kCsCols + c * 8;
    uint4 v[2];
    cs_load<kVec>(a, v, rl, col);
    __shared__ float s_row[kCsRows];
    __shared__ uint32_t sb[kCsCols / 32];
    __shared__ int32_t wsum[2][4];
    // Every global load of the scratch is issued before the first is used:
    // the slice maxima (16 lanes per row) and the bitmap words (for the
    // popcounts) of up to kCsBatch * 16 slices.  Indexes past the end are
    // clamped to the last entry: a repeated maximum changes nothing, and a
    // repeated word is not counted.
    const int64_t w0 = (int64_t)blockIdx.x * (kCsCols / 32);
    const int64_t r16 = tid >> 4;
    const int u = tid & 15;
    const int64_t rr = r16 < a.m ? r16 : a.m - 1;
    float pv[kCsBatch];
    uint32_t wv[kCsBatch / 2];
#pragma unroll
    for (int i = 0; i < kCsBatch; ++i) {
        const int64_t sl = u + 16 * i;
        pv[i] = spart[(sl < nslices ? sl : nslices - 1) * a.m + rr];
    }
#pragma unroll
    for (int i = 0; i < kCsBatch / 2; ++i) {
        const int64_t w = tid + 256 * i;
        wv[i] = sbits[w < a.words ? w : a.words - 1];
    }
    if (tid < kCsCols / 32) sb[tid] = w0 + tid < a.words ? sbits[w0 + tid] : 0u;
    // row absmax
    {
        float pm = 0.0f;
#pragma unroll
        for (int i = 0; i < kCsBatch; ++i) pm = fmaxf(pm, pv[i]);
        for (int64_t sl = u + 16 * kCsBatch; sl < nslices; sl += 16) pm = fmaxf(pm, spart[sl * a.m + rr]);
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) pm = fmaxf(pm, __shfl_xor(pm, off, 64));
        if (u == 0 && r16 < a.m) s_row[r16] = pm;
    }
    // outlier columns before this slice, and in all
    int32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kCsBatch / 2; ++i) {
        const int64_t w = tid + 256 * i;
        const int32_t p = w < a.words ? __popc(wv[i]) : 0;
        tot += p;
        before += w < w0 ? p : 0;
    }
    for (int64_t w = tid + 256 * (kCsBatch / 2); w < a.words; w += 256) {
        const int32_t p = __popc(sbits[w]);
        tot += p;
        before += w < w0 ? p : 0;
    }
    before = wave_sum_i32(before);
    tot = wave_sum_i32(tot);
    if (lane == 0) {
        wsum[0][wave] = before;
        wsum[1][wave] = tot;
    }
    __syncthreads();
    const int32_t base = wsum[0][0] + wsum[0][1] + wsum[0][2] + wsum[0][3];
    const int32_t total = wsum[1][0] + wsum[1][1] + wsum[1][2] + wsum[1][3];
    const uint32_t cb = (sb[c >> 2] >> (8 * (c & 3))) & 0xffu;
    int32_t slot0 = base + __popc(sb[c >> 2] & ((1u << (8 * (c & 3))) - 1u));
    for (int w = 0; w < (c >> 2); ++w) slot0 += __popc(sb[w]);

    const bool vec_q = ((a.ldq & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.q) & 7) == 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t r = rl + 8 * h;
        if (r >= a.m) continue;
        if (a.q && col < a.kpad) {
            const float sr = s_row[r];
            const float inv = sr > 0.0f ? 127.0f / sr : 0.0f;   // IEEE division
            const uint2 code = codes8_plain(mask_outliers(v[h], cb), inv);
            int8_t* qr = a.q + r * a.ldq + col;
            if (vec_q && col + 8 <= a.kpad) {
                *reinterpret_cast<uint2*>(qr) = code;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < a.kpad) qr[e] = (int8_t)(((e < 4 ? code.x : code.y) >> (8 * (e & 3))) & 0xffu);
            }
        }
        if (cb) {
            int32_t slot = slot0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (!((cb >> e) & 1u)) continue;
                if (a.x_out && slot < a.cap) a.x_out[r * a.ldo + slot] = half_at(v[h], e);
                if (h == 0 && rl == 0 && a.idx_out && slot < a.idx_len) a.idx_out[slot] = (int32_t)(col + e);
                ++slot;
            }
        }
    }
    if (blockIdx.x == 0) {
        if (a.count_out && tid == 0) *a.count_out = total;
        if (a.absmax && tid < a.m) a.absmax[tid] = s_row[tid];
        if (a.idx_out)
            for (int32_t sl = total + tid; sl < a.idx_len; sl += 256) a.idx_out[sl] = -1;
        if (a.x_out) {
            const int32_t kept = total < a.cap ? total : a.cap;
            const int32_t pad = a.xo_cols - kept;
            for (int32_t i = tid; i < (int32_t)a.m * pad; i += 256)
                a.x_out[(int64_t)(i / pad) * a.ldo + kept + i % pad] = 0;
        }
    }
}

// the two launches; false when the scratch cannot hold the slice data
bool launch_col_slices(const QuantArgs& a, hipStream_t stream, hipError_t* err) {
    const int64_t span = a.kpad > a.k ? a.kpad : a.k;
    const int64_t nslices = ceil_div(span, kCsCols);
    const size_t need = (size_t)ceil_div(span, 32) * 4 + (size_t)nslices * a.m * 4;
    if (a.m > kCsRows || need > quant_scratch_bytes(a.k)) return false;
    uint32_t* sbits = a.partial;
    float* spart = reinterpret_cast<float*>(a.partial + ceil_div(span, 32));
    const bool vec = vector_rows(a);
    if (vec)
        hipLaunchKernelGGL((cs1_kernel<true>), dim3((unsigned)nslices), dim3(256), 0, stream, a, sbits, spart);
    else
        hipLaunchKernelGGL((cs1_kernel<false>), dim3((unsigned)nslices), dim3(256), 0, stream, a, sbits, spart);
    if ((*err = hipGetLastError()) != hipSuccess) return true;
    if (vec)
        hipLaunchKernelGGL((cs2_kernel<true>), dim3((unsigned)nslices), dim3(256), 0, stream, a, sbits, spart, nslices);
    else
        hipLaunchKernelGGL((cs2_kernel<false>), dim3((unsigned)nslices), dim3(256), 0, stream, a, sbits, spart, nslices);
    *err = hipGetLastError();
    return true;
}

// ---------------------------------------------------------------------------
// One or two rows (decode): one workgroup of 1024 threads holds all of x in
// registers and so sees the whole outlier set itself: detection, calibration,
// quantization and extraction in one launch, x read once.  Chunk f = tid +
// 1024 i of the flattened (row, 8-column chunk) range, L per thread.  (For
// more rows one workgroup's memory pipeline measured slower than the two
// kernels, which spread the rows over the CUs.)
constexpr int kSmallThreads = 1024;
// rows from which the quantizer reads x once (three launches) instead of twice
// (detection, then quantization: two launches)
constexpr int64_t kSingleReadMinRows = 1024;
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

namespace {

template <bool kVec, bool kBlockRow>
hipError_t launch_pass1(const QuantArgs& a, int64_t blocks, uint32_t* gbm, hipStream_t stream) {
    constexpr int P = kBlockRow ? 256 : 64;
    const int64_t per_lane = ceil_div(ceil_div(a.k, 8), P);
    const dim3 grid((unsigned)blocks), block(256);
    const size_t lds = (size_t)a.words * sizeof(uint32_t);
    if (per_lane <= 2)
        hipLaunchKernelGGL((quant1_kernel<kVec, kBlockRow, 2>), grid, block, lds, stream, a, gbm);
    else if (per_lane <= 4)
        hipLaunchKernelGGL((quant1_kernel<kVec, kBlockRow, 4>), grid, block, lds, stream, a, gbm);
    else if (per_lane <= 8)
        hipLaunchKernelGGL((quant1_kernel<kVec, kBlockRow, 8>), grid, block, lds, stream, a, gbm);
    else
        hipLaunchKernelGGL((quant1_kernel<kVec, kBlockRow, 16>), grid, block, lds, stream, a, gbm);
    return hipGetLastError();
}

// threshold > 0: zero the partial bitmaps (scratch), the single read of x,
// then the pass over the outlier set
hipError_t launch_single_read(const QuantArgs& in, hipStream_t stream) {
    QuantArgs a = in;
    uint32_t* gbm = a.partial;   // kMaxRowBlocks x words
    const int64_t pwords = kMaxRowBlocks * a.words;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(pwords > 8192 ? 16 : 1)), dim3(256), 0, stream, gbm,
                       pwords);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const bool vec = vector_rows(a) && ((a.ldq & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.q) & 7) == 0);
    const int64_t cpr = (a.k + 7) / 8;
    const bool block_row = cpr > 512 || (cpr >= 256 && a.m <= 512);
    int64_t blocks;
    if (block_row) {
        a.rows_per_block = ceil_div(a.m, 1024);
        blocks = ceil_div(a.m, a.rows_per_block);
    } else {
        a.rows_per_block = 4 * ceil_div(a.m, 4 * 512);
        blocks = ceil_div(a.m, a.rows_per_block);
    }
    hipError_t e = vec ? (block_row ? launch_pass1<true, true>(a, blocks, gbm, stream)
                                    : launch_pass1<true, false>(a, blocks, gbm, stream))
                       : (block_row ? launch_pass1<false, true>(a, blocks, gbm, stream)
                                    : launch_pass1<false, false>(a, blocks, gbm, stream));
    if (e != hipSuccess) return e;
    // a wave per row, up to 512 workgroups
    QuantArgs b = in;
    b.rows_per_block = 4 * ceil_div(a.m, 4 * 512);
    const int64_t blocks2 = ceil_div(a.m, b.rows_per_block);
    const size_t lds2 = ((size_t)a.words * 2 + kQ2Cols) * sizeof(uint32_t);
    if (vec)
        hipLaunchKernelGGL((quant2_kernel<true>), dim3((unsigned)blocks2), dim3(256), lds2, stream, b, gbm);
    else
        hipLaunchKernelGGL((quant2_kernel<false>), dim3((unsigned)blocks2), dim3(256), lds2, stream, b, gbm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& in, hipStream_t stream) {
    QuantArgs a = in;
    const bool vec = vector_rows(a);
    a.bitmap_in = nullptr;
    const int64_t per_thread = ceil_div(a.m * ceil_div(a.k, 8), kSmallThreads);
    if (a.m > 0 && a.m <= kSmallMaxRows && per_thread <= kSmallMaxL) {
        const size_t lds = ((size_t)a.words * 2 + (size_t)a.m * 2) * sizeof(uint32_t);
        return vec ? launch_small<true>(a, per_thread, lds, stream) : launch_small<false>(a, per_thread, lds, stream);
    }
    if (a.threshold > 0.0f && a.m >= kSingleReadMinRows && a.q) return launch_single_read(a, stream);
    if (a.threshold > 0.0f && a.m > kSmallMaxRows && a.m <= kCsRows) {
        hipError_t e;
        if (launch_col_slices(a, stream, &e)) return e;
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

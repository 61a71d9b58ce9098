// Decode-shaped int8 GEMM (m <= 16 activation rows) for gfx950.
//
// With a handful of tokens the linear is a stream of the int8 weight through
// HBM (the GEMV regime of generation): every weight byte is used m times, so
// the kernel is built to keep HBM busy, not the matrix cores.
//
//  * A group of 16 weight rows (the N side of v_mfma_i32_16x16x64_i8, whose
//    other side holds the m <= 16 activation rows with no padding) is shared
//    by G waves that split K: wave part p takes the 128-byte K chunks p, p+G,
//    p+2G, ...  A workgroup of 4 waves holds 4/G groups; G is chosen so that
//    each wave streams a long run of chunks and the grid fits the CUs in one
//    round.
//  * Each wave streams its weight chunks through a private ring of kStages
//    LDS stages with buffer_load ... lds (16 bytes per lane, whole 128-byte
//    lines, 2 KB per stage).  The matching activation fragments (m <= 16 rows,
//    L2-resident) go to a ring of registers.  The rings are private, so a
//    wave only waits for its own loads (s_waitcnt vmcnt), never for a
//    barrier; kStages - 1 chunks stay in flight.
//  * The G partial 16x16 int32 blocks of a group are summed through LDS and
//    the group's first wave runs the fused epilogue: row / column absmax, the
//    fp16 outlier-column sub-matmul on v_mfma_f32_16x16x32_f16, bias, fp16
//    output.
//
// Requests past the last chunk go through a zero-length buffer range (they
// fetch nothing), which keeps every vmcnt wait a constant.
#include "common.h"

namespace i8mp {

namespace {

constexpr int kRows = 16;     // weight rows per group
constexpr int kWaves = 4;     // waves per workgroup
constexpr int kStages = 8;    // per-wave ring depth
constexpr int kChunk = 128;   // K bytes per stage
constexpr int kStageBytes = kRows * kChunk;  // weight rows only
constexpr int kRsrcWord3 = 0x00020000;

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

__device__ inline float h2f(half_bits h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ inline half_bits f2h(float f) { return __builtin_bit_cast(half_bits, (_Float16)f); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    if (bytes < 0) bytes = 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

__device__ inline void dma16(__amdgpu_buffer_rsrc_t src, int8_t* lds, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, voffset,
                                             soffset, 0, 0);
}

// 128-byte LDS rows; lanes 0-15 of a fragment read rows 0-15 at one 16-byte
// chunk, so the chunk is XOR-ed with (row >> 1) & 7 to spread them over all
// sixteen 16-byte bank groups.
__device__ inline int swz(int row, int chunk) { return row * kChunk + ((chunk ^ ((row >> 1) & 7)) << 4); }

}  // namespace

template <int G, bool kFused>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs g) {
    // one LDS array (a second __shared__ object makes the compiler drain every
    // DMA before each LDS read): the rings, then the partial-sum blocks
    __shared__ __attribute__((aligned(1024))) int8_t ring[kWaves * kStages * kStageBytes + kWaves * 4 * 64 * 4];
    int32_t* red = reinterpret_cast<int32_t*>(ring + kWaves * kStages * kStageBytes);

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wid % G;                 // this wave's share of K
    const int64_t n0 = ((int64_t)blockIdx.x * (kWaves / G) + wid / G) * kRows;
    const bool active = n0 < g.n;

    const int64_t kr = (g.k + kChunk - 1) / kChunk * kChunk;
    // the weight's range ends at the last row's k rounded up to a dword (the
    // range check is per dword); the activations are zero-padded to kr
    const __amdgpu_buffer_rsrc_t rw = rsrc(g.b + n0 * g.ldb, (g.n - n0 - 1) * g.ldb + ((g.k + 3) & ~(int64_t)3));
    const __amdgpu_buffer_rsrc_t rx = rsrc(g.a, (g.m - 1) * g.lda + kr);
    const __amdgpu_buffer_rsrc_t r_none = rsrc(g.a, 0);

    // DMA lane mapping: instruction j covers weight rows 8j .. 8j+7 (1 KB);
    // lane i -> row 8j + i/8, LDS slot i%8, which holds global chunk
    // slot ^ ((row>>1)&7).  Activation fragment of lane l: row l%16, the 32
    // bytes at (l/16)*32 of the chunk (two 16-byte loads, one per MFMA).
    int w_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 8 * j + (lane >> 3);
        const int gchunk = (lane & 7) ^ ((row >> 1) & 7);
        w_off[j] = (int)(row * g.ldb + gchunk * 16);
    }
    const int x_off = (int)((lane & 15) * g.lda + (lane >> 4) * 32);
    int8_t* my_ring = ring + wid * kStages * kStageBytes;
    const int64_t nchunks = kr / kChunk;
    const int64_t mine = (active && nchunks > part) ? (nchunks - part + G - 1) / G : 0;
    v4i_t xr[kStages][2];
    // every chunk issues 4 loads (2 weight DMA, 2 activation); past this
    // wave's last chunk they read nothing (zero-length range)
    auto issue = [&](int64_t j, int slot) {
        const bool real = j < mine;
        const int kb = (int)((part + j * G) * kChunk);
        int8_t* st = my_ring + slot * kStageBytes;
        const __amdgpu_buffer_rsrc_t sw = real ? rw : r_none;
        const __amdgpu_buffer_rsrc_t sx = real ? rx : r_none;
        dma16(sw, st, w_off[0] + kb, 0);
        dma16(sw, st + 1024, w_off[1] + kb, 0);
        xr[slot][0] = __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(sx, x_off + kb, 0, 0));
        xr[slot][1] = __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(sx, x_off + 16 + kb, 0, 0));
    };

    v4i_t acc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j) issue(j, j);
    const int row = lane & 15;
    for (int64_t j0 = 0; j0 < mine; j0 += kStages) {
#pragma unroll
        for (int u = 0; u < kStages; ++u) {
            // chunk j0+u landed once only the kStages-2 later chunks (4 loads each) remain
            __builtin_amdgcn_s_waitcnt(0x0f70 | (((kStages - 2) * 4) & 15) | ((((kStages - 2) * 4) >> 4) << 14));
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const int8_t* st = my_ring + u * kStageBytes;
            v4i_t wf[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) wf[t] = *reinterpret_cast<const v4i_t*>(st + swz(row, (lane >> 4) * 2 + t));
            const v4i_t x0 = xr[u][0], x1 = xr[u][1];
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            issue(j0 + u + kStages - 1, (u + kStages - 1) % kStages);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(x0, wf[0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1, wf[1], acc, 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // no DMA left in flight into the ring

    // sum each group's partial blocks
    if (part > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(wid * 4 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (part > 0 || !active) return;  // no barrier below
#pragma unroll
    for (int w = 1; w < G; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += red[((wid + w) * 4 + r) * 64 + lane];

    // acc[r] of lane l: activation row 4*(l/16) + r, weight row n0 + l%16
    const int64_t col = n0 + (lane & 15);
    const int64_t row0 = 4 * (lane >> 4);
    if constexpr (!kFused) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (row0 + r < g.m && col < g.n) g.c[(row0 + r) * g.ldc + col] = acc[r];
    } else {
        const float r127 = 1.0f / 127.0f;
        int cnt = 0;
        if (g.x_out) {
            cnt = *g.count;
            if (cnt > g.cap) cnt = g.cap;
        }
        v4f_t p = {0.0f, 0.0f, 0.0f, 0.0f};
        int64_t arow = lane & 15;
        if (arow >= g.m) arow = g.m - 1;
        const int64_t bcol = col < g.n ? col : g.n - 1;
        for (int s0 = 0; s0 < cnt; s0 += 32) {
            const int s1 = s0 + (lane >> 4) * 8;
            const v8h xa = *reinterpret_cast<const v8h*>(g.x_out + arow * g.ldo + s1);
            v8h wb;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                wb[e] = s1 + e < cnt ? (_Float16)(float)g.b[bcol * g.ldb + g.idx[s1 + e]] : (_Float16)0.0f;
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, wb, p, 0, 0, 0);
        }
        if (col < g.n) {
            const float sw = g.col_absmax[col] * r127;
            const float bj = g.bias ? h2f(g.bias[col]) : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = row0 + r;
                if (row < g.m) {
                    const float sx = g.row_absmax[row] * r127;
                    g.out[row * g.ldout + col] = f2h(sw * ((float)acc[r] * sx + p[r]) + bj);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// m <= 4 (and m x K fits 32 KB): a dot-product GEMV on the vector ALUs.
// With one to four activation rows the matrix cores would idle over zero
// padding, and the MFMA kernel above spends as many load instructions on the
// activations as on the weights.  Here the int8 activations are copied to LDS
// once per workgroup, and the weight streams straight into registers: each
// wave owns 8 weight rows and a share of the 128-byte K chunks (chunks p,
// p + G, ...), one 1 KB load per chunk (lane i: row i / 8, bytes 16 (i % 8)
// of the chunk), kGvBatch loads in flight.  v_dot4_i32_i8 against the LDS
// activation bytes (lanes with equal i % 8 read the same 16 bytes: a
// broadcast) accumulates exactly in int32.  The outlier sub-matmul is taken
// from the streamed weight bytes as they pass: a chunk that contains an
// outlier column adds W[n, j] * x[r, j] (fp16 x, fp32 sum) for the lanes that
// hold that byte, so no weight byte is read twice.  Sums meet across the 8
// lanes of a row (shuffles) and the G waves of a row group (LDS).
namespace {

constexpr int kGvRows = 8;     // weight rows per wave
constexpr int kGvBatch = 8;    // weight loads in flight per wave
constexpr int kGvOutl = 64;    // outlier columns handled in the stream (more: gathered at the end)

__device__ inline int8_t byte_of(const v4i_t& v, int b) {
    return (int8_t)(((uint32_t)v[b >> 2] >> (8 * (b & 3))) & 0xffu);
}

}  // namespace

template <int G, int M, bool kFused>
__global__ __launch_bounds__(256) void gemv_kernel(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) int8_t gsm[];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wid % G;
    const int64_t n0 = ((int64_t)blockIdx.x * (4 / G) + wid / G) * kGvRows;
    const int64_t kr = (g.k + kChunk - 1) / kChunk * kChunk;
    const int64_t nchunks = kr / kChunk;
    const int64_t mine = nchunks > part ? (nchunks - part + G - 1) / G : 0;

    // LDS: activations [M][kr] | int32 partials [4][M][8] | fp32 partials [4][M][8] |
    //      outlier columns [kGvOutl] | outlier values [M][kGvOutl]
    int8_t* xs = gsm;
    int32_t* red = reinterpret_cast<int32_t*>(gsm + M * kr);
    float* pred = reinterpret_cast<float*>(red + 4 * M * kGvRows);
    int32_t* oidx = reinterpret_cast<int32_t*>(pred + 4 * M * kGvRows);
    float* oval = reinterpret_cast<float*>(oidx + kGvOutl);

    // 1. the first batch of weight loads goes out first
    const __amdgpu_buffer_rsrc_t rw =
        rsrc(g.b + n0 * g.ldb, n0 < g.n ? (g.n - n0 - 1) * g.ldb + ((g.k + 3) & ~(int64_t)3) : 0);
    const int w_off = (int)((lane >> 3) * g.ldb + (lane & 7) * 16);
    v4i_t w[kGvBatch];
    auto load_batch = [&](int64_t j0) {
#pragma unroll
        for (int u = 0; u < kGvBatch; ++u) {
            const int64_t j = j0 + u;
            const int kb = (int)((part + j * G) * kChunk);
            // the K offset goes in the range-checked VGPR offset: bytes past
            // the end of the weight read as 0
            w[u] = j < mine ? __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(rw, w_off + kb, 0, 0))
                            : v4i_t{0, 0, 0, 0};
        }
    };
    load_batch(0);

    // 2. activations (rows >= m as zeros), and the outlier columns / values
    {
        const __amdgpu_buffer_rsrc_t rx = rsrc(g.a, (g.m - 1) * g.lda + kr);
        const int64_t per_row = kr / 16;
        for (int64_t f = threadIdx.x; f < M * per_row; f += 256) {
            const int64_t r = f / per_row, c = f - r * per_row;
            v4i_t v = {0, 0, 0, 0};
            if (r < g.m)
                v = __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(r * g.lda + c * 16), 0, 0));
            *reinterpret_cast<v4i_t*>(xs + r * kr + c * 16) = v;
        }
    }
    int cnt = 0;
    if (kFused && g.x_out) {
        cnt = *g.count;
        cnt = cnt > g.cap ? g.cap : (cnt < 0 ? 0 : cnt);
        const int lc = cnt < kGvOutl ? cnt : kGvOutl;
        for (int t = threadIdx.x; t < kGvOutl; t += 256) oidx[t] = t < lc ? g.idx[t] : 0x7fffffff;
        for (int t = threadIdx.x; t < M * kGvOutl; t += 256) {
            const int r = t / kGvOutl, s2 = t % kGvOutl;
            oval[t] = (s2 < lc && r < g.m) ? h2f(g.x_out[r * g.ldo + s2]) : 0.0f;
        }
    }
    __syncthreads();
    const int lc = cnt < kGvOutl ? cnt : kGvOutl;

    // 3. stream: dot4 per 4 weight bytes, outliers from the bytes in flight
    int32_t acc[M];
    float pacc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        acc[r] = 0;
        pacc[r] = 0.0f;
    }
    const int slice = (lane & 7) * 16;  // this lane's 16 bytes of each chunk
    int next = 0;                        // first outlier column not yet behind the stream
    for (int64_t j0 = 0; j0 < mine; j0 += kGvBatch) {
        if (j0 > 0) load_batch(j0);
#pragma unroll
        for (int u = 0; u < kGvBatch; ++u) {
            const int64_t j = j0 + u;
            if (j >= mine) break;
            const int64_t kb = (part + j * G) * kChunk;
#pragma unroll
            for (int r = 0; r < M; ++r) {
                const v4i_t xv = *reinterpret_cast<const v4i_t*>(xs + r * kr + kb + slice);
#pragma unroll
                for (int d = 0; d < 4; ++d) acc[r] = __builtin_amdgcn_sdot4(w[u][d], xv[d], acc[r], false);
            }
            if (kFused) {
                while (next < lc && oidx[next] < kb) ++next;  // columns in other waves' chunks
                for (int s2 = next; s2 < lc && oidx[s2] < kb + kChunk; ++s2) {
                    const int off = oidx[s2] - (int)kb - slice;  // byte of this lane's slice, if any
                    if (off >= 0 && off < 16) {
                        const float wv = (float)byte_of(w[u], off);
#pragma unroll
                        for (int r = 0; r < M; ++r) pacc[r] += wv * oval[r * kGvOutl + s2];
                    }
                }
            }
        }
    }

    // 4. sums over the 8 lanes of a row, then over the G waves of the group
#pragma unroll
    for (int r = 0; r < M; ++r) {
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
            acc[r] += __shfl_xor(acc[r], off, 64);
            if (kFused) pacc[r] += __shfl_xor(pacc[r], off, 64);
        }
    }
    const int row = lane >> 3;
    if (part > 0 && (lane & 7) == 0) {
#pragma unroll
        for (int r = 0; r < M; ++r) {
            red[(wid * M + r) * kGvRows + row] = acc[r];
            if (kFused) pred[(wid * M + r) * kGvRows + row] = pacc[r];
        }
    }
    __syncthreads();
    if (part > 0 || (lane & 7) != 0) return;  // no barrier below
#pragma unroll
    for (int w2 = 1; w2 < G; ++w2)
#pragma unroll
        for (int r = 0; r < M; ++r) {
            acc[r] += red[((wid + w2) * M + r) * kGvRows + row];
            if (kFused) pacc[r] += pred[((wid + w2) * M + r) * kGvRows + row];
        }

    // 5. epilogue: lane 8 q owns weight row n0 + q
    const int64_t n = n0 + row;
    if (n >= g.n) return;
    if constexpr (!kFused) {
#pragma unroll
        for (int r = 0; r < M; ++r)
            if (r < g.m) g.c[r * g.ldc + n] = acc[r];
    } else {
        // outlier columns past the streamed ones: gathered
        for (int s2 = lc; s2 < cnt; ++s2) {
            const float wv = (float)g.b[n * g.ldb + g.idx[s2]];
#pragma unroll
            for (int r = 0; r < M; ++r)
                if (r < g.m) pacc[r] += wv * h2f(g.x_out[r * g.ldo + s2]);
        }
        const float r127 = 1.0f / 127.0f;
        const float sw = g.col_absmax[n] * r127;
        const float bj = g.bias ? h2f(g.bias[n]) : 0.0f;
#pragma unroll
        for (int r = 0; r < M; ++r)
            if (r < g.m) {
                const float sx = g.row_absmax[r] * r127;
                g.out[r * g.ldout + n] = f2h(sw * ((float)acc[r] * sx + pacc[r]) + bj);
            }
    }
}

// m <= 4 with the activations in at most 32 KB of LDS
bool gemv_fits(const GemmArgs& g) {
    const int64_t kr = (g.k + kChunk - 1) / kChunk * kChunk;
    // at most 32 KB: four workgroups per CU by LDS (a larger block measured slower
    // than the MFMA kernel: too few workgroups resident)
    return g.m >= 1 && g.m <= 4 && (g.m > 2 ? 4 : g.m) * kr <= 32 * 1024;
}

template <int M, bool kFused>
hipError_t launch_gemv_m(const GemmArgs& g, hipStream_t stream) {
    const int64_t kr = (g.k + kChunk - 1) / kChunk * kChunk;
    const int64_t nchunks = kr / kChunk;
    const int64_t groups = (g.n + kGvRows - 1) / kGvRows;
    // K splits: about 2500 waves or more, each with at least 8 chunks
    int gs = 1;
    while (gs < 4 && groups * gs < 2560 && nchunks / (2 * gs) >= kGvBatch) gs *= 2;
    const size_t lds = (size_t)M * kr + (size_t)4 * M * kGvRows * 8 + (size_t)kGvOutl * 4 + (size_t)M * kGvOutl * 4;
    const dim3 grid((unsigned)((groups * gs + 3) / 4));
    switch (gs) {
        case 1: hipLaunchKernelGGL((gemv_kernel<1, M, kFused>), grid, dim3(256), lds, stream, g); break;
        case 2: hipLaunchKernelGGL((gemv_kernel<2, M, kFused>), grid, dim3(256), lds, stream, g); break;
        default: hipLaunchKernelGGL((gemv_kernel<4, M, kFused>), grid, dim3(256), lds, stream, g); break;
    }
    return hipGetLastError();
}

template <bool kFused>
hipError_t launch_gemv(const GemmArgs& g, hipStream_t stream) {
    if (g.m == 1) return launch_gemv_m<1, kFused>(g, stream);
    if (g.m == 2) return launch_gemv_m<2, kFused>(g, stream);
    return launch_gemv_m<4, kFused>(g, stream);
}

hipError_t launch_decode(const GemmArgs& g, bool fused, hipStream_t stream) {
    if (gemv_fits(g)) return fused ? launch_gemv<true>(g, stream) : launch_gemv<false>(g, stream);
    // waves per 16-row group: enough K splits that each wave has a long run of
    // 128-byte chunks, with all groups resident at once (two workgroups per CU)
    const int64_t groups = (g.n + kRows - 1) / kRows;
    const int64_t nchunks = (g.k + kChunk - 1) / kChunk;
    int gsplit = 1;
    while (gsplit < kWaves && nchunks / (2 * gsplit) >= 16) gsplit *= 2;
    while (gsplit > 1 && groups * gsplit / kWaves > 2 * 256 && nchunks / gsplit < 32) gsplit /= 2;
    dim3 grid((unsigned)((groups * gsplit + kWaves - 1) / kWaves));
    switch (gsplit * 2 + (fused ? 1 : 0)) {
        case 2: hipLaunchKernelGGL((gemm_decode_kernel<1, false>), grid, dim3(256), 0, stream, g); break;
        case 3: hipLaunchKernelGGL((gemm_decode_kernel<1, true>), grid, dim3(256), 0, stream, g); break;
        case 4: hipLaunchKernelGGL((gemm_decode_kernel<2, false>), grid, dim3(256), 0, stream, g); break;
        case 5: hipLaunchKernelGGL((gemm_decode_kernel<2, true>), grid, dim3(256), 0, stream, g); break;
        case 8: hipLaunchKernelGGL((gemm_decode_kernel<4, false>), grid, dim3(256), 0, stream, g); break;
        default: hipLaunchKernelGGL((gemm_decode_kernel<4, true>), grid, dim3(256), 0, stream, g); break;
    }
    return hipGetLastError();
}

}  // namespace i8mp

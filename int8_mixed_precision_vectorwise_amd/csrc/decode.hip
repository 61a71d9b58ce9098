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
    const __amdgpu_buffer_rsrc_t rw = rsrc(g.b + n0 * g.ldb, (g.n - n0 - 1) * g.ldb + kr);
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
        dma16(sw, st, w_off[0], kb);
        dma16(sw, st + 1024, w_off[1], kb);
        xr[slot][0] = __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(sx, x_off, kb, 0));
        xr[slot][1] = __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(sx, x_off + 16, kb, 0));
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

hipError_t launch_decode(const GemmArgs& g, bool fused, hipStream_t stream) {
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

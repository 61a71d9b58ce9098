// int8 x int8 -> int32 GEMM on gfx950 matrix cores, with the dequantization
// epilogue of the mixed-precision linear fused in.
//
// C = A . B^T with A int8 [m x k] (activation codes) and B int8 [n x k] (weight
// codes), both K-contiguous row-major (bitsandbytes PR "LLM.int8()
// Refactoring: Part 1": int8_linear_matmul on row-major data).  The fused
// epilogue applies the row and column absmax, adds the fp16 outlier-column
// sub-matmul (sparse decomposition) on the fp16 matrix cores, adds the bias and
// writes fp16 (int8_mm_dequant of the same PR).
//
// Design (CDNA4): 256 threads = 4 wave64 in a 2 x 2 grid; each wave owns a
// (BM/2) x (BN/2) block of 32x32 accumulators fed by v_mfma_i32_32x32x32_i8.
// K advances in 128-byte tiles staged through LDS, double-buffered, loaded
// with 16-byte global loads into registers one tile ahead.  LDS rows are
// 128 bytes with the 16-byte chunk index XOR-swizzled by (row & 7), so the
// 16-byte fragment reads of 8 consecutive lanes hit distinct banks.  The
// contraction order inside an MFMA does not matter: A and B fragments use the
// same lane -> k mapping, and integer sums are exact in any order.
#include "common.h"

namespace i8mp {

namespace {

constexpr int BK = 128;
constexpr int kGroupM = 8;

__device__ inline float h2f(half_bits h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ inline half_bits f2h(float f) {
    return __builtin_bit_cast(half_bits, (_Float16)f);
}

// 16 bytes of row `row` at byte offset `col` (k-relative), zero past k.
template <bool kAligned>
__device__ inline v4i load16(const int8_t* __restrict__ base, int64_t ld, int64_t row, int64_t nrows,
                             int64_t col, int64_t k) {
    v4i r = {0, 0, 0, 0};
    if (row >= nrows || col >= k) return r;
    const int8_t* p = base + row * ld + col;
    if (kAligned && col + 16 <= k) return *reinterpret_cast<const v4i*>(p);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 16; ++e)
        if (col + e < k) w[e >> 2] |= ((uint32_t)(uint8_t)p[e]) << (8 * (e & 3));
    r[0] = (int)w[0];
    r[1] = (int)w[1];
    r[2] = (int)w[2];
    r[3] = (int)w[3];
    return r;
}

__device__ inline int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

}  // namespace

template <int BM, int BN, bool kFused, bool kAligned>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int A_CH = BM * BK / 16 / 256;
    constexpr int B_CH = BN * BK / 16 / 256;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // grouped tile order: kGroupM tile rows walk the N tiles together
    const int64_t tiles_m = (g.m + BM - 1) / BM;
    const int64_t tiles_n = (g.n + BN - 1) / BN;
    const int64_t bid = blockIdx.x;
    const int64_t in_group = (int64_t)kGroupM * tiles_n;
    const int64_t group = bid / in_group;
    const int64_t first_m = group * kGroupM;
    int64_t gsize = tiles_m - first_m;
    if (gsize > kGroupM) gsize = kGroupM;
    const int64_t tm = first_m + (bid % in_group) % gsize;
    const int64_t tn = (bid % in_group) / gsize;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    v4i ra[A_CH], rb[B_CH];
    const int64_t ktiles = (g.k + BK - 1) / BK;

    auto gload = [&](int64_t kt) {
#pragma unroll
        for (int p = 0; p < A_CH; ++p) {
            const int id = p * 256 + tid;
            ra[p] = load16<kAligned>(g.a, g.lda, m0 + (id >> 3), g.m, kt * BK + (id & 7) * 16, g.k);
        }
#pragma unroll
        for (int p = 0; p < B_CH; ++p) {
            const int id = p * 256 + tid;
            rb[p] = load16<kAligned>(g.b, g.ldb, n0 + (id >> 3), g.n, kt * BK + (id & 7) * 16, g.k);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < A_CH; ++p) {
            const int id = p * 256 + tid;
            *reinterpret_cast<v4i*>(&As[buf][swz(id >> 3, id & 7)]) = ra[p];
        }
#pragma unroll
        for (int p = 0; p < B_CH; ++p) {
            const int id = p * 256 + tid;
            *reinterpret_cast<v4i*>(&Bs[buf][swz(id >> 3, id & 7)]) = rb[p];
        }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < ktiles) gload(kt + 1);
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            v4i af[FM], bf[FN];
            const int ch = 2 * s + (lane >> 5);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WM + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const v4i*>(&As[buf][swz(row, ch)]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * WN + j * 32 + (lane & 31);
                bf[j] = *reinterpret_cast<const v4i*>(&Bs[buf][swz(row, ch)]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < ktiles) sstore(buf ^ 1);
        __syncthreads();
    }

    // accumulator (i, j, r) of lane l holds row 8*(r/4) + 4*(l/32) + r%4 and
    // column l%32 of the 32x32 block (i, j)
    const int64_t wrow0 = m0 + wm * WM + 4 * (lane >> 5);
    const int64_t wcol0 = n0 + wn * WN + (lane & 31);

    if constexpr (!kFused) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t col = wcol0 + 32 * j;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = wrow0 + 32 * i + 8 * (r >> 2) + (r & 3);
                    if (row < g.m && col < g.n) g.c[row * g.ldc + col] = acc[i][j][r];
                }
            }
    } else {
        const float r127 = 1.0f / 127.0f;
        int cnt = 0;
        if (g.x_out) {
            cnt = *g.count;
            if (cnt > g.cap) cnt = g.cap;
        }
        const int nsteps = (cnt + 15) / 16;
        float swj[FN], bj[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t col = wcol0 + 32 * j;
            const bool ok = col < g.n;
            swj[j] = ok ? g.col_absmax[col] * r127 : 0.0f;
            bj[j] = (ok && g.bias) ? h2f(g.bias[col]) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            float sxr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = wrow0 + 32 * i + 8 * (r >> 2) + (r & 3);
                sxr[r] = row < g.m ? g.row_absmax[row] * r127 : 0.0f;
            }
            int64_t arow = m0 + wm * WM + i * 32 + (lane & 31);
            if (arow >= g.m) arow = g.m - 1;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                v16f p;
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = 0.0f;
                int64_t bcol = wcol0 + 32 * j;
                if (bcol >= g.n) bcol = g.n - 1;
                for (int st = 0; st < nsteps; ++st) {
                    const int s0 = st * 16 + (lane >> 5) * 8;
                    const v8h xa = *reinterpret_cast<const v8h*>(g.x_out + arow * g.ldo + s0);
                    v8h wb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int s = s0 + e;
                        wb[e] = s < cnt ? (_Float16)(float)g.b[bcol * g.ldb + g.idx[s]] : (_Float16)0.0f;
                    }
                    p = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa, wb, p, 0, 0, 0);
                }
                const int64_t col = wcol0 + 32 * j;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = wrow0 + 32 * i + 8 * (r >> 2) + (r & 3);
                    if (row < g.m && col < g.n) {
                        const float y = swj[j] * ((float)acc[i][j][r] * sxr[r] + p[r]) + bj[j];
                        g.out[row * g.ldout + col] = f2h(y);
                    }
                }
            }
        }
    }
}

template <bool kFused>
static hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    constexpr int BM = 256, BN = 256;
    const bool aligned = ((g.lda & 15) == 0) && ((g.ldb & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(g.a) & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(g.b) & 15) == 0);
    const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
    dim3 grid((unsigned)tiles);
    if (aligned)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, kFused, true>), grid, dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, kFused, false>), grid, dim3(256), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_gemm_i32(const GemmArgs& g, hipStream_t stream) { return launch_gemm<false>(g, stream); }
hipError_t launch_gemm_fused(const GemmArgs& g, hipStream_t stream) { return launch_gemm<true>(g, stream); }

}  // namespace i8mp

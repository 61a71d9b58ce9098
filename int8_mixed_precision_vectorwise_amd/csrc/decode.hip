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
//    round.  Where that would give some CUs more groups than others (257
//    to 1024 groups), a group is instead ceil(n / 256) or ceil(n / 512) rows,
//    held as NB = 2 blocks of 16 that share the activation fragments, one
//    workgroup per CU.
//  * Each wave streams its chunks through a private ring of kStages LDS
//    stages with buffer_load ... lds (16 bytes per lane, eight lanes per
//    whole 128-byte line): the weight rows' chunk (2 KB) and the matching
//    chunk of the m <= 16 activation rows (2 KB, L2-resident).  Loaded
//    straight into the MFMA fragment layout, the activations would put four
//    rows, four cache lines, under every four lanes; the L1 then spends about
//    four times the cycles of whole-line requests on them, and with two
//    workgroups on a CU that alone bounded the stream.  The ring is private,
//    so a wave only waits for its own loads (s_waitcnt vmcnt), never for a
//    barrier; kStages - 1 chunks stay in flight.  With m <= 8 the activation
//    rows 8-15 are zeros written once, so a chunk takes three DMA instead of
//    four.
//  * The G partial 16x16 int32 blocks of a group are summed through LDS and
//    the group's first wave runs the fused epilogue: row / column absmax, the
//    fp16 outlier-column sub-matmul on v_mfma_f32_16x16x32_f16, bias, fp16
//    output.
//
// Requests past the last chunk go through a zero-length buffer range (they
// fetch nothing), which keeps every vmcnt wait a constant.
#include "common.h"
#include "quant_util.h"

namespace i8mp {

namespace {

constexpr int kRows = 16;     // weight rows per group
constexpr int kWaves = 4;     // waves per workgroup
constexpr int kChunk = 128;   // K bytes per stage
constexpr int kHalfBytes = kRows * kChunk;       // one operand's chunk
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kDecOutl = 32;  // outlier columns the MFMA decode kernel takes from its ring

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));


__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    if (bytes < 0) bytes = 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16 bytes per lane global -> LDS; the weight is streamed once per call, so
// its loads carry the nt (non-temporal) cache policy, while the activations,
// read by every group, keep the default one
constexpr int kWeightPolicy = 2;
template <int kPolicy>
__device__ inline void dma16(__amdgpu_buffer_rsrc_t src, int8_t* lds, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, voffset,
                                             soffset, 0, kPolicy);
}

// 128-byte LDS rows; lanes 0-15 of a fragment read rows 0-15 at one 16-byte
// chunk, so the chunk is XOR-ed with (row >> 1) & 7 to spread them over all
// sixteen 16-byte bank groups.
__device__ inline int swz(int row, int chunk) { return row * kChunk + ((chunk ^ ((row >> 1) & 7)) << 4); }

}  // namespace

template <int G, bool kFused, bool kHalfA, int NB>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs g, int rg) {
    // per-wave ring depth: 16-row groups with at most 8 activation rows (one
    // activation DMA per chunk) measured faster with three stages than with
    // four (13B down m = 4: 17.5 -> 16.2 us), with 16 rows with four; groups
    // of two blocks (one workgroup per CU) with four rather than three, five
    // or six (13B down m = 8: 17.4 -> 16.0 us)
    constexpr int kStages = (kHalfA && NB == 1) ? 3 : 4;
    constexpr int kWBytes = NB * kRows * kChunk;      // the weight rows of a stage (NB blocks of 16)
    constexpr int kStBytes = kWBytes + kHalfBytes;    // then the 16 activation rows
    constexpr int kRingBytes = kStages * kStBytes;    // one wave's ring
    static_assert(2 * NB * 4 * 64 * 4 <= kRingBytes, "a wave's partial blocks fit its ring");
    // one LDS array (a second __shared__ object makes the compiler drain every
    // DMA before each LDS read): the rings, then the outlier values
    __shared__ __attribute__((aligned(1024))) int8_t
        ring[kWaves * kRingBytes + (kFused ? kRows * kDecOutl * 4 : 0)];
    float* xo = reinterpret_cast<float*>(ring + kWaves * kRingBytes);  // [16 activation rows][kDecOutl] (fused)

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int part = wid % G;                 // this wave's share of K
    // group: weight rows n0 .. n0 + rg - 1 (rg <= 16 NB), of which
    // rows_here exist
    const int64_t n0 = ((int64_t)blockIdx.x * (kWaves / G) + wid / G) * rg;
    const bool active = n0 < g.n;
    const int rows_here = active ? (int)(g.n - n0 < rg ? g.n - n0 : rg) : 0;

    const int64_t kr = (g.k + kChunk - 1) / kChunk * kChunk;
    // the weight's range ends at the last row's k rounded up to a dword (the
    // range check is per dword); the activations are zero-padded to kr
    const __amdgpu_buffer_rsrc_t rw = rsrc(g.b + n0 * g.ldb, (g.n - n0 - 1) * g.ldb + ((g.k + 3) & ~(int64_t)3));
    const __amdgpu_buffer_rsrc_t rx = rsrc(g.a, (g.m - 1) * g.lda + kr);
    const __amdgpu_buffer_rsrc_t r_none = rsrc(g.a, 0);

    // DMA lane mapping, the same for both operands: instruction j covers rows
    // 8j .. 8j+7 (1 KB); lane i -> row 8j + i/8, LDS slot i%8, which holds
    // global chunk slot ^ ((row>>1)&7).  Weight rows past the group's (the
    // next group's, or past n) and activation rows past m read nothing.
    int w_off[2 * NB], a_off[2];
    bool w_ok[2 * NB];
#pragma unroll
    for (int j = 0; j < 2 * NB; ++j) {
        const int row = 8 * j + (lane >> 3);
        const int gchunk = (lane & 7) ^ ((row >> 1) & 7);
        w_off[j] = (int)(row * g.ldb + gchunk * 16);
        w_ok[j] = row < rows_here;
        if (j < 2) a_off[j] = (int)(row * g.lda + gchunk * 16);
    }
    int8_t* my_ring = ring + wid * kRingBytes;
    const int64_t nchunks = kr / kChunk;
    const int64_t mine = (active && nchunks > part) ? (nchunks - part + G - 1) / G : 0;
    // kHalfA (m <= 8): activation rows 8-15 are zeros, written into every
    // stage once here instead of by a DMA per chunk
    if constexpr (kHalfA) {
#pragma unroll
        for (int sl = 0; sl < kStages; ++sl)
            *reinterpret_cast<v4i_t*>(my_ring + sl * kStBytes + kWBytes + 1024 + lane * 16) = v4i_t{0, 0, 0, 0};
    }
    // every chunk issues kLoads loads (2 NB weight DMA, 2 or 1 activation
    // DMA); past this wave's last chunk they read nothing (zero-length range)
    constexpr int kLoads = 2 * NB + (kHalfA ? 1 : 2);
    auto issue = [&](int64_t j, int slot) {
        const bool real = j < mine;
        const int kb = (int)((part + j * G) * kChunk);
        int8_t* st = my_ring + slot * kStBytes;
        const __amdgpu_buffer_rsrc_t sw = real ? rw : r_none;
        const __amdgpu_buffer_rsrc_t sx = real ? rx : r_none;
#pragma unroll
        for (int jj = 0; jj < 2 * NB; ++jj)
            dma16<kWeightPolicy>(sw, st + jj * 1024, w_ok[jj] ? w_off[jj] + kb : (int)0x80000000, 0);
        dma16<0>(sx, st + kWBytes, a_off[0] + kb, 0);
        if constexpr (!kHalfA) dma16<0>(sx, st + kWBytes + 1024, a_off[1] + kb, 0);
    };

    v4i_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = v4i_t{0, 0, 0, 0};
    const int row = lane & 15;

    // The first kDecOutl outlier columns (ascending) are taken from the ring
    // as their chunk passes: lane l reads its weight rows' bytes (row l % 16
    // of each block) and adds byte * x into p, laid out like acc (activation
    // rows 4 (l / 16) + r).  ocol is the next such column (wave-uniform);
    // columns in other waves' chunks are passed over.  Later columns are
    // gathered in the epilogue.
    int cnt = 0, n_ring = 0, optr = 0;
    int64_t ocol = INT64_MAX;
    int ocol_lane = 0x7fffffff;  // lane s: column of slot s
    v4f_t p[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) p[b] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
    // The ring's outlier operands are loaded before the stream's first chunks
    // (vector loads complete in order, so waiting for them then does not wait
    // for the weight): the first index entries and X_O values, bounded by the
    // lengths of their arrays rather than by the count, which arrives with
    // them; slots past the count are dropped afterwards.  Unconditional
    // buffer loads (zeros out of range) keep the waits for them in one place.
    constexpr int kXoPer = kRows * kDecOutl / 256;
    int32_t cnt_raw = 0;
    uint32_t idx_raw = 0;
    uint16_t xo_raw[kXoPer];
    if constexpr (kFused) {
        const int lim = (g.count && g.cap > 0) ? (g.cap < kDecOutl ? g.cap : kDecOutl) : 0;
        // the range is X_O's whole extent, rounded up to a dword (the range
        // check is per dword)
        const __amdgpu_buffer_rsrc_t rxo = rsrc(g.x_out, lim > 0 ? (g.m * g.ldo * 2 + 3) & ~(int64_t)3 : 0);
#pragma unroll
        for (int i = 0; i < kXoPer; ++i) {
            const int t = threadIdx.x + 256 * i, r = t / kDecOutl, s2 = t % kDecOutl;
            // byte offsets < 2^31: at most 16 rows of a short X_O row
            const int off = (r < g.m && s2 < lim) ? (int)((r * g.ldo + s2) * 2) : (int)0x80000000;
            xo_raw[i] = __builtin_amdgcn_raw_buffer_load_b16(rxo, off, 0, 0);
        }
        const int ilim = g.count ? (g.idx_len < kDecOutl ? g.idx_len : kDecOutl) : 0;
        const __amdgpu_buffer_rsrc_t ridx = rsrc(g.idx, (int64_t)ilim * 4);
        idx_raw = __builtin_amdgcn_raw_buffer_load_b32(ridx, lane < ilim ? lane * 4 : (int)0x80000000, 0, 0);
        if (g.count) cnt_raw = *g.count;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int j = 0; j < kStages - 1; ++j) issue(j, j);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if constexpr (kFused) {
        if (g.count) cnt = outlier_count(g, cnt_raw);
        n_ring = cnt < kDecOutl ? cnt : kDecOutl;
#pragma unroll
        for (int i = 0; i < kXoPer; ++i) {
            const int t = threadIdx.x + 256 * i, r = t / kDecOutl, s2 = t % kDecOutl;
            xo[t] = (r < g.m && s2 < n_ring) ? (s2 < g.cap ? h2f(xo_raw[i]) : outlier_x(g, r, s2)) : 0.0f;
        }
        if (lane < n_ring) ocol_lane = (int)idx_raw;
        if (n_ring > 0) ocol = __builtin_amdgcn_readfirstlane(ocol_lane);
        // this wave's LDS writes done, then s_barrier; a memory fence would
        // also wait for the ring's DMA, which must stay in flight
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt unconstrained
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    const int arow0 = 4 * (lane >> 4);
    auto take_outliers = [&](int64_t chunk, const int8_t* st) {
        const int64_t c0 = chunk * kChunk;
        while (ocol < c0 + kChunk) {
            if (ocol >= c0) {
                const int cb = (int)(ocol - c0);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float wv = (float)st[swz(kRows * b + row, cb >> 4) + (cb & 15)];
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[b][r] += wv * xo[(arow0 + r) * kDecOutl + optr];
                }
            }
            ++optr;
            ocol = optr < n_ring ? (int64_t)__builtin_amdgcn_readlane(ocol_lane, optr) : INT64_MAX;
        }
    };

    for (int64_t j0 = 0; j0 < mine; j0 += kStages) {
#pragma unroll
        for (int u = 0; u < kStages; ++u) {
            // chunk j0+u landed once only the kStages-2 later chunks (kLoads each) remain
            __builtin_amdgcn_s_waitcnt(0x0f70 | (((kStages - 2) * kLoads) & 15) |
                                       ((((kStages - 2) * kLoads) >> 4) << 14));
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            const int8_t* st = my_ring + u * kStBytes;
            // fragments of lane l: row l % 16 (of each weight block), the 32
            // bytes at 32 (l / 16) of the chunk (one 16-byte piece per MFMA)
            v4i_t wf[NB][2], af[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[t] = *reinterpret_cast<const v4i_t*>(st + kWBytes + swz(row, (lane >> 4) * 2 + t));
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    wf[b][t] = *reinterpret_cast<const v4i_t*>(st + swz(kRows * b + row, (lane >> 4) * 2 + t));
            }
            if constexpr (kFused)
                if (j0 + u < mine) take_outliers(part + (j0 + u) * G, st);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            issue(j0 + u + kStages - 1, (u + kStages - 1) % kStages);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[0], wf[b][0], acc[b], 0, 0, 0);
                acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[1], wf[b][1], acc[b], 0, 0, 0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // no DMA left in flight into the ring

    // sum each group's partial blocks, through the rings (each wave writes
    // its own, whose DMA is done; the group's first wave reads after the
    // barrier)
    if (part > 0) {
        int32_t* red = reinterpret_cast<int32_t*>(my_ring);
        float* pred = reinterpret_cast<float*>(my_ring + NB * 4 * 64 * 4);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                red[(b * 4 + r) * 64 + lane] = acc[b][r];
                if (kFused) pred[(b * 4 + r) * 64 + lane] = p[b][r];
            }
    }
    __syncthreads();
    if (part > 0 || !active) return;  // no barrier below
#pragma unroll
    for (int w = 1; w < G; ++w) {
        const int32_t* red = reinterpret_cast<const int32_t*>(ring + (wid + w) * kRingBytes);
        const float* pred = reinterpret_cast<const float*>(ring + (wid + w) * kRingBytes + NB * 4 * 64 * 4);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[b][r] += red[(b * 4 + r) * 64 + lane];
                if (kFused) p[b][r] += pred[(b * 4 + r) * 64 + lane];
            }
    }

    // acc[b][r] of lane l: activation row 4*(l/16) + r, weight row n0 + 16 b + l%16
    const int64_t row0 = 4 * (lane >> 4);
    if constexpr (!kFused) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int lr = kRows * b + (lane & 15);
            const int64_t col = n0 + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (row0 + r < g.m && lr < rows_here) g.c[(row0 + r) * g.ldc + col] = acc[b][r];
        }
    } else {
        const float r127 = 1.0f / 127.0f;
        int64_t arow = lane & 15;
        if (arow >= g.m) arow = g.m - 1;
        // columns past the ring's kDecOutl: gathered (kDecOutl is a multiple of
        // 32); x values as 8-slot vectors from X_O below xo_lim (zero from the
        // count to ldo), past it slot by slot
        const int xo_lim = cnt <= g.cap ? (int)g.ldo : g.cap;
        for (int s0 = n_ring; s0 < cnt; s0 += 32) {
            const int s1 = s0 + (lane >> 4) * 8;
            v8h xa;
            if (s1 + 8 <= xo_lim) {
                xa = *reinterpret_cast<const v8h*>(g.x_out + arow * g.ldo + s1);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xa[e] = s1 + e < cnt ? (_Float16)outlier_x(g, arow, s1 + e) : (_Float16)0.0f;
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int lr = kRows * b + (lane & 15);
                const int64_t bcol = n0 + (lr < rows_here ? lr : 0);
                v8h wb;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    wb[e] = s1 + e < cnt ? (_Float16)(float)g.b[bcol * g.ldb + g.idx[s1 + e]] : (_Float16)0.0f;
                p[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, wb, p[b], 0, 0, 0);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int lr = kRows * b + (lane & 15);
            if (lr < rows_here) {
                const int64_t col = n0 + lr;
                const float sw = g.col_absmax[col] * r127;
                const float bj = g.bias ? h2f(g.bias[col]) : 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = row0 + r;
                    if (row < g.m) {
                        const float sx = g.row_absmax[row] * r127;
                        g.out[row * g.ldout + col] = f2h(sw * ((float)acc[b][r] * sx + p[b][r]) + bj);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// m <= 2: a dot-product GEMV on the vector ALUs.  With one or two activation
// rows the matrix cores would idle over zero padding.  (From three rows on
// the MFMA decode kernel above streams the weight faster: 13B up at m = 4
// took 20.4 us here and takes 16.1 us there.)  The int8 activations
// sit in LDS (rows of kx = K rounded up to 1 KB, zeros past K), and each wave
// reads R weight rows front to back, one row after the other: a load is one
// row's next 1 KB of K (lane i: bytes 16 i .. 16 i + 15).  Wave v of the nw
// waves takes rows v, v + nw, ..., so the grid reads one band of neighbouring
// rows at a time (plain reads of 70 MB measured fastest as one such sweep on
// MI355X, with about 2048 waves).  Batches of kGvBatch loads are
// double-buffered: the next batch is in flight while this one is used (the
// first goes out before the activations are staged).  The weight loads
// carry the nt cache policy (each byte is read once).  A row's bytes past K
// read through the row's own buffer range and come back as zeros, with no
// memory traffic.  v_dot4_i32_i8 against the LDS
// activation bytes accumulates exactly in int32; the outlier sub-matmul is
// taken from the streamed weight bytes as they pass (a lane holding byte j of
// an outlier column adds W[n, j] * x[r, j] in fp32), so no weight byte is read
// twice.  At the end of a row the 64 lanes' sums are added up (DPP) and lane
// 0 runs the fused epilogue.
//
// The whole forward in one launch (kQuantL > 0): every workgroup holds all
// of the one or two rows of x, so it runs the quantizer's steps itself and
// no grid-wide step separates them.  x sits in registers (kQuantL 8-column
// chunks per thread); chunk maxima come from packed fp16 maxima; a chunk
// reaching the threshold sets its outlier bits in an LDS bitmap; the row
// absmax over the non-outlier columns comes from wave maxima and an LDS
// atomicMax; the codes go straight into the LDS activation rows and the
// outlier values into the stream's list.  The codes are the quantization
// kernels' own, bit for bit (same helpers, same IEEE operations).  The
// intermediates (codes, absmax, bitmap, index list, count, gathered outlier
// values) are written to the workspace spread over the grid.
namespace {

constexpr int kGvChunk = 1024;   // K bytes per wave load
constexpr int kGvBatch = 8;      // loads per batch (two batches in flight)
constexpr int kGvOutl = 64;      // outlier columns handled in the stream (more: gathered per row)
constexpr int kGvWaves = 2048;   // waves the grid aims at
constexpr int kGvOwn = 2;        // outlier columns a lane keeps in registers

__device__ inline int8_t byte_of(const v4i_t& v, int b) {
    return (int8_t)(((uint32_t)v[b >> 2] >> (8 * (b & 3))) & 0xffu);
}

// LDS of the fused forward's quantizer state, after the stream's arrays
struct GvQuantLds {
    uint32_t* bm;        // [words] outlier bitmap
    int32_t* pre;        // [words] exclusive prefix of the word popcounts
    uint32_t* rmax;      // [M] row absmax (fp32 bits)
    int32_t* wave_tot;   // [waves]
    float* wmax;         // [waves][M] each wave's row maxima
};

// x as 8-column chunks, chunk-major: thread tid holds chunks c = tid + T q
// (q < L / M) with all M rows of each, v[q M + r] = x[r, c].  A chunk's
// outlier bits are then the OR over the thread's own rows, with no global
// view needed.  With k a multiple of 8 and 16-byte aligned rows every chunk
// is one 16-byte load; chunks past k and rows past m read zeros through the
// range check, so all L loads are in flight together.
template <int M, int L, int T>
__device__ inline void load_x_chunks(const QuantArgs& a, uint4 (&v)[L]) {
    static_assert(L % M == 0, "whole chunks of M rows");
    const int tid = threadIdx.x;
    const int32_t cpr = (int32_t)(a.k / 8);
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, ((int64_t)(a.m - 1) * a.ldx + a.k) * 2);
#pragma unroll
    for (int q = 0; q < L / M; ++q)
#pragma unroll
        for (int r = 0; r < M; ++r) {
            const int32_t c = tid + T * q;
            // byte offsets < 2^31: m <= 2 rows of at most I8MP_MAX_LD elements
            const int off = (c < cpr && r < a.m) ? (int)(((int64_t)r * a.ldx + (int64_t)c * 8) * 2) : (int)0x80000000;
            v[q * M + r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
}

// Quantize the chunks of load_x_chunks into the LDS activation rows xs
// [M][kr] (kr >= k, zeros past k and in rows past m); the first kGvOutl
// outlier columns and their values go to oidx / oval; the bitmap, its prefix
// and the row absmax to q.  Returns the outlier count.  Every thread calls;
// one workgroup barrier between the local pass and the codes, two inside the
// prefix.
template <int M, int L, int T>
__device__ inline int32_t quantize_rows_lds(const QuantArgs& a, const uint4 (&v)[L], int64_t kr, int8_t* xs,
                                            int32_t* oidx, float* oval, const GvQuantLds& q) {
    constexpr int NQ = L / M;
    constexpr int NW = T / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool outl = a.threshold > 0.0f;
    const int32_t cpr = (int32_t)(a.k / 8);  // k % 8 == 0

    // zero: the stream's outlier list, activation bytes past k and rows past m
    for (int t = tid; t < kGvOutl; t += T) oidx[t] = 0x7fffffff;
    for (int t = tid; t < M * kGvOutl; t += T) oval[t] = 0.0f;
    for (int64_t r = 0; r < a.m; ++r)
        for (int64_t col = a.k + tid; col < kr; col += T) xs[r * kr + col] = 0;
    for (int64_t u = tid; u < (M - a.m) * kr / 16; u += T)
        *reinterpret_cast<v4i_t*>(xs + a.m * kr + u * 16) = v4i_t{0, 0, 0, 0};

    // local pass: each chunk's outlier bits (OR over its rows), the rows'
    // maxima over the chunk's other columns, and the bitmap words: the four
    // chunks of a word sit in the four lanes of a quad (c % 4 == lane % 4)
    uint32_t obits[NQ];
    float tmax[M];
#pragma unroll
    for (int r = 0; r < M; ++r) tmax[r] = 0.0f;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
        float cm[M];
        uint32_t ob = 0;
#pragma unroll
        for (int r = 0; r < M; ++r) {
            cm[r] = chunk_absmax(v[qq * M + r]);
            if (outl && cm[r] >= a.threshold) ob |= outlier_bits8(v[qq * M + r], a.threshold);
        }
        obits[qq] = ob;
#pragma unroll
        for (int r = 0; r < M; ++r) tmax[r] = fmaxf(tmax[r], ob ? chunk_max(v[qq * M + r], ob) : cm[r]);
        const int32_t c = tid + T * qq;
        int32_t wv = (int32_t)(ob << (8 * (lane & 3)));
        wv |= dpp_i32<kDppQuadSwap1>(wv);
        wv |= dpp_i32<kDppQuadSwap2>(wv);
        if ((lane & 3) == 0 && (c >> 2) < a.words) q.bm[c >> 2] = (uint32_t)wv;
    }
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const float t = wave_max_uniform(tmax[r]);
        if (lane == 0) q.wmax[wave * M + r] = t;
    }
    __syncthreads();

    // row absmax from the waves' maxima; codes of the chunks into LDS
    float inv[M];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s = fmaxf(s, q.wmax[w * M + r]);
        inv[r] = s > 0.0f ? 127.0f / s : 0.0f;  // IEEE division
        if (tid == 0) q.rmax[r] = __float_as_uint(s);
    }
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
        const int32_t c = tid + T * qq;
        if (c >= cpr) continue;
#pragma unroll
        for (int r = 0; r < M; ++r) {
            const uint4& x8 = v[qq * M + r];
            uint2 code;
            if (obits[qq] == 0u) {
                code = codes8_plain(x8, inv[r]);
            } else {
                const bool zero_row = !(inv[r] > 0.0f);
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t b = code_byte(h2f(half_at(x8, e)), inv[r], zero_row || ((obits[qq] >> e) & 1u));
                    if (e < 4) lo |= b << (8 * e);
                    else hi |= b << (8 * (e - 4));
                }
                code = make_uint2(lo, hi);
            }
            *reinterpret_cast<uint2*>(xs + r * kr + (int64_t)c * 8) = code;
        }
    }
    const int32_t total = outl ? bitmap_prefix(q.bm, q.pre, a.words, q.wave_tot) : 0;
    // the first kGvOutl outlier columns and their values, in slot order
    const int32_t lc = total < kGvOutl ? total : kGvOutl;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
        const uint32_t ob = obits[qq];
        if (ob == 0u) continue;
        const int32_t c = tid + T * qq;
        const int32_t w = c >> 2;
        const uint32_t below = q.bm[w] & ((1u << (8 * (c & 3))) - 1u);   // bits of the word's earlier chunks
        int32_t slot = q.pre[w] + __popc(below);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((ob >> e) & 1u) {
                if (slot < lc) {
                    oidx[slot] = c * 8 + e;
#pragma unroll
                    for (int r = 0; r < M; ++r) oval[r * kGvOutl + slot] = h2f(half_at(v[qq * M + r], e));
                }
                ++slot;
            }
    }
    return total;
}

// The forward's intermediates into the workspace, spread over the grid (each
// thread writes at most a few entries): codes (the LDS rows, kpad == ldq),
// absmax, bitmap, count, index list (-1 past the count) and gathered outlier
// values (the first cap slots, zero past them).  The first kGvOutl slots come
// from the stream's LDS list (columns, and values as fp32 that convert back
// to the same fp16); later slots, if any, from the bitmap and x.  After the
// barrier that follows quantize_rows_lds.
template <int M, int T>
__device__ inline void publish_spread(const QuantArgs& a, int64_t kx, const int8_t* xs, const GvQuantLds& q,
                                      const int32_t* oidx, const float* oval, bool any, int32_t total) {
    const int32_t kept = total < a.cap ? total : a.cap;   // slots with gathered x values
    const int64_t gt = (int64_t)blockIdx.x * T + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * T;
    const int64_t units = a.ldq / 16;  // 16-byte units per code row (ldq <= kx, zeros past k)
    for (int64_t u = gt; u < a.m * units; u += stride) {
        const int64_t r = u / units, c = u - r * units;
        *reinterpret_cast<v4i_t*>(a.q + r * a.ldq + c * 16) = *reinterpret_cast<const v4i_t*>(xs + r * kx + c * 16);
    }
    if (gt < a.m) a.absmax[gt] = __uint_as_float(q.rmax[gt]);
    if (gt == 0 && a.count_out) *a.count_out = total;
    if (a.bitmap_out)
        for (int64_t w = gt; w < a.words; w += stride) a.bitmap_out[w] = any ? q.bm[w] : 0u;
    const int32_t lc = total < kGvOutl ? total : kGvOutl;
    if (a.idx_out)
        for (int64_t s = gt; s < a.idx_len; s += stride)
            if (s < lc) a.idx_out[s] = oidx[s];
            else if (s >= total) a.idx_out[s] = -1;
    if (a.x_out)
        for (int64_t f = gt; f < a.m * a.xo_cols; f += stride) {
            const int64_t r = f / a.xo_cols, s = f - r * a.xo_cols;
            if (s < lc && s < kept) a.x_out[r * a.ldo + s] = f2h(oval[r * kGvOutl + s]);
            else if (s >= kept) a.x_out[r * a.ldo + s] = 0;
        }
    if (total > kGvOutl)  // slots from kGvOutl on: walk the bitmap words
        for (int64_t w = gt; w < a.words; w += stride) {
            uint32_t bits = q.bm[w];
            int32_t slot = bits ? q.pre[w] : 0;
            while (bits) {
                const int64_t j = w * 32 + (__ffs(bits) - 1);
                bits &= bits - 1u;
                if (slot >= kGvOutl && slot < total) {
                    if (a.idx_out && slot < a.idx_len) a.idx_out[slot] = (int32_t)j;
                    if (a.x_out && slot < kept)
                        for (int64_t r = 0; r < a.m; ++r) a.x_out[r * a.ldo + slot] = a.x[r * a.ldx + j];
                }
                ++slot;
            }
        }
}

}  // namespace

// rows_per_wave weight rows per wave, W waves per workgroup.
template <int M, bool kFused, int kQuantL, int W>
__global__ __launch_bounds__(64 * W) void gemv_kernel(GemmArgs g, QuantArgs qa, int rows_per_wave) {
    constexpr bool kQuant = kQuantL > 0;
    static_assert(!kQuant || kFused, "the one-launch forward has the fused epilogue");
    extern __shared__ __attribute__((aligned(16))) int8_t gsm[];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t kx = (g.k + kGvChunk - 1) / kGvChunk * kGvChunk;
    const int nck = (int)(kx / kGvChunk);                         // 1 KB chunks per row
    const int bpr = (nck + kGvBatch - 1) / kGvBatch;              // batches per row
    const int R = rows_per_wave;
    // wave v of nw takes rows v, v + nw, v + 2 nw, ...: at any time the grid
    // reads one band of neighbouring rows
    const int64_t nw = (g.n + R - 1) / R;
    const int64_t wv = (int64_t)blockIdx.x * W + wid;
    auto row_of = [&](int rr) -> int64_t { return wv + (int64_t)rr * nw; };
    const int nb = R * bpr;                                       // batches of this wave

    // LDS: activations [M][kx] | outlier columns [kGvOutl] | outlier values [M][kGvOutl] |
    //      per-wave outlier slot tables [W][64 (1 + kGvOwn)] |
    //      (one-launch forward) bitmap [words] | prefix [words] | row absmax [M] |
    //      wave totals [W] | wave row maxima [W][M]
    int8_t* xs = gsm;
    int32_t* oidx = reinterpret_cast<int32_t*>(gsm + M * kx);
    float* oval = reinterpret_cast<float*>(oidx + kGvOutl);
    int32_t* own_lds = reinterpret_cast<int32_t*>(oval + M * kGvOutl);  // [W][64 * (1 + kOwn)]
    GvQuantLds ql;
    ql.bm = reinterpret_cast<uint32_t*>(own_lds + W * 64 * (1 + kGvOwn));
    ql.pre = reinterpret_cast<int32_t*>(ql.bm + qa.words);
    ql.rmax = reinterpret_cast<uint32_t*>(ql.pre + qa.words);
    ql.wave_tot = reinterpret_cast<int32_t*>(ql.rmax + M);
    ql.wmax = reinterpret_cast<float*>(ql.wave_tot + W);

    // weight loads: batch b covers row b / bpr, chunks from (b % bpr) * kGvBatch.
    // Past a row's K, past the wave's rows or past n: zero-length / range-checked
    // reads (nothing fetched, zeros returned); no branches, so every wait
    // counts all loads in flight.
    const int64_t row_bytes = (g.k + 3) & ~(int64_t)3;  // the range check is per dword
    const __amdgpu_buffer_rsrc_t r_none = rsrc(g.b, 0);
    auto issue = [&](int b, v4i_t (&wb)[kGvBatch]) {
        const int rr = b / bpr;
        const int c0 = (b - rr * bpr) * kGvBatch;
        const int64_t n = row_of(rr);
        const __amdgpu_buffer_rsrc_t rw = (b < nb && n < g.n) ? rsrc(g.b + n * g.ldb, row_bytes) : r_none;
#pragma unroll
        for (int u = 0; u < kGvBatch; ++u)
            wb[u] = __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rw, (c0 + u) * kGvChunk + lane * 16, 0, kWeightPolicy));
    };
    v4i_t w[2][kGvBatch];
    // Every small load goes out before the weight stream, so that the waits
    // of the prologue count only them (loads complete in order): x (one-launch
    // forward) or the codes and the outlier list (unfused), and the epilogue
    // operands of the wave's rows (lane i: the wave's row i).  Then the first
    // weight batch streams while the prologue runs (a second one in flight
    // there measured slower).
    constexpr int kXL = kQuant ? kQuantL : 1;
    uint4 xv[kXL];
    if constexpr (kQuant) load_x_chunks<M, kXL, 64 * W>(qa, xv);
    // unfused: the codes (M rows of kx bytes, at most 32 KB: 16-byte chunks f =
    // tid + 64 W i), the first kGvOutl outlier columns and their x values
    constexpr int kCL = kQuant ? 1 : (32 * 1024 / 16 + 64 * W - 1) / (64 * W);
    v4i_t cv[kCL];
    // (raw load results only: converting them here would wait for the load
    // before the weight batches go out)
    int32_t idx_t = 0x7fffffff;
    uint32_t oval_bits = 0;
    int cnt = 0;
    const int64_t per_row = kx / 16;
    if constexpr (!kQuant) {
        // the codes' rows hold zeros from k to a multiple of 128 (lda >= that)
        const int64_t kr = (g.k + kChunk - 1) / kChunk * kChunk;
        const __amdgpu_buffer_rsrc_t rx = rsrc(g.a, (g.m - 1) * g.lda + kr);
        const int pr = (int)per_row;   // <= 2048
        int r = (int)threadIdx.x / pr, c = (int)threadIdx.x - r * pr;
#pragma unroll
        for (int i = 0; i < kCL; ++i) {
            const int f = (int)threadIdx.x + 64 * W * i;
            const int off = (f < M * pr && r < g.m && (int64_t)c * 16 < kr) ? (int)(r * g.lda + c * 16) : (int)0x80000000;
            cv[i] = __builtin_bit_cast(v4i_t, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
            c += 64 * W;   // the next chunk of this thread: row and chunk without a division
            while (c >= pr) {
                c -= pr;
                ++r;
            }
        }
        if (kFused && g.count) {
            cnt = outlier_count(g, *g.count);
            // thread t < M kGvOutl: slot s2 = t % kGvOutl of row r = t / kGvOutl,
            // idx[s2] and, below cap, x_out[r, s2] (past the list, cap or m:
            // zeros through the range checks; masked by the count below)
            const int t = threadIdx.x;
            const __amdgpu_buffer_rsrc_t ri = rsrc(g.idx, (int64_t)g.idx_len * 4);
            const __amdgpu_buffer_rsrc_t ro = rsrc(g.x_out, g.x_out ? (int64_t)g.m * g.ldo * 2 : 0);
            const int r = t / kGvOutl, s2 = t % kGvOutl;
            idx_t = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, t < M * kGvOutl ? s2 * 4 : (int)0x80000000, 0, 0);
            oval_bits = __builtin_amdgcn_raw_buffer_load_b16(
                ro, t < M * kGvOutl && r < g.m && s2 < g.cap ? (int)((r * g.ldo + s2) * 2) : (int)0x80000000, 0, 0);
        }
    }
    const float r127 = 1.0f / 127.0f;
    uint32_t sw_bits = 0, bias_bits = 0;
    float sx_raw[M];   // unfused: the row absmax of x, read before the stream too
#pragma unroll
    for (int r = 0; r < M; ++r) sx_raw[r] = (kFused && !kQuant && r < g.m) ? g.row_absmax[r] : 0.0f;
    if constexpr (kFused) {
        const int64_t nl = row_of(lane);
        const bool own = lane < R && nl < g.n;
        const __amdgpu_buffer_rsrc_t rs = rsrc(g.col_absmax, g.n * 4);
        const __amdgpu_buffer_rsrc_t rb = rsrc(g.bias, g.bias ? g.n * 2 : 0);
        sw_bits = __builtin_amdgcn_raw_buffer_load_b32(rs, own ? (int)(nl * 4) : (int)0x80000000, 0, 0);
        bias_bits = __builtin_amdgcn_raw_buffer_load_b16(rb, own ? (int)(nl * 2) : (int)0x80000000, 0, 0);
    }
    issue(0, w[0]);
    // keeps the compiler from converting the x value right after its load
    // (a wait ahead of the weight batches)
    asm volatile("" : "+v"(oval_bits));
    const float sw_lane = __uint_as_float(sw_bits) * r127;
    const float bias_lane = h2f((half_bits)bias_bits);

    // activations (rows >= m and bytes past K as zeros), outlier columns / values
    if constexpr (kQuant) {
        const int32_t total = quantize_rows_lds<M, kQuantL, 64 * W>(qa, xv, kx, xs, oidx, oval, ql);
        cnt = total;   // every outlier column takes the fp16 path
        __syncthreads();
        publish_spread<M, 64 * W>(qa, kx, xs, ql, oidx, oval, total > 0, total);
    } else {
#pragma unroll
        for (int i = 0; i < kCL; ++i) {
            const int f = (int)threadIdx.x + 64 * W * i;
            if (f < M * (int)per_row) *reinterpret_cast<v4i_t*>(xs + f * 16) = cv[i];  // row f / per_row, chunk f % per_row
        }
        if (kFused && g.count) {
            const int lc0 = cnt < kGvOutl ? cnt : kGvOutl;
            const int t = threadIdx.x;
            if (t < kGvOutl) oidx[t] = t < lc0 ? idx_t : 0x7fffffff;
            if (t < M * kGvOutl) {
                const int r = t / kGvOutl, s2 = t % kGvOutl;
                float v = 0.0f;
                if (s2 < lc0)  // past X_O's capacity: from x through the index list
                    v = s2 < g.cap ? h2f((half_bits)oval_bits) : (r < g.m ? h2f(g.x[r * g.ldx + idx_t]) : 0.0f);
                oval[t] = v;
            }
        } else {
            for (int t = threadIdx.x; t < kGvOutl; t += 64 * W) oidx[t] = 0x7fffffff;
            for (int t = threadIdx.x; t < M * kGvOutl; t += 64 * W) oval[t] = 0.0f;
        }
    }
    __syncthreads();
    const int lc = cnt < kGvOutl ? cnt : kGvOutl;
    float sx[M];
    if constexpr (kFused) {
#pragma unroll
        for (int r = 0; r < M; ++r)
            sx[r] = r < g.m ? (kQuant ? __uint_as_float(ql.rmax[r]) : sx_raw[r]) * r127 : 0.0f;
    }
    // The streamed outlier columns: column j of a chunk sits in lane
    // (j % 1024) / 16, byte j % 16, of every row's load of chunk j / 1024.
    // Each lane takes up to kOwn of the columns it will hold (chunk, byte, x
    // values in registers), so that per chunk the owning lanes add their
    // terms together; a column past its lane's kOwn is walked one by one
    // (spill: a wave-uniform slot mask, empty unless three or more columns
    // share a lane).  Slot lane s finds its rank at its owner with an LDS
    // atomic on the wave's counters; the owner reads its entries back.
    // chunks_hit (uniform): bit c set if chunk c holds an outlier column.
    constexpr int kOwn = kGvOwn;
    int own_chunk[kOwn], own_byte[kOwn];
    float own_x[kOwn][M];
    uint64_t spill = 0;
    uint32_t chunks_hit = 0;
    const int ocol = lane < lc ? oidx[lane] : 0x7fffffff;  // lane s: column of slot s
    // the counters and slot tables are the wave's own: ordering its LDS
    // accesses is enough, no workgroup barrier
    auto wave_lds_sync = [] {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS accesses are done
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_wave_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    if constexpr (kFused) {
        int32_t* cnt_w = own_lds + wid * 64 * (1 + kOwn);   // [64] counters | [64][kOwn] slots
        int32_t* tab_w = cnt_w + 64;
        cnt_w[lane] = 0;
#pragma unroll
        for (int e = 0; e < kOwn; ++e) tab_w[lane * kOwn + e] = -1;
        wave_lds_sync();
        bool spilled = false;
        if (lane < lc) {
            const int owner = (ocol & (kGvChunk - 1)) >> 4;
            const int rank = atomicAdd(&cnt_w[owner], 1);
            if (rank < kOwn) tab_w[owner * kOwn + rank] = lane;
            else spilled = true;
        }
        spill = __ballot(spilled);
        uint32_t hit = lane < lc ? 1u << (ocol / kGvChunk) : 0u;  // chunks < 32 (k <= 32 KB)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) hit |= (uint32_t)__shfl_xor((int)hit, off, 64);
        chunks_hit = __builtin_amdgcn_readfirstlane(hit);
        wave_lds_sync();
#pragma unroll
        for (int e = 0; e < kOwn; ++e) {
            const int sl = tab_w[lane * kOwn + e];
            const int col = sl >= 0 ? oidx[sl] : 0;
            own_chunk[e] = sl >= 0 ? col / kGvChunk : -1;
            own_byte[e] = col & 15;
#pragma unroll
            for (int r = 0; r < M; ++r) own_x[e][r] = sl >= 0 ? oval[r * kGvOutl + sl] : 0.0f;
        }
    }
    float oxv[M];  // lane s: x values of slot s (for spilled columns)
#pragma unroll
    for (int r = 0; r < M; ++r) oxv[r] = oval[r * kGvOutl + lane];

    int32_t acc[M];
    float pacc[M];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        acc[r] = 0;
        pacc[r] = 0.0f;
    }

    // end of row rr: sums over the 64 lanes, epilogue in lane 0
    auto finish_row = [&](int rr) {
#pragma unroll
        for (int r = 0; r < M; ++r) {
            acc[r] = wave_sum_i32(acc[r]);
            if (kFused) pacc[r] = wave_sum_f32(pacc[r]);
        }
        const int64_t n = row_of(rr);
        float sw = 0.0f, bj = 0.0f;
        if constexpr (kFused) {
            sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sw_lane), rr));
            bj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bias_lane), rr));
        }
        if (lane == 0 && n < g.n) {
            if constexpr (!kFused) {
#pragma unroll
                for (int r = 0; r < M; ++r)
                    if (r < g.m) g.c[r * g.ldc + n] = acc[r];
            } else {
                // outlier columns past the streamed ones: gathered, in slot order
                if constexpr (kQuant) {
                    // slots from the LDS bitmap and its prefix, values from x
                    for (int64_t wd = 0; wd < qa.words && cnt > lc; ++wd) {
                        uint32_t bits = ql.bm[wd];
                        int32_t slot = ql.pre[wd];
                        if (slot >= cnt) break;
                        while (bits) {
                            const int64_t j = wd * 32 + (__ffs(bits) - 1);
                            bits &= bits - 1u;
                            if (slot >= lc && slot < cnt) {
                                const float wv = (float)g.b[n * g.ldb + j];
#pragma unroll
                                for (int r = 0; r < M; ++r)
                                    if (r < g.m) pacc[r] += wv * h2f(qa.x[r * qa.ldx + j]);
                            }
                            ++slot;
                        }
                    }
                } else {
                    for (int s2 = lc; s2 < cnt; ++s2) {
                        const float wv = (float)g.b[n * g.ldb + g.idx[s2]];
#pragma unroll
                        for (int r = 0; r < M; ++r)
                            if (r < g.m) pacc[r] += wv * outlier_x(g, r, s2);
                    }
                }
#pragma unroll
                for (int r = 0; r < M; ++r)
                    if (r < g.m) g.out[r * g.ldout + n] = f2h(sw * ((float)acc[r] * sx[r] + pacc[r]) + bj);
            }
        }
#pragma unroll
        for (int r = 0; r < M; ++r) {
            acc[r] = 0;
            pacc[r] = 0.0f;
        }
    };

    // dot4 per 4 weight bytes against the LDS activations; outliers from the bytes in flight
    const int slice = lane * 16;  // this lane's 16 bytes of each chunk
    auto consume = [&](int b, const v4i_t (&wb)[kGvBatch]) {
        const int rr = b / bpr;
        const int c0 = (b - rr * bpr) * kGvBatch;
#pragma unroll
        for (int u = 0; u < kGvBatch; ++u) {
            const int c = c0 + u;
            if (c >= nck) break;
            const int kb = c * kGvChunk;
#pragma unroll
            for (int r = 0; r < M; ++r) {
                const v4i_t xw = *reinterpret_cast<const v4i_t*>(xs + r * kx + kb + slice);
#pragma unroll
                for (int d = 0; d < 4; ++d) acc[r] = __builtin_amdgcn_sdot4(wb[u][d], xw[d], acc[r], false);
            }
            if (kFused && ((chunks_hit >> c) & 1u)) {
#pragma unroll
                for (int e = 0; e < kOwn; ++e)
                    if (own_chunk[e] == c) {
                        const float wv = (float)byte_of(wb[u], own_byte[e]);
#pragma unroll
                        for (int r = 0; r < M; ++r) pacc[r] += wv * own_x[e][r];
                    }
                // spilled columns inside this chunk, one by one
                uint64_t hits = spill ? (__ballot(ocol >= kb && ocol < kb + kGvChunk) & spill) : 0;
                while (hits) {
                    const int s2 = __builtin_ctzll(hits);
                    hits &= hits - 1;
                    const int off = __builtin_amdgcn_readlane(ocol, s2) - kb - slice;  // byte of this lane's slice?
                    float xo[M];
#pragma unroll
                    for (int r = 0; r < M; ++r) xo[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(oxv[r]), s2));
                    if (off >= 0 && off < 16) {
                        const float wv = (float)byte_of(wb[u], off);
#pragma unroll
                        for (int r = 0; r < M; ++r) pacc[r] += wv * xo[r];
                    }
                }
            }
        }
        if (c0 + kGvBatch >= nck) finish_row(rr);
    };

    // batches b and b + 1 in flight while b is consumed
    for (int b = 0; b < nb; b += 2) {
        issue(b + 1, w[1]);
        consume(b, w[0]);
        issue(b + 2, w[0]);
        if (b + 1 < nb) consume(b + 1, w[1]);
    }
}

namespace {

// Rows per wave: about kGvWaves waves over the n weight rows, at most 64
// (a row's epilogue operands sit in one lane each).
int gemv_rows_per_wave(int64_t n) {
    const int64_t r = (n + kGvWaves - 1) / kGvWaves;
    return (int)(r < 64 ? r : 64);
}

size_t gemv_lds(int64_t m_pad, int64_t k, int64_t words, int W, bool quant) {
    const int64_t kx = (k + kGvChunk - 1) / kGvChunk * kGvChunk;
    size_t lds = (size_t)m_pad * kx + (size_t)kGvOutl * 4 + (size_t)m_pad * kGvOutl * 4 +
                 (size_t)W * 64 * (1 + kGvOwn) * 4;
    if (quant) lds += ((size_t)2 * words + m_pad + W + (size_t)W * m_pad) * 4;
    return lds;
}

// m <= 2 with the activations in at most 32 KB of LDS
bool gemv_fits(const GemmArgs& g) {
    const int64_t kx = (g.k + kGvChunk - 1) / kGvChunk * kGvChunk;
    return g.m >= 1 && g.m <= 2 && g.m * kx <= 32 * 1024;
}

template <int M, bool kFused, int kQuantL, int W>
hipError_t launch_gemv_m(const GemmArgs& g, const QuantArgs& qa, hipStream_t stream) {
    const int R = gemv_rows_per_wave(g.n);
    const int64_t waves = (g.n + R - 1) / R;
    const size_t lds = gemv_lds(M, g.k, qa.words, W, kQuantL > 0);
    const dim3 grid((unsigned)((waves + W - 1) / W)), block(64 * W);
    hipLaunchKernelGGL((gemv_kernel<M, kFused, kQuantL, W>), grid, block, lds, stream, g, qa, R);
    return hipGetLastError();
}

template <bool kFused>
hipError_t launch_gemv(const GemmArgs& g, hipStream_t stream) {
    const QuantArgs none{};
    if (g.m == 1) return launch_gemv_m<1, kFused, 0, 4>(g, none, stream);
    return launch_gemv_m<2, kFused, 0, 4>(g, none, stream);
}

// 8-wave workgroups: x is quantized by 512 threads, at most 8 chunks each
template <int M>
hipError_t launch_forward_m(const QuantArgs& qa, const GemmArgs& g, hipStream_t stream) {
    // chunk-major x: each of the 512 threads holds ceil(k/8 / 512) chunks of all M rows
    const int64_t per_thread = M * ((qa.k / 8 + 511) / 512);
    if (per_thread <= 4) return launch_gemv_m<M, true, 4, 8>(g, qa, stream);
    return launch_gemv_m<M, true, 8, 8>(g, qa, stream);
}

}  // namespace

bool decode_forward_fits(const QuantArgs& qa, const GemmArgs& g) {
    const bool w_aligned = ((g.ldb & 15) == 0) && ((reinterpret_cast<uintptr_t>(g.b) & 15) == 0);
    // whole 16-byte chunks of x: k and ldx multiples of 8, x 16-byte aligned
    const bool x_vec = ((qa.k & 7) == 0) && ((qa.ldx & 7) == 0) && ((reinterpret_cast<uintptr_t>(qa.x) & 15) == 0);
    // at most 8 chunks of x per thread of 512 (chunk-major over the rows)
    const bool x_regs = qa.m * ((qa.k / 8 + 511) / 512) <= 8;
    // the codes are copied from the LDS rows in 16-byte units
    const bool q_rows = qa.q && qa.kpad == qa.ldq && (qa.ldq & 15) == 0 &&
                        ((reinterpret_cast<uintptr_t>(qa.q) & 15) == 0);
    return qa.m == g.m && qa.k == g.k && gemv_fits(g) && w_aligned && x_vec && x_regs && q_rows && qa.absmax;
}

hipError_t launch_decode_forward(const QuantArgs& qa, const GemmArgs& g, hipStream_t stream) {
    if (g.m == 1) return launch_forward_m<1>(qa, g, stream);
    return launch_forward_m<2>(qa, g, stream);
}

namespace {
constexpr int64_t kDecCUs = 256;   // MI355X compute units

// whole 16-row groups (NB = 1), gsplit waves per group
template <bool kHalfA>
hipError_t launch_decode_g(const GemmArgs& g, int gsplit, bool fused, dim3 grid, hipStream_t stream) {
    switch (gsplit * 2 + (fused ? 1 : 0)) {
        case 2: hipLaunchKernelGGL((gemm_decode_kernel<1, false, kHalfA, 1>), grid, dim3(256), 0, stream, g, kRows); break;
        case 3: hipLaunchKernelGGL((gemm_decode_kernel<1, true, kHalfA, 1>), grid, dim3(256), 0, stream, g, kRows); break;
        case 4: hipLaunchKernelGGL((gemm_decode_kernel<2, false, kHalfA, 1>), grid, dim3(256), 0, stream, g, kRows); break;
        case 5: hipLaunchKernelGGL((gemm_decode_kernel<2, true, kHalfA, 1>), grid, dim3(256), 0, stream, g, kRows); break;
        case 8: hipLaunchKernelGGL((gemm_decode_kernel<4, false, kHalfA, 1>), grid, dim3(256), 0, stream, g, kRows); break;
        default: hipLaunchKernelGGL((gemm_decode_kernel<4, true, kHalfA, 1>), grid, dim3(256), 0, stream, g, kRows); break;
    }
    return hipGetLastError();
}

// groups of rg rows in NB blocks, G waves (splitting K) per group
template <bool kHalfA, int NB, int G>
hipError_t launch_decode_wide(const GemmArgs& g, int rg, bool fused, hipStream_t stream) {
    const int64_t groups = (g.n + rg - 1) / rg;
    const dim3 grid((unsigned)((groups * G + kWaves - 1) / kWaves));
    if (fused)
        hipLaunchKernelGGL((gemm_decode_kernel<G, true, kHalfA, NB>), grid, dim3(256), 0, stream, g, rg);
    else
        hipLaunchKernelGGL((gemm_decode_kernel<G, false, kHalfA, NB>), grid, dim3(256), 0, stream, g, rg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const GemmArgs& g, bool fused, hipStream_t stream) {
    if (gemv_fits(g)) return fused ? launch_gemv<true>(g, stream) : launch_gemv<false>(g, stream);
    const int64_t groups = (g.n + kRows - 1) / kRows;
    const int64_t nchunks = (g.k + kChunk - 1) / kChunk;
    // Between one and four 16-row groups per CU and K long enough for 16
    // chunks per wave: one workgroup per CU instead, with one group of
    // ceil(n / 256) rows (four waves) or two of ceil(n / 512) (two waves
    // each), each at most 32 rows in two blocks that share the activation
    // fragments.  With whole 16-row groups the CUs that take more of them set
    // the time (13B down, 320 groups: m = 16 22.1 -> 17.9 us, m = 4 16.2 ->
    // 14.7 us).  Groups of three or four blocks measured slower: one
    // workgroup of 122 KB per CU and short runs.
    if (groups > kDecCUs && groups <= 4 * kDecCUs) {
        const bool two = groups > 2 * kDecCUs;
        if (nchunks / (two ? 2 : 4) >= 16) {
            const int rg = (int)((g.n + (two ? 2 : 1) * kDecCUs - 1) / ((two ? 2 : 1) * kDecCUs));
            if (two)
                return g.m <= 8 ? launch_decode_wide<true, 2, 2>(g, rg, fused, stream)
                                : launch_decode_wide<false, 2, 2>(g, rg, fused, stream);
            return g.m <= 8 ? launch_decode_wide<true, 2, 4>(g, rg, fused, stream)
                            : launch_decode_wide<false, 2, 4>(g, rg, fused, stream);
        }
    }
    // waves per 16-row group: enough K splits that each wave has a long run of
    // 128-byte chunks; fewer where that would put more than two workgroups on
    // each CU and leave the runs short
    int gsplit = 1;
    while (gsplit < kWaves && nchunks / (2 * gsplit) >= 16) gsplit *= 2;
    while (gsplit > 1 && groups * gsplit / kWaves > 2 * 256 && nchunks / gsplit < 32) gsplit /= 2;
    dim3 grid((unsigned)((groups * gsplit + kWaves - 1) / kWaves));
    if (g.m <= 8) return launch_decode_g<true>(g, gsplit, fused, grid, stream);
    return launch_decode_g<false>(g, gsplit, fused, grid, stream);
}

}  // namespace i8mp

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
// K advances in 128-byte tiles staged through LDS.  gemm_dtl_kernel, used
// whenever both operands are 16-byte aligned, copies them global -> LDS with
// buffer_load ... lds and keeps 2-4 tiles in flight (optionally two K
// pipelines per workgroup); gemm_kernel, for unaligned operands, double-buffers
// one tile through registers.  Buffer loads return 0 past the end of the
// matrix, so rows beyond m or n need no branches.  LDS rows are 128 bytes with
// the 16-byte chunk index XOR-swizzled so that fragment reads are free of bank
// conflicts.  The contraction order inside an MFMA does not matter: A and B
// fragments use the same lane -> k mapping, and integer sums are exact in any
// order.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile index is
// remapped so that each XCD works on a contiguous run of tiles (sharing
// operand rows in its own L2), walked in groups of group_m tile rows.
#include <stdint.h>

#include "common.h"

namespace i8mp {

namespace {

constexpr int BK = 128;
constexpr int kXcds = 8;

// Tile rows per group of the launch order.  An XCD runs 32 of its tiles at a
// time: a group of r rows walks them r x 32/r, and the K stage of those tiles
// touches r A blocks of BM rows and 32/r B blocks of BN rows.
template <int BM, int BN>
constexpr int group_m() { return BM > BN ? 4 : 8; }
constexpr int kRsrcWord3 = 0x00020000;


__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
    if (bytes < 0) bytes = 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 128-byte LDS rows.  A wave's 16-byte LDS accesses are served 16 lanes
// (256 bytes) at a time; lanes 0-15 of an MFMA fragment read rows r..r+15 at
// the same K chunk, so the chunk is XOR-ed with (row >> 1) & 7: the 16 rows
// then cover all 16 distinct 16-byte bank groups of a 256-byte bank line.
__device__ inline int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// zero the bytes of a 16-byte chunk at or beyond `valid` (0..16)
__device__ inline v4i mask_tail(v4i v, int valid) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        int nb = valid - 4 * d;
        nb = nb < 0 ? 0 : (nb > 4 ? 4 : nb);
        const uint32_t m = nb >= 4 ? 0xffffffffu : ((1u << (8 * nb)) - 1u);
        v[d] = (int)((uint32_t)v[d] & m);
    }
    return v;
}

// Unaligned operands (leading dimension or base not 16-byte aligned): bytes.
__device__ inline v4i load16_bytes(const int8_t* __restrict__ base, int64_t ld, int64_t row,
                                   int64_t nrows, int64_t col, int64_t k) {
    v4i r = {0, 0, 0, 0};
    if (row >= nrows) return r;
    const int8_t* p = base + row * ld + col;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        if (col + e < k) r[e >> 2] |= (int)(((uint32_t)(uint8_t)p[e]) << (8 * (e & 3)));
    return r;
}

template <int kGroupM>
__device__ inline void tile_coords(int64_t bid, int64_t nblocks, int64_t tiles_m, int64_t tiles_n,
                                   int64_t& tm, int64_t& tn) {
    const int64_t full = (nblocks / kXcds) * kXcds;
    int64_t t = bid;
    if (bid < full) t = (bid % kXcds) * (full / kXcds) + bid / kXcds;
    const int64_t in_group = (int64_t)kGroupM * tiles_n;
    const int64_t group = t / in_group;
    const int64_t first_m = group * kGroupM;
    int64_t gsize = tiles_m - first_m;
    if (gsize > kGroupM) gsize = kGroupM;
    tm = first_m + (t % in_group) % gsize;
    tn = (t % in_group) / gsize;
}

}  // namespace

// One wave-wide global -> LDS copy through a buffer resource: lane i's
// `bytes` (4 or 16) land at lds + bytes * i (lds must be wave-uniform).
// Lanes whose VGPR offset is out of range write zeros; the range check does
// not cover the SGPR offset, so every kernel here passes its K offset in the
// VGPR offset and 0 as the SGPR offset.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t src, int8_t* lds, int voffset, int soffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, voffset,
                                             soffset, 0, 0);
}
__device__ inline void dma4(__amdgpu_buffer_rsrc_t src, void* lds, int voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, voffset, 0,
                                             0, 0);
}

// Epilogue operands of a BM x BN tile, copied to LDS when the kernel starts
// (their latency then hides behind the K loop): the tile's row and column
// absmax, the first kEpiIdx outlier column indices and the outlier count.
constexpr int kEpiIdx = 64;
// Outlier slots whose weight bytes the pipelined kernel stashes in LDS as the
// K tiles pass: int32 [kStash][BN], slot s of tile row r = W[n0 + r, idx[s]]
// zero-extended (a 1-byte buffer_load ... lds writes one dword per lane).
// Later slots are gathered from memory in the epilogue.  Only the 256 x 256
// tile stashes: the large GEMMs that use it stream weights far larger than L2,
// so the epilogue's gather would miss; with smaller weights the gather hits
// L2 and the stash measured slower.
constexpr int kStash = 24;
template <int BM, int BN, bool kFused>
constexpr bool stash_on() { return kFused && BM == 256 && BN == 256; }

// MFMA steps of a pipelined iteration over which the DMA of the tile it
// requests is spread.  With two stages that tile is waited for at the end of
// the same iteration, so its DMA goes out in the first two steps (more bytes
// in flight on average); deeper pipelines spread it over every step.
template <int STAGES, int NSTEP>
constexpr int dma_steps() { return STAGES == 2 && NSTEP > 2 ? 2 : NSTEP; }
template <int BM, int BN>
struct __attribute__((aligned(16))) EpiLds {
    float sx[BM];
    float sw[BN];
    int32_t idx[kEpiIdx];
    int32_t cnt[64];
};

template <int BM, int BN, bool kFused>
__device__ inline void epi_prefetch(const GemmArgs& g, int64_t m0, int64_t n0, EpiLds<BM, BN>& e, int wave,
                                    int lane) {
    static_assert(BM % 64 == 0 && BN % 64 == 0, "scale copies are 64 lanes wide");
    if constexpr (kFused) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.row_absmax + m0, (g.m - m0) * 4);
        const __amdgpu_buffer_rsrc_t cs = make_rsrc(g.col_absmax + n0, (g.n - n0) * 4);
        for (int c = wave; c < BM / 64; c += 4) dma4(rs, e.sx + c * 64, (c * 64 + lane) * 4);
        for (int c = wave; c < BN / 64; c += 4) dma4(cs, e.sw + c * 64, (c * 64 + lane) * 4);
        if (g.count) {
            if (wave == 0) dma4(make_rsrc(g.idx, (int64_t)g.idx_len * 4), e.idx, lane * 4);
            if (wave == 1) dma4(make_rsrc(g.count, 4), e.cnt, 0);
        }
    }
}

// Epilogue shared by the GEMM kernels.  Accumulator (i, j, r) of lane l holds
// row wr0 + 32 i + 8 (r/4) + 4 (l/32) + r%4 and column wc0 + 32 j + l%32 of the
// tile at (m0, n0); the same layout holds for the fp32 32x32 MFMA.  Every
// load and store goes through a buffer resource, so rows past m and columns
// past n need no branches (out-of-range loads return 0, stores are dropped),
// and the loads of each phase are issued together.
//
// Fused: acc becomes float(C) * row_absmax / 127 in place, the outlier
// sub-matmul accumulates into it on v_mfma_f32_32x32x16_f16 (16 outlier
// columns per step: x values from X_O in the workspace, or for slots past its
// capacity from x through the index list; weight bytes gathered through the
// index list), then out = col_absmax / 127 * acc + bias in fp16.
template <int BM, int BN, int FM, int FN, bool kFused, int kStageBytes>
__device__ inline void epilogue(const GemmArgs& g, v16i (&acc)[FM][FN], int64_t m0, int64_t n0, int wr0, int wc0,
                                int lane, const EpiLds<BM, BN>& e, int8_t* stage, const int32_t* stash = nullptr,
                                int n_stash = 0) {
    const int hi = lane >> 5, l32 = lane & 31;
    const int64_t rows_left = g.m - m0, cols_left = g.n - n0;
    if constexpr (!kFused) {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.c + m0 * g.ldc + n0, ((rows_left - 1) * g.ldc + cols_left) * 4);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int lcol = wc0 + 32 * j + l32;
            const bool okc = lcol < cols_left;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int lrow = wr0 + 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const int off = okc ? (lrow * (int)g.ldc + lcol) * 4 : (int)0x80000000;
                    __builtin_amdgcn_raw_buffer_store_b32(acc[i][j][r], rc, off, 0, 0);
                }
        }
    } else {
        const float r127 = 1.0f / 127.0f;
        // bias first: its loads are in flight during the conversion and the outlier term
        const __amdgpu_buffer_rsrc_t rbias = make_rsrc(g.bias ? g.bias + n0 : nullptr, g.bias ? cols_left * 2 : 0);
        float bj[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bj[j] = (float)__builtin_bit_cast(
                _Float16, __builtin_amdgcn_raw_buffer_load_b16(rbias, (wc0 + 32 * j + l32) * 2, 0, 0));

        int cnt = 0;
        if (g.count) cnt = outlier_count(g, e.cnt[0]);
        cnt = __builtin_amdgcn_readfirstlane(cnt);
        // slots below xo_lim read their x values from X_O as 8-slot vectors
        // (X_O is zero from the count to ldo); past it, slot by slot
        const int xo_lim = cnt <= g.cap ? (int)g.ldo : g.cap;
        const __amdgpu_buffer_rsrc_t rxo = make_rsrc(g.x_out ? g.x_out + m0 * g.ldo : nullptr,
                                                     g.x_out ? rows_left * g.ldo * 2 : 0);
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.x ? g.x + m0 * g.ldx : nullptr, g.x ? rows_left * g.ldx * 2 : 0);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.b + n0 * g.ldb, (cols_left - 1) * g.ldb + g.k);
        const __amdgpu_buffer_rsrc_t ridx = make_rsrc(g.idx, g.count ? (int64_t)g.idx_len * 4 : 0);
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(g.out + m0 * g.ldout + n0, ((rows_left - 1) * g.ldout + cols_left) * 2);

        // rows of blocks in chunks of IC, so that at most 128 fp32 values are live
        constexpr int IC = FM * FN * 16 <= 128 ? FM : (128 / (FN * 16) > 0 ? 128 / (FN * 16) : 1);
        constexpr int WN = FN * 32;
        constexpr int kPitch = WN * 2 + 16;   // LDS row pitch of the output staging area
        static_assert(4 * IC * 32 * kPitch <= kStageBytes, "output staging does not fit the K stages");
        const int wave = (wr0 / (FM * 32)) * 2 + wc0 / WN;
        int8_t* area = stage + wave * (IC * 32 * kPitch);
        const bool vec_ok = (g.ldout & 7) == 0 && (reinterpret_cast<uintptr_t>(g.out) & 15) == 0;

        // The operands of the first 16 outlier slots are copied to LDS before
        // the conversion, so that their latency hides behind it: the wave's
        // X_O rows (fp16 [FM*32][16]; X_O is zero past the count) and, for
        // slots the stash does not hold, the weight bytes of its columns (one
        // zero-extended dword each, [16][WN]).  Each wave has a private area:
        // in the idle K stages past the output staging, or where that does not
        // fit, at the start of its own staging area (one row chunk only: the
        // wave reads the copies before it writes its results there).
        constexpr int kXoOff = (4 * IC * 32 * kPitch + 1023) / 1024 * 1024;
        constexpr int kXoBytes = FM * 32 * 16 * 2;
        constexpr int kPreBytes = kXoBytes + 16 * WN * 4;
        constexpr bool kSep = kXoOff + 4 * kPreBytes <= kStageBytes;
        static_assert(kSep || (IC == FM && kPreBytes <= IC * 32 * kPitch), "outlier operands do not fit the K stages");
        int8_t* const pre = kSep ? stage + kXoOff + wave * kPreBytes : area;
        const int32_t* const pre_w = reinterpret_cast<const int32_t*>(pre + kXoBytes);
        // the 256 x 256 tile's weight bytes come from its stash instead
        constexpr bool kPreW = !(BM == 256 && BN == 256);
        constexpr int kWIns = 16 * WN / 64;   // weight-byte copies: entry q*64 + lane -> slot, column
        const int npre = cnt < 16 ? cnt : 16;
        // every slot below npre has LDS operands: X_O holds it, and so does
        // the stash where the weight bytes come from there
        const bool pre_ok = npre > 0 && npre <= g.cap && (kPreW || npre <= n_stash);
        if (pre_ok) {
            int ixv[kPreW ? kWIns : 1];
            if constexpr (kPreW) {
                // index reads first: an LDS read issued after a copy to LDS waits for it
#pragma unroll
                for (int q = 0; q < kWIns; ++q) ixv[q] = e.idx[(q * 64 + lane) / WN];
            }
#pragma unroll
            for (int q = 0; q < FM; ++q)   // 32 rows per instruction: lane -> row lane / 2, half lane % 2
                dma16(rxo, pre + q * 1024, ((wr0 + q * 32 + (lane >> 1)) * (int)g.ldo + 8 * (lane & 1)) * 2, 0);
            if constexpr (kPreW) {
                if (npre > n_stash) {
#pragma unroll
                    for (int q = 0; q < kWIns; ++q) {
                        const int ent = q * 64 + lane, slot = ent / WN;
                        const int off = slot < npre && slot >= n_stash ? (wc0 + ent % WN) * (int)g.ldb + ixv[q]
                                                                      : (int)0x80000000;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rw, (__attribute__((address_space(3))) void*)(pre + kXoBytes + q * 256), 1, off, 0, 0,
                            0);
                    }
                }
            }
        }
#pragma unroll
        for (int ic = 0; ic < FM; ic += IC) {
            v16f f[IC][FN];
#pragma unroll
            for (int ii = 0; ii < IC; ++ii) {
                const int i = ic + ii;
                float sxr[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4f s4 = *reinterpret_cast<const v4f*>(&e.sx[wr0 + 32 * i + 8 * q + 4 * hi]);
#pragma unroll
                    for (int t = 0; t < 4; ++t) sxr[4 * q + t] = s4[t] * r127;
                }
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) f[ii][j][r] = (float)acc[i][j][r] * sxr[r];
            }

            if (ic == 0 && pre_ok) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the LDS copies landed
            for (int s0 = 0; s0 < cnt; s0 += 16) {
                const int sb = s0 + 8 * hi;   // this lane's 8 outlier slots
                if (s0 == 0 && pre_ok) {
                    // the slots copied to LDS above (and the stash)
                    v8h xa[IC];
#pragma unroll
                    for (int ii = 0; ii < IC; ++ii)
                        xa[ii] = *reinterpret_cast<const v8h*>(pre + (32 * (ic + ii) + l32) * 32 + hi * 16);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int lc = 32 * j + l32;
                        v8h wb;
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            // the copies hold zeros past npre; the stash holds npre <= n_stash slots
                            const int slot = sb + t;
                            int32_t w;
                            if constexpr (kPreW) {
                                w = pre_w[slot * WN + lc];
                            } else {
                                const int32_t v = stash[slot * BN + wc0 + lc];
                                w = slot < npre ? v : 0;
                            }
                            wb[t] = (_Float16)(float)(int8_t)(uint8_t)(uint32_t)w;
                        }
#pragma unroll
                        for (int ii = 0; ii < IC; ++ii)
                            f[ii][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[ii], wb, f[ii][j], 0, 0, 0);
                    }
                    continue;
                }
                int ix[8];
                if (s0 + 16 <= kEpiIdx) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) ix[t] = e.idx[sb + t];
                } else {
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        ix[t] = (int)__builtin_amdgcn_raw_buffer_load_b32(ridx, (sb + t) * 4, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) ix[t] = sb + t < cnt ? ix[t] : -1;
                v8h xa[IC];
                if (sb + 8 <= xo_lim) {
#pragma unroll
                    for (int ii = 0; ii < IC; ++ii) {
                        const int lrow = wr0 + 32 * (ic + ii) + l32;
                        xa[ii] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(
                                                             rxo, (lrow * (int)g.ldo + sb) * 2, 0, 0));
                    }
                } else {
                    // slots past X_O's capacity: x[row, idx[slot]] one by one
#pragma unroll
                    for (int ii = 0; ii < IC; ++ii) {
                        const int lrow = wr0 + 32 * (ic + ii) + l32;
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            const int slot = sb + t;
                            const uint16_t h =
                                slot < g.cap ? __builtin_amdgcn_raw_buffer_load_b16(rxo, (lrow * (int)g.ldo + slot) * 2, 0, 0)
                                             : __builtin_amdgcn_raw_buffer_load_b16(
                                                   rx, ix[t] >= 0 ? (lrow * (int)g.ldx + ix[t]) * 2 : (int)0x80000000, 0, 0);
                            xa[ii][t] = __builtin_bit_cast(_Float16, h);
                        }
                    }
                }
                uint32_t wby[FN][8];
                if (sb + 8 <= n_stash) {
                    // weight bytes stashed from the K tiles: 8 slots of the lane's column
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int lcol = wc0 + 32 * j + l32;
#pragma unroll
                        for (int t = 0; t < 8; ++t) wby[j][t] = (uint32_t)stash[(sb + t) * BN + lcol];
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int lcol = wc0 + 32 * j + l32;
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            const int slot = sb + t;
                            const int off = ix[t] >= 0 ? lcol * (int)g.ldb + ix[t] : (int)0x80000000;
                            wby[j][t] = slot < n_stash ? (uint32_t)stash[slot * BN + lcol]
                                                       : __builtin_amdgcn_raw_buffer_load_b8(rw, off, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    v8h wb;
#pragma unroll
                    for (int t = 0; t < 8; ++t) wb[t] = (_Float16)(float)(int8_t)(uint8_t)wby[j][t];
#pragma unroll
                    for (int ii = 0; ii < IC; ++ii)
                        f[ii][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[ii], wb, f[ii][j], 0, 0, 0);
                }
            }

            // fp16 results go through this wave's LDS area (the idle K stages) so
            // that each lane writes 16 contiguous bytes of a row: 8 columns per
            // store instead of one
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int ccol = 32 * j + l32;
                const float swj = e.sw[wc0 + ccol] * r127;
#pragma unroll
                for (int ii = 0; ii < IC; ++ii)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int crow = 32 * ii + 8 * (r >> 2) + 4 * hi + (r & 3);
                        *reinterpret_cast<_Float16*>(area + crow * kPitch + ccol * 2) =
                            (_Float16)(swj * f[ii][j][r] + bj[j]);
                    }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
            constexpr int CPR = WN / 8;          // 16-byte chunks per row
            constexpr int RPI = 64 / CPR;        // rows per store instruction
#pragma unroll
            for (int q = 0; q < IC * 32 / RPI; ++q) {
                const int crow = q * RPI + lane / CPR;
                const int c = lane % CPR;
                const v4i v = *reinterpret_cast<const v4i*>(area + crow * kPitch + c * 16);
                const int trow = wr0 + 32 * ic + crow;   // tile row (rows past m are dropped by the range)
                const int tcol = wc0 + 8 * c;
                const int off = (trow * (int)g.ldout + tcol) * 2;
                if (vec_ok && tcol + 8 <= cols_left) {
                    // streaming (nt) stores: every tile writes its whole output
                    // at once at the end, and nothing here reads it back
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), ro, off, 0, 2);
                } else if (tcol < cols_left) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const uint32_t h = ((uint32_t)v[t >> 1] >> (16 * (t & 1))) & 0xffffu;
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)h, ro,
                                                              tcol + t < cols_left ? off + 2 * t : (int)0x80000000, 0, 0);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the area is written again
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int BM, int BN, bool kFused, bool kAligned>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int A_CH = BM * BK / 16 / 256;
    constexpr int B_CH = BN * BK / 16 / 256;
    // one LDS array: A stages, B stages, the epilogue operands
    __shared__ __attribute__((aligned(16))) int8_t smem[2 * (BM + BN) * BK + sizeof(EpiLds<BM, BN>)];
    int8_t(*As)[BM * BK] = reinterpret_cast<int8_t(*)[BM * BK]>(smem);
    int8_t(*Bs)[BN * BK] = reinterpret_cast<int8_t(*)[BN * BK]>(smem + 2 * BM * BK);
    EpiLds<BM, BN>& epi = *reinterpret_cast<EpiLds<BM, BN>*>(smem + 2 * (BM + BN) * BK);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int64_t tiles_m = (g.m + BM - 1) / BM;
    const int64_t tiles_n = (g.n + BN - 1) / BN;
    int64_t tm, tn;
    tile_coords<group_m<BM, BN>()>(blockIdx.x, (int64_t)gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    epi_prefetch<BM, BN, kFused>(g, m0, n0, epi, __builtin_amdgcn_readfirstlane(wave), lane);

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int64_t ktiles = (g.k + BK - 1) / BK;
    const int ktail = (int)(g.k - (ktiles - 1) * BK);  // valid bytes in the last K tile

    // per-thread chunk coordinates within a tile: row = id >> 3, chunk = id & 7
    // The range ends 16-byte-rounded past the last valid row's k bytes: with
    // 16-byte aligned rows that never leaves the row's final 16-byte granule.
    // ranges end at the last row's k rounded up to a dword: the range check is
    // per dword, so no load reaches more than 3 bytes past the operands
    const int64_t k4 = (g.k + 3) & ~(int64_t)3;
    const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(g.a + m0 * g.lda, (g.m - m0 - 1) * g.lda + k4);
    const __amdgpu_buffer_rsrc_t rb_src = make_rsrc(g.b + n0 * g.ldb, (g.n - n0 - 1) * g.ldb + k4);
    int a_off[A_CH], b_off[B_CH];
#pragma unroll
    for (int p = 0; p < A_CH; ++p) {
        const int id = p * 256 + tid;
        a_off[p] = (int)((id >> 3) * g.lda + (id & 7) * 16);
    }
#pragma unroll
    for (int p = 0; p < B_CH; ++p) {
        const int id = p * 256 + tid;
        b_off[p] = (int)((id >> 3) * g.ldb + (id & 7) * 16);
    }

    v4i ra[A_CH], rb[B_CH];
    auto gload = [&](int64_t kt) {
        const int kb = (int)(kt * BK);
        if constexpr (kAligned) {
#pragma unroll
            for (int p = 0; p < A_CH; ++p)
                ra[p] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ra_src, a_off[p] + kb, 0, 0));
#pragma unroll
            for (int p = 0; p < B_CH; ++p)
                rb[p] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rb_src, b_off[p] + kb, 0, 0));
            if (kt == ktiles - 1 && ktail < BK) {
                // bytes past k belong to the next row: zero them in A (B's are then harmless)
#pragma unroll
                for (int p = 0; p < A_CH; ++p) {
                    const int id = p * 256 + tid;
                    ra[p] = mask_tail(ra[p], ktail - (id & 7) * 16);
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < A_CH; ++p) {
                const int id = p * 256 + tid;
                ra[p] = load16_bytes(g.a, g.lda, m0 + (id >> 3), g.m, kb + (id & 7) * 16, g.k);
            }
#pragma unroll
            for (int p = 0; p < B_CH; ++p) {
                const int id = p * 256 + tid;
                rb[p] = load16_bytes(g.b, g.ldb, n0 + (id >> 3), g.n, kb + (id & 7) * 16, g.k);
            }
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

    // Fragments are double-buffered across the four 32-deep K steps of a tile:
    // step s multiplies set s&1 while set (s+1)&1 is read from LDS.  The last
    // step's MFMAs are split around the barrier so that reading the next
    // tile's first fragments overlaps the second half of them.
    v4i fa[2][FM], fb[2][FN];
    auto read_frags = [&](int buf, int s, int set) {
        const int ch = 2 * s + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WM + i * 32 + (lane & 31);
            fa[set][i] = *reinterpret_cast<const v4i*>(&As[buf][swz(row, ch)]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * WN + j * 32 + (lane & 31);
            fb[set][j] = *reinterpret_cast<const v4i*>(&Bs[buf][swz(row, ch)]);
        }
    };
    auto mfmas = [&](int set, int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
    };
    constexpr int kFrags = FM + FN;   // LDS reads per step
    constexpr int kMfma = FM * FN;    // MFMAs per step

    gload(0);
    sstore(0);
    __syncthreads();
    read_frags(0, 0, 0);
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int buf = (int)(kt & 1);
        const bool more = kt + 1 < ktiles;
        if (more) gload(kt + 1);
#pragma unroll
        for (int s = 0; s < BK / 32 - 1; ++s) {
            read_frags(buf, s + 1, (s + 1) & 1);
            mfmas(s & 1, 0, FM);
            // interleave: one LDS read between consecutive MFMAs
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
            for (int t = 0; t < kFrags; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kFrags - 1 > 0 ? kMfma - kFrags - 1 : 0, 0);
        }
        if (more) sstore(buf ^ 1);
        mfmas(1, 0, FM / 2);
        __syncthreads();
        if (more) read_frags(buf ^ 1, 0, 0);
        mfmas(1, FM / 2, FM);
    }

    __syncthreads();  // K loop done everywhere; the epilogue operands copied at the start are visible
    epilogue<BM, BN, FM, FN, kFused, 2 * (BM + BN) * BK>(g, acc, m0, n0, wm * WM, wn * WN, lane, epi, smem);
}

// ---------------------------------------------------------------------------
// Pipelined variant for 16-byte aligned operands whose K extent is covered by
// whole stages (k % BKS == 0, or A zero-padded past k as the forward's codes
// are): operands go global -> LDS with buffer_load ... lds (no register
// staging), STAGES stages of BKS bytes of K deep.  A wave's DMA instruction
// writes 1 KB of LDS contiguously (1024 / BKS rows of BKS bytes; lane i ->
// row i / (BKS/16), 16-byte slot i % (BKS/16)); the lane fetches the global
// chunk that belongs in that slot under the swizzle of swz_k.

// LDS rows of BKS bytes.  A wave's 16-byte LDS accesses are served 16 lanes
// (256 bytes) at a time and lanes 0-15 of an MFMA fragment read rows r..r+15 at
// one K chunk, so the chunk is XOR-ed with bits of the row that differ within
// each group of rows sharing a 256-byte bank line.
template <int BKS>
__device__ inline int swz_k(int row, int chunk) {
    if constexpr (BKS == 128) return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
    else return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

__device__ inline void wait_vm(int n) {
    // s_waitcnt with only vmcnt constrained (expcnt / lgkmcnt at their maxima);
    // gfx9 encoding: vmcnt bits [3:0] and [15:14]
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;
        case 1: __builtin_amdgcn_s_waitcnt(0x0f71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0f72); break;
        case 3: __builtin_amdgcn_s_waitcnt(0x0f73); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0f75); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0f76); break;
        case 7: __builtin_amdgcn_s_waitcnt(0x0f77); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0f78); break;
        case 9: __builtin_amdgcn_s_waitcnt(0x0f79); break;
        case 10: __builtin_amdgcn_s_waitcnt(0x0f7a); break;
        case 11: __builtin_amdgcn_s_waitcnt(0x0f7b); break;
        case 12: __builtin_amdgcn_s_waitcnt(0x0f7c); break;
        case 13: __builtin_amdgcn_s_waitcnt(0x0f7d); break;
        case 14: __builtin_amdgcn_s_waitcnt(0x0f7e); break;
        case 15: __builtin_amdgcn_s_waitcnt(0x0f7f); break;
        case 16: __builtin_amdgcn_s_waitcnt(0x4f70); break;
        case 17: __builtin_amdgcn_s_waitcnt(0x4f71); break;
        case 18: __builtin_amdgcn_s_waitcnt(0x4f72); break;
        case 19: __builtin_amdgcn_s_waitcnt(0x4f73); break;
        case 20: __builtin_amdgcn_s_waitcnt(0x4f74); break;
        case 21: __builtin_amdgcn_s_waitcnt(0x4f75); break;
        case 22: __builtin_amdgcn_s_waitcnt(0x4f76); break;
        case 23: __builtin_amdgcn_s_waitcnt(0x4f77); break;
        case 24: __builtin_amdgcn_s_waitcnt(0x4f78); break;
        case 25: __builtin_amdgcn_s_waitcnt(0x4f79); break;
        case 26: __builtin_amdgcn_s_waitcnt(0x4f7a); break;
        case 27: __builtin_amdgcn_s_waitcnt(0x4f7b); break;
        case 28: __builtin_amdgcn_s_waitcnt(0x4f7c); break;
        case 29: __builtin_amdgcn_s_waitcnt(0x4f7d); break;
        case 30: __builtin_amdgcn_s_waitcnt(0x4f7e); break;
        case 31: __builtin_amdgcn_s_waitcnt(0x4f7f); break;
        case 32: __builtin_amdgcn_s_waitcnt(0x8f70); break;
        case 33: __builtin_amdgcn_s_waitcnt(0x8f71); break;
        case 34: __builtin_amdgcn_s_waitcnt(0x8f72); break;
        case 35: __builtin_amdgcn_s_waitcnt(0x8f73); break;
        case 36: __builtin_amdgcn_s_waitcnt(0x8f74); break;
        case 37: __builtin_amdgcn_s_waitcnt(0x8f75); break;
        case 38: __builtin_amdgcn_s_waitcnt(0x8f76); break;
        case 39: __builtin_amdgcn_s_waitcnt(0x8f77); break;
        case 40: __builtin_amdgcn_s_waitcnt(0x8f78); break;
        case 41: __builtin_amdgcn_s_waitcnt(0x8f79); break;
        case 42: __builtin_amdgcn_s_waitcnt(0x8f7a); break;
        case 43: __builtin_amdgcn_s_waitcnt(0x8f7b); break;
        case 44: __builtin_amdgcn_s_waitcnt(0x8f7c); break;
        case 45: __builtin_amdgcn_s_waitcnt(0x8f7d); break;
        case 46: __builtin_amdgcn_s_waitcnt(0x8f7e); break;
        case 47: __builtin_amdgcn_s_waitcnt(0x8f7f); break;
        default: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    }
}

// KS > 1: KS pipelines of 4 waves in one workgroup split the K tiles (pipe p
// takes global tiles t KS + p), each with its own stages, in lockstep at the
// same barriers; the accumulators meet through LDS at the end.  For grids
// with at most one workgroup per CU, where a single pipeline leaves the CU's
// memory pipe half idle.
template <int BM, int BN, int BKS, int STAGES, bool kFused, int MINW = 1, int KS = 1>
__global__ __launch_bounds__(256 * KS, MINW) void gemm_dtl_kernel(GemmArgs g) {
    static_assert(KS == 1 || !stash_on<BM, BN, kFused>(), "the split pipelines do not stash");
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int NSTEP = BKS / 32;               // 32-deep MFMA steps per stage
    constexpr int LPR = BKS / 16;                 // lanes per row in a DMA instruction
    constexpr int RPI = 64 / LPR;                 // rows per DMA instruction
    constexpr int STAGE_A = BM * BKS, STAGE_B = BN * BKS;
    constexpr int STAGE = STAGE_A + STAGE_B;
    constexpr int A_INS = STAGE_A / 1024 / 4;     // DMA instructions per wave per stage
    constexpr int B_INS = STAGE_B / 1024 / 4;
    constexpr int INS = A_INS + B_INS;
    static_assert(A_INS >= 1 && B_INS >= 1, "tile too small for 4-wave DMA");
    static_assert(STAGES >= 2, "need at least two stages");
    // one LDS array: the stages, then the epilogue operands (a second
    // __shared__ object makes the compiler drain every DMA before each LDS read)
    __shared__ __attribute__((aligned(1024))) int8_t
        smem[KS * STAGES * STAGE + sizeof(EpiLds<BM, BN>) + (stash_on<BM, BN, kFused>() ? kStash * BN * 4 : 0)];
    EpiLds<BM, BN>& epi = *reinterpret_cast<EpiLds<BM, BN>*>(smem + KS * STAGES * STAGE);
    int32_t* stash = reinterpret_cast<int32_t*>(smem + KS * STAGES * STAGE + sizeof(EpiLds<BM, BN>));  // fused only

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pipe = wave_all >> 2;    // K pipeline
    const int wave = wave_all & 3;     // wave within the pipeline
    const int wm = wave >> 1, wn = wave & 1;
    int8_t* const pstage = smem + pipe * STAGES * STAGE;  // this pipeline's stages

    const int64_t tiles_m = (g.m + BM - 1) / BM;
    const int64_t tiles_n = (g.n + BN - 1) / BN;
    int64_t tm, tn;
    tile_coords<group_m<BM, BN>()>(blockIdx.x, (int64_t)gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    if (pipe == 0) epi_prefetch<BM, BN, kFused>(g, m0, n0, epi, wave, lane);

    const int64_t kr = (g.k + BKS - 1) / BKS * BKS;
    const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(g.a + m0 * g.lda, (g.m - m0 - 1) * g.lda + kr);
    // the weight's range ends at the last row's k rounded up to a dword (the
    // range check is per dword); A's codes are zero-padded to whole stages
    const __amdgpu_buffer_rsrc_t rb_src = make_rsrc(g.b + n0 * g.ldb, (g.n - n0 - 1) * g.ldb + ((g.k + 3) & ~(int64_t)3));
    int a_off[A_INS], b_off[B_INS];
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
        const int row = (wave * A_INS + j) * RPI + lane / LPR;
        const int slot = lane % LPR;
        a_off[j] = (int)(row * g.lda + ((swz_k<BKS>(row, slot) - row * BKS)));
    }
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
        const int row = (wave * B_INS + j) * RPI + lane / LPR;
        const int slot = lane % LPR;
        b_off[j] = (int)(row * g.ldb + ((swz_k<BKS>(row, slot) - row * BKS)));
    }
    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    v4i fa[2][FM], fb[2][FN];
    auto read_frags = [&](int stage, int s, int set) {
        const int8_t* base = pstage + stage * STAGE;
        const int ch = 2 * s + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WM + i * 32 + (lane & 31);
            fa[set][i] = *reinterpret_cast<const v4i*>(base + swz_k<BKS>(row, ch));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * WN + j * 32 + (lane & 31);
            fb[set][j] = *reinterpret_cast<const v4i*>(base + STAGE_A + swz_k<BKS>(row, ch));
        }
    };
    auto mfma_rows = [&](int set, int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
    };
    auto barrier = [&]() {
        // LDS reads done, then s_barrier; the signal fences only stop the
        // compiler from moving memory accesses across it.  A memory fence
        // would also wait for the later tiles' DMA, which must stay in flight.
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt unconstrained
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // Tile t lives in stage t % STAGES; STAGES - 1 tiles are requested ahead.
    // The tile that refills stage (kt-1) % STAGES (free once every wave passed
    // the barrier that ends iteration kt-1) is requested during iteration kt,
    // its DMA instructions spread between the MFMAs so that the wave never
    // stalls on a burst of them with the matrix core idle.  A wave waits for
    // its own DMA of a tile with s_waitcnt vmcnt (the tiles requested after it
    // stay in flight); the barrier then makes every wave's part visible.
    // Requests past the last tile read through a zero-length buffer range:
    // they fetch nothing, return zeros, and land in a stage that is not read
    // again.  Issuing them keeps the instruction stream branch-free (so the DMA
    // can be interleaved with the MFMAs) and every vmcnt wait a constant.
    const __amdgpu_buffer_rsrc_t r_none = make_rsrc(g.a, 0);
    const int64_t ktiles = (g.k + BKS - 1) / BKS;
    // pipeline step t holds global K tile t KS + pipe; every pipeline takes
    // the same number of steps (a step past the last tile reads zeros)
    const int64_t nsteps = (ktiles + KS - 1) / KS;
    auto dma_part = [&](int64_t t, int stage, int first, int count) {
        const int64_t gt = t * KS + pipe;
        const bool real = gt < ktiles;
        const int kb = real ? (int)(gt * BKS) : 0;
        int8_t* base = pstage + stage * STAGE;
        const __amdgpu_buffer_rsrc_t sa = real ? ra_src : r_none;
        const __amdgpu_buffer_rsrc_t sb = real ? rb_src : r_none;
#pragma unroll
        for (int q = 0; q < INS; ++q) {
            if (q < first || q >= first + count) continue;
            if (q < A_INS)
                dma16(sa, base + (wave * A_INS + q) * 1024, a_off[q] + kb, 0);
            else
                dma16(sb, base + STAGE_A + (wave * B_INS + (q - A_INS)) * 1024, b_off[q - A_INS] + kb, 0);
        }
    };
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) dma_part(st, st, 0, INS);
    wait_vm((STAGES - 2) * INS);  // tile 0 landed (tiles 1 .. STAGES-2 may be in flight)
    barrier();                    // ... and the epilogue operands copied at the start
    read_frags(0, 0, 0);

    // The weight bytes of the first n_st outlier columns (ascending) are
    // stashed in LDS by 1-byte DMA issued next to the DMA of the K tile that
    // holds them (the line is then on its way through L2 anyway): waves 0 ..
    // BN/64 - 1 take 64 weight rows each.  st_col is the next column to stash
    // (wave-uniform).  These loads only make the vmcnt waits of the wave that
    // issued them stricter (loads complete in order).
    int n_st = 0, st_next = 0;
    int64_t st_col = INT64_MAX;
    if constexpr (stash_on<BM, BN, kFused>()) {
        if (g.count) {
            const int cnt = outlier_count(g, epi.cnt[0]);
            n_st = __builtin_amdgcn_readfirstlane(cnt < kStash ? cnt : kStash);
            if (n_st > 0) st_col = __builtin_amdgcn_readfirstlane(epi.idx[0]);
        }
    }
    auto stash_upto = [&](int64_t col_end) {  // the slots whose column is below col_end
        while (st_col < col_end) {
            if (wave < BN / 64)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb_src, (__attribute__((address_space(3))) void*)(stash + st_next * BN + wave * 64), 1,
                    (int)((wave * 64 + lane) * g.ldb + st_col), 0, 0, 0);
            ++st_next;
            st_col = st_next < n_st ? (int64_t)__builtin_amdgcn_readfirstlane(epi.idx[st_next]) : INT64_MAX;
        }
    };
    if constexpr (stash_on<BM, BN, kFused>()) stash_upto((int64_t)(STAGES - 1) * BKS);  // the tiles requested so far
    // The DMA instructions of the tile requested in an iteration go out over
    // its first DSTEPS MFMA steps, DPS per step, each next to an MFMA.
    constexpr int DSTEPS = dma_steps<STAGES, NSTEP>();
    constexpr int DPS = (INS + DSTEPS - 1) / DSTEPS;
    auto dma_count = [](int s) { const int c = INS - s * DPS; return c < 0 ? 0 : (c > DPS ? DPS : c); };
    // one step's order: MFMAs paired with its fragment reads, then with its
    // DMA; MFMA, fragment read and DMA triples where front-loaded DMA makes
    // more of them than MFMAs
    auto schedule_step = [](int nvm) {
        if (DSTEPS == NSTEP || FM + FN + nvm <= FM * FN) {
#pragma unroll
            for (int t = 0; t < FM + FN; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int t = 0; t < nvm; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < FM * FN; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (t < FM + FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (t < nvm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
    };
    for (int64_t kt = 0; kt < nsteps; ++kt) {
        const int stage = (int)(kt % STAGES);
        const int64_t nt = kt + STAGES - 1;              // step requested in this iteration
        const int rstage = (int)(nt % STAGES);
#pragma unroll
        for (int s = 0; s < NSTEP - 1; ++s) {
            read_frags(stage, s + 1, (s + 1) & 1);
            dma_part(nt, rstage, s * DPS, dma_count(s));
            mfma_rows(s & 1, 0, FM);
            schedule_step(dma_count(s));
        }
        constexpr int LAST = (NSTEP - 1) & 1;
        dma_part(nt, rstage, (NSTEP - 1) * DPS, dma_count(NSTEP - 1));
        mfma_rows(LAST, 0, FM - 1);
#pragma unroll
        for (int t = 0; t < dma_count(NSTEP - 1); ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        if (kt + 1 < nsteps) {
            // steps requested after kt+1: kt+2 .. kt+STAGES-1 (real or not)
            wait_vm((STAGES - 2) * INS);
            barrier();  // tile kt+1 is in LDS everywhere; stage kt is no longer read
            read_frags((int)((kt + 1) % STAGES), 0, 0);
        }
        // the last row of MFMAs covers the next fragments' LDS latency
        mfma_rows(LAST, FM - 1, FM);
        if constexpr (stash_on<BM, BN, kFused>()) stash_upto((nt + 1) * BKS);  // with tile nt, requested in this iteration
    }

    if constexpr (stash_on<BM, BN, kFused>()) wait_vm(0);  // the stash DMA
    __syncthreads();  // no DMA in flight, K loop done everywhere, epilogue operands and stash visible
    if constexpr (KS > 1) {
        // pipelines 1 .. KS-1 hand their accumulators to pipeline 0 through
        // the idle stages: [pipe - 1][wave][i][j][r][lane] int32
        int32_t* red = reinterpret_cast<int32_t*>(smem);
        static_assert((KS - 1) * 4 * FM * FN * 16 * 64 * 4 <= KS * STAGES * STAGE, "reduction area");
        if (pipe > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        red[((((pipe - 1) * 4 + wave) * FM + i) * FN + j) * 16 * 64 + r * 64 + lane] = acc[i][j][r];
        }
        __syncthreads();
        if (pipe == 0) {
#pragma unroll
            for (int p = 1; p < KS; ++p)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[i][j][r] += red[((((p - 1) * 4 + wave) * FM + i) * FN + j) * 16 * 64 + r * 64 + lane];
        }
        __syncthreads();  // the area is free for the epilogue's staging
        if (pipe > 0) return;
    }
    epilogue<BM, BN, FM, FN, kFused, KS * STAGES * STAGE>(g, acc, m0, n0, wm * WM, wn * WN, lane, epi, smem, stash,
                                                      st_next);
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles on 8 waves in ping-pong: two waves per SIMD.
//
// With one wave per SIMD (gemm_dtl_kernel), a wave whose DMA instruction the
// memory pipeline cannot take yet stalls, and the MFMAs behind it in its
// in-order stream wait with it.  Here each SIMD holds two waves of 128 x 64
// int32 accumulators (128 of them per lane).  The waves form two groups of
// four (waves w and w + 4 share SIMD w % 4) that alternate between a memory
// phase (this stage's fragments LDS -> registers, this wave's share of the
// DMA of the stage three ahead) and an MFMA phase (16 MFMAs on the
// fragments), separated by workgroup barriers: group 1 runs one barrier
// behind group 0, so while one group issues memory instructions the other
// keeps the matrix cores busy, and a stalled DMA issue delays only the
// memory phase.  K goes in 64-byte stages, four in LDS: a stage's DMA is
// requested three stages ahead and waited for (by the wave that issued it)
// one stage ahead, so every wave's part has landed at the barrier before
// any wave reads it.  The MFMA phase runs at raised wave priority.
//
// The MFMAs take the weight fragment as their first operand, so lane l
// holds row l % 32 of a 32 x 32 block and four consecutive columns per
// group of four accumulators: the epilogue stores fp16 (or int32) results
// straight from registers, 8 (or 16) bytes per store.
namespace {
constexpr int kPpBK = 64;                  // K bytes per stage
constexpr int kPpStages = 4;
constexpr int kPpWaves = 8;
constexpr int kPpStage = (256 + 256) * kPpBK;
constexpr int kPpLds = kPpStages * kPpStage + (int)sizeof(EpiLds<256, 256>) + kStash * 256 * 4;
static_assert(kPpLds <= 160 * 1024, "ping-pong tile does not fit LDS");

typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_h2(float a, float b) {
    const h2_t h = {(_Float16)a, (_Float16)b};   // round to nearest even
    return __builtin_bit_cast(uint32_t, h);
}

// Epilogue of the transposed layout.  Accumulator (i, j, r) of lane l holds
// row wr0 + 32 i + l % 32 and column wc0 + 32 j + 8 (r / 4) + 4 (l / 32) +
// r % 4 of the tile at (m0, n0).  Loads and stores go through buffer
// resources, so rows past m need no branch; columns past n are masked.
//
// fp16 results are staged through this wave's LDS area (stage, at least
// 2 * 32 * (FN * 64 + 16) bytes, free of other use): each lane writes its
// four-column quads (8 bytes), then reads back 16 contiguous bytes of a row,
// so that every global store covers whole 128-byte row segments.
template <int BM, int BN, int FM, int FN, bool kFused>
__device__ inline void epilogue_tr(const GemmArgs& g, v16i (&acc)[FM][FN], int64_t m0, int64_t n0, int wr0, int wc0,
                                   int lane, const EpiLds<BM, BN>& e, const int32_t* stash, int n_stash,
                                   int8_t* stage) {
    const int hi = lane >> 5, l32 = lane & 31;
    const int64_t rows_left = g.m - m0, cols_left = g.n - n0;
    if constexpr (!kFused) {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.c + m0 * g.ldc + n0, ((rows_left - 1) * g.ldc + cols_left) * 4);
        const bool vec = (g.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(g.c) & 15) == 0;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wr0 + 32 * i + l32;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = wc0 + 32 * j + 8 * q + 4 * hi;
                    const int off = (row * (int)g.ldc + col) * 4;
                    if (vec && col + 4 <= cols_left) {
                        const v4i v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rc, off, 0, 0);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            __builtin_amdgcn_raw_buffer_store_b32(acc[i][j][4 * q + t], rc,
                                                                  col + t < cols_left ? off + 4 * t : (int)0x80000000, 0, 0);
                    }
                }
        }
    } else {
        const float r127 = 1.0f / 127.0f;
        int cnt = 0;
        if (g.count) cnt = outlier_count(g, e.cnt[0]);
        cnt = __builtin_amdgcn_readfirstlane(cnt);
        const int xo_lim = cnt <= g.cap ? (int)g.ldo : g.cap;
        const __amdgpu_buffer_rsrc_t rxo = make_rsrc(g.x_out ? g.x_out + m0 * g.ldo : nullptr,
                                                     g.x_out ? rows_left * g.ldo * 2 : 0);
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.x ? g.x + m0 * g.ldx : nullptr, g.x ? rows_left * g.ldx * 2 : 0);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.b + n0 * g.ldb, (cols_left - 1) * g.ldb + g.k);
        const __amdgpu_buffer_rsrc_t ridx = make_rsrc(g.idx, g.count ? (int64_t)g.idx_len * 4 : 0);
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(g.out + m0 * g.ldout + n0, ((rows_left - 1) * g.ldout + cols_left) * 2);
        const __amdgpu_buffer_rsrc_t rbias = make_rsrc(g.bias ? g.bias + n0 : nullptr, g.bias ? cols_left * 2 : 0);
        const bool vec = (g.ldout & 7) == 0 && (reinterpret_cast<uintptr_t>(g.out) & 15) == 0;

        // the x values of the first 16 outlier slots for every row of the
        // wave, and the bias, go out first: their latency hides behind the
        // conversion
        v8h xa0[FM];
        const bool xa0_vec = cnt > 0 && 8 * hi + 8 <= xo_lim;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int lrow = wr0 + 32 * i + l32;
            xa0[i] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rxo, xa0_vec ? (lrow * (int)g.ldo + 8 * hi) * 2 : (int)0x80000000, 0, 0));
        }
        // (two dword loads per four columns: this compiler folds the second
        // dword of an 8-byte buffer load's result onto the first)
        uint32_t braw[FN][4][2];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int d = 0; d < 2; ++d)
                    braw[j][q][d] = __builtin_amdgcn_raw_buffer_load_b32(rbias, (wc0 + 32 * j + 8 * q + 4 * hi) * 2 + 4 * d, 0, 0);

        // x values of 8 outlier slots (from sb) of tile row lrow: X_O as a
        // vector below xo_lim, else slot by slot (X_O or x through idx)
        auto x_slots = [&](int sb, int lrow, const int (&ix)[8]) -> v8h {
            if (sb + 8 <= xo_lim)
                return __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rxo, (lrow * (int)g.ldo + sb) * 2, 0, 0));
            v8h v;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int slot = sb + t;
                const uint16_t h = slot < g.cap ? __builtin_amdgcn_raw_buffer_load_b16(rxo, (lrow * (int)g.ldo + slot) * 2, 0, 0)
                                                : __builtin_amdgcn_raw_buffer_load_b16(
                                                      rx, ix[t] >= 0 ? (lrow * (int)g.ldx + ix[t]) * 2 : (int)0x80000000, 0, 0);
                v[t] = __builtin_bit_cast(_Float16, h);
            }
            return v;
        };

        constexpr int IC = 2;   // rows of blocks per pass: 32 fp32 results per block and lane
        static_assert(FM % IC == 0, "row blocks in pairs");
#pragma unroll
        for (int ic = 0; ic < FM; ic += IC) {
            v16f f[IC][FN];
#pragma unroll
            for (int ii = 0; ii < IC; ++ii) {
                const float sxr = e.sx[wr0 + 32 * (ic + ii) + l32] * r127;
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) f[ii][j][r] = (float)acc[ic + ii][j][r] * sxr;
            }
            // outlier sub-matmul: 16 slots per step; weight bytes (first
            // operand: this lane's column) from the stash or gathered
            for (int s0 = 0; s0 < cnt; s0 += 16) {
                const int sb = s0 + 8 * hi;
                int ix[8];
                if (s0 + 16 <= kEpiIdx) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) ix[t] = e.idx[sb + t];
                } else {
#pragma unroll
                    for (int t = 0; t < 8; ++t) ix[t] = (int)__builtin_amdgcn_raw_buffer_load_b32(ridx, (sb + t) * 4, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) ix[t] = sb + t < cnt ? ix[t] : -1;
                v8h xa[IC];
#pragma unroll
                for (int ii = 0; ii < IC; ++ii)
                    xa[ii] = (s0 == 0 && xa0_vec) ? xa0[ic + ii] : x_slots(sb, wr0 + 32 * (ic + ii) + l32, ix);
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int lcol = wc0 + 32 * j + l32;
                    v8h wb;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int slot = sb + t;
                        uint32_t w;
                        if (slot < n_stash) {
                            w = (uint32_t)stash[slot * BN + lcol];
                        } else {
                            const int off = ix[t] >= 0 ? lcol * (int)g.ldb + ix[t] : (int)0x80000000;
                            w = __builtin_amdgcn_raw_buffer_load_b8(rw, off, 0, 0);
                        }
                        wb[t] = (_Float16)(float)(int8_t)(uint8_t)w;
                    }
#pragma unroll
                    for (int ii = 0; ii < IC; ++ii)
                        f[ii][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wb, xa[ii], f[ii][j], 0, 0, 0);
                }
            }
            // out = fp16(sw / 127 * f + bias): each lane's four-column quads
            // into the staging area (row pitch kPitch), then rows back out
            constexpr int WN = FN * 32;
            constexpr int kPitch = WN * 2 + 16;
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ccol = 32 * j + 8 * q + 4 * hi;   // column within the wave's block
                    const v4f sw4 = *reinterpret_cast<const v4f*>(&e.sw[wc0 + ccol]);
                    const h2_t b01 = __builtin_bit_cast(h2_t, braw[j][q][0]);
                    const h2_t b23 = __builtin_bit_cast(h2_t, braw[j][q][1]);
                    const float bb[4] = {(float)b01[0], (float)b01[1], (float)b23[0], (float)b23[1]};
#pragma unroll
                    for (int ii = 0; ii < IC; ++ii) {
                        float y[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) y[t] = sw4[t] * r127 * f[ii][j][4 * q + t] + bb[t];
                        const v2u_t v = {pack_h2(y[0], y[1]), pack_h2(y[2], y[3])};
                        *reinterpret_cast<v2u_t*>(stage + (32 * ii + l32) * kPitch + ccol * 2) = v;
                    }
                }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
            constexpr int CPR = WN / 8;          // 16-byte chunks per row
            constexpr int RPI = 64 / CPR;        // rows per store instruction
#pragma unroll
            for (int it = 0; it < IC * 32 / RPI; ++it) {
                const int crow = it * RPI + lane / CPR;
                const int c = lane % CPR;
                const v4i v = *reinterpret_cast<const v4i*>(stage + crow * kPitch + c * 16);
                const int trow = wr0 + 32 * ic + crow;   // tile row (rows past m are dropped by the range)
                const int tcol = wc0 + 8 * c;
                const int off = (trow * (int)g.ldout + tcol) * 2;
                if (vec && tcol + 8 <= cols_left) {
                    // streaming (nt): every tile writes its output at the end, nothing here reads it back
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), ro, off, 0, 2);
                } else if (tcol < cols_left) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const uint32_t h = ((uint32_t)v[t >> 1] >> (16 * (t & 1))) & 0xffffu;
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)h, ro,
                                                              tcol + t < cols_left ? off + 2 * t : (int)0x80000000, 0, 0);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the area is written again
            __builtin_amdgcn_wave_barrier();
        }
    }
}

}  // namespace

template <bool kFused>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256, BKS = kPpBK, NSTAGE = kPpStages;
    constexpr int FM = 4, FN = 2;                 // 128 x 64 per wave
    constexpr int STAGE_A = BM * BKS, STAGE = kPpStage;
    constexpr int INS = 4;                        // DMA instructions per wave per stage (2 A, 2 B)
    constexpr bool kSt = kFused;                  // stash the outlier columns' weight bytes
    __shared__ __attribute__((aligned(1024))) int8_t smem[kPpLds];
    EpiLds<BM, BN>& epi = *reinterpret_cast<EpiLds<BM, BN>*>(smem + NSTAGE * STAGE);
    int32_t* stash = reinterpret_cast<int32_t*>(smem + NSTAGE * STAGE + sizeof(EpiLds<BM, BN>));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..7; SIMD wave % 4
    const int group = wave >> 2;
    const int wm = wave & 1, wn = wave >> 1;                     // 2 x 4 blocks of 128 x 64

    const int64_t tiles_m = (g.m + BM - 1) / BM;
    const int64_t tiles_n = (g.n + BN - 1) / BN;
    int64_t tm, tn;
    tile_coords<group_m<BM, BN>()>(blockIdx.x, (int64_t)gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    epi_prefetch<BM, BN, kFused>(g, m0, n0, epi, wave, lane);

    const int64_t kr = (g.k + BKS - 1) / BKS * BKS;
    const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(g.a + m0 * g.lda, (g.m - m0 - 1) * g.lda + kr);
    const __amdgpu_buffer_rsrc_t rb_src = make_rsrc(g.b + n0 * g.ldb, (g.n - n0 - 1) * g.ldb + ((g.k + 3) & ~(int64_t)3));
    const __amdgpu_buffer_rsrc_t r_none = make_rsrc(g.a, 0);
    // DMA: wave w writes 1 KB blocks 2w, 2w + 1 of the A and of the B part of
    // a stage (16 rows of 64 bytes each; lane i -> row i / 4, slot i % 4,
    // holding the global chunk slot ^ ((row >> 2) & 3))
    int a_off[2], b_off[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = (wave * 2 + q) * 16 + (lane >> 2);
        const int gchunk = (lane & 3) ^ ((row >> 2) & 3);
        a_off[q] = (int)(row * g.lda + gchunk * 16);
        b_off[q] = (int)(row * g.ldb + gchunk * 16);
    }
    const int64_t ktiles = kr / BKS;
    // Stages past the last read through a zero-length range: nothing is
    // fetched, zeros land in a stage that is not read again, and every
    // vmcnt wait stays a constant.
    auto dma_stage = [&](int64_t t) {
        const bool real = t < ktiles;
        const int kb = real ? (int)(t * BKS) : 0;
        int8_t* base = smem + (int)(t % NSTAGE) * STAGE;
        const __amdgpu_buffer_rsrc_t sa = real ? ra_src : r_none;
        const __amdgpu_buffer_rsrc_t sb = real ? rb_src : r_none;
#pragma unroll
        for (int q = 0; q < 2; ++q) dma16(sa, base + (wave * 2 + q) * 1024, a_off[q] + kb, 0);
#pragma unroll
        for (int q = 0; q < 2; ++q) dma16(sb, base + STAGE_A + (wave * 2 + q) * 1024, b_off[q] + kb, 0);
    };
    v4i fa[2][FM], fb[2][FN];
    auto read_frags = [&](int64_t t) {
        const int8_t* base = smem + (int)(t % NSTAGE) * STAGE;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 2 * s + (lane >> 5);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[s][i] = *reinterpret_cast<const v4i*>(base + swz_k<BKS>(wm * 128 + 32 * i + (lane & 31), ch));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[s][j] = *reinterpret_cast<const v4i*>(base + STAGE_A + swz_k<BKS>(wn * 64 + 32 * j + (lane & 31), ch));
        }
    };
    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    auto barrier = [&]() {
        // the wave's LDS reads done, then s_barrier; nothing is scheduled
        // across it (the signal fences keep memory accesses, the scheduling
        // barriers everything else on their side)
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
    };

    dma_stage(0);
    dma_stage(1);
    dma_stage(2);
    wait_vm(2 * INS);   // this wave's part of stage 0 landed
    barrier();          // ... everyone's, and the epilogue operands

    // Outlier columns' weight bytes: the first n_st slots (ascending columns)
    // are copied into the stash by group 0 (64 weight rows per wave) next to
    // the DMA of the stage that holds them, so the lines are on their way
    // through L2 anyway.
    int n_st = 0, st_next = 0;
    int64_t st_col = INT64_MAX;
    if constexpr (kSt) {
        if (g.count) {
            const int cnt = outlier_count(g, epi.cnt[0]);
            n_st = __builtin_amdgcn_readfirstlane(cnt < kStash ? cnt : kStash);
            if (n_st > 0) st_col = __builtin_amdgcn_readfirstlane(epi.idx[0]);
        }
    }
    auto stash_upto = [&](int64_t col_end) {
        while (st_col < col_end) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb_src, (__attribute__((address_space(3))) void*)(stash + st_next * BN + wave * 64), 1,
                (int)((wave * 64 + lane) * g.ldb + st_col), 0, 0, 0);
            ++st_next;
            st_col = st_next < n_st ? (int64_t)__builtin_amdgcn_readfirstlane(epi.idx[st_next]) : INT64_MAX;
        }
    };
    if constexpr (kSt)
        if (group == 0) stash_upto(3 * BKS);

    if (group == 1) barrier();   // group 1 runs one phase behind
    for (int64_t t = 0; t < ktiles; ++t) {
        // memory phase: fragments of stage t, DMA of stage t + 3 (into the
        // stage both groups finished reading before the last barrier)
        read_frags(t);
        dma_stage(t + 3);
        if constexpr (kSt)
            if (group == 0) stash_upto((t + 4) * BKS);
        wait_vm(2 * INS);   // this wave's part of stage t + 1 landed (t + 2, t + 3 in flight)
        barrier();
        // MFMA phase
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[s][j], fa[s][i], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        barrier();
    }
    if (group == 0) barrier();   // both groups have passed the same number of barriers

    wait_vm(0);          // the DMA of the stages past the last and the stash
    __syncthreads();     // the K stages are free: each wave stages its results in its own part
    constexpr int kEpiArea = 2 * 32 * (FN * 64 + 16);
    static_assert(kPpWaves * kEpiArea <= NSTAGE * STAGE, "output staging does not fit the K stages");
    epilogue_tr<BM, BN, FM, FN, kFused>(g, acc, m0, n0, wm * 128, wn * 64, lane, epi, stash, n_st,
                                        smem + wave * kEpiArea);
}

namespace {

// Launch one tile shape: the pipelined direct-to-LDS kernel (128-byte K
// stages, as many stages as fit 160 KB of LDS, at most 4) when both operands
// are 16-byte aligned and A covers whole stages; the register-staged kernel
// otherwise.
template <int BM, int BN, bool kFused>
hipError_t launch_tile(const GemmArgs& g, bool aligned, bool staged, hipStream_t stream) {
    const int64_t tiles = ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
    dim3 grid((unsigned)tiles);
    // stages that fit 160 KB of LDS beside the epilogue operands and the stash, at most 4
    constexpr int kFit =
        (160 * 1024 - (int)sizeof(EpiLds<BM, BN>) - (stash_on<BM, BN, kFused>() ? kStash * BN * 4 : 0)) / ((BM + BN) * 128);
    constexpr int kStages = kFit > 4 ? 4 : kFit;
    // two K pipelines per workgroup when the grid leaves a CU per workgroup
    // and K is long enough; their stages share the same 160 KB
    constexpr int kFit2 = (160 * 1024 - (int)sizeof(EpiLds<BM, BN>)) / (2 * (BM + BN) * 128);
    constexpr int kStages2 = kFit2 > 4 ? 4 : kFit2;
    constexpr bool kCanSplit = !stash_on<BM, BN, kFused>() && kStages2 >= 2;
    const bool split = kCanSplit && tiles <= 256 && (g.k + 127) / 128 >= 16;
    if (staged && BM == 256 && BN == 256) {
        hipLaunchKernelGGL((gemm_pp_kernel<kFused>), grid, dim3(512), 0, stream, g);
    } else if (staged && split) {
        if constexpr (kCanSplit)
            hipLaunchKernelGGL((gemm_dtl_kernel<BM, BN, 128, kStages2, kFused, 1, 2>), grid, dim3(512), 0, stream, g);
    } else if (staged)
        hipLaunchKernelGGL((gemm_dtl_kernel<BM, BN, 128, kStages, kFused>), grid, dim3(256), 0, stream, g);
    else if (aligned)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, kFused, true>), grid, dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, kFused, false>), grid, dim3(256), 0, stream, g);
    return hipGetLastError();
}

// Tile shape by a cost model fitted to traced runs of the pipelined kernel on
// MI355X: a workgroup costs a fixed ~3 us (first stage in flight, epilogue)
// plus k-tiles x the per-128-byte-K-tile time of its shape; workgroups run in
// rounds over the CUs (two 64 x 64 workgroups fit one CU's LDS).
struct TileCand { int bm, bn, per_cu; double tk, tk_shared; };
constexpr int kCands = 6;
constexpr TileCand kTileCands[kCands] = {{256, 256, 1, 1.71, 1.71}, {256, 128, 1, 0.97, 0.97},
                                         {128, 128, 1, 0.50, 0.50}, {128, 64, 1, 0.30, 0.30},
                                         {64, 128, 1, 0.33, 0.33},  {64, 64, 2, 0.26, 0.38}};
constexpr int64_t kCUs = 256;
// the host-side gap between two launches on one stream, in the same units (us)
constexpr double kLaunchGap = 4.0;

int64_t cand_tiles(int c, int64_t m, int64_t n) {
    return ((m + kTileCands[c].bm - 1) / kTileCands[c].bm) * ((n + kTileCands[c].bn - 1) / kTileCands[c].bn);
}
double cand_cost(int c, int64_t m, int64_t n, int64_t k) {
    const int64_t tiles = cand_tiles(c, m, n);
    const int64_t slots = kCUs * kTileCands[c].per_cu;
    const int64_t rounds = (tiles + slots - 1) / slots;
    const double tk = tiles > kCUs ? kTileCands[c].tk_shared : kTileCands[c].tk;
    return (double)rounds * (3.0 + (double)((k + 127) / 128) * tk);
}
int pick_tile(int64_t m, int64_t n, int64_t k, double* cost = nullptr) {
    int best = 0;
    double best_t = 1e300;
    for (int c = 0; c < kCands; ++c) {
        const double t = cand_cost(c, m, n, k);
        if (t < best_t * 0.999) {
            best_t = t;
            best = c;
        }
    }
    if (cost) *cost = best_t;
    return best;
}

// A launch plan: tile `main` over output columns [0, n_main), and, when the
// last round of `main` would leave CUs idle, tile `tail` over the columns
// [n_main, n) in a second launch.  The split is on whole tile columns of the
// main shape that fill whole rounds (65B up, 4096 x 22016: 1280 tiles of
// 256 x 256 in five rounds, then 4096 x 1536 in smaller tiles, instead of a
// sixth round with 96 of 256 CUs busy).
struct TilePlan { int main; int64_t n_main; int tail; };
TilePlan plan_tiles(int64_t m, int64_t n, int64_t k) {
    double single;
    TilePlan plan{pick_tile(m, n, k, &single), n, 0};
    double best_t = single;
    for (int c = 0; c < kCands; ++c) {
        const int64_t slots = kCUs * kTileCands[c].per_cu;
        const int64_t tm = (m + kTileCands[c].bm - 1) / kTileCands[c].bm;
        const int64_t full = cand_tiles(c, m, n) / slots;   // whole rounds
        const int64_t cols = full * slots / tm;              // whole tile columns in them
        const int64_t n_main = cols * kTileCands[c].bn;
        if (cols <= 0 || n_main >= n) continue;
        double tail_t;
        const int tail = pick_tile(m, n - n_main, k, &tail_t);
        const double t = cand_cost(c, m, n_main, k) + kLaunchGap + tail_t;
        if (t < best_t * 0.97) {
            best_t = t;
            plan = TilePlan{c, n_main, tail};
        }
    }
    return plan;
}

template <bool kFused>
hipError_t launch_shape(int c, const GemmArgs& g, bool aligned, bool staged, hipStream_t stream) {
    switch (c) {
        case 0: return launch_tile<256, 256, kFused>(g, aligned, staged, stream);
        case 1: return launch_tile<256, 128, kFused>(g, aligned, staged, stream);
        case 2: return launch_tile<128, 128, kFused>(g, aligned, staged, stream);
        case 3: return launch_tile<128, 64, kFused>(g, aligned, staged, stream);
        case 4: return launch_tile<64, 128, kFused>(g, aligned, staged, stream);
        default: return launch_tile<64, 64, kFused>(g, aligned, staged, stream);
    }
}

template <bool kFused>
hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
    const bool aligned = ((g.lda & 15) == 0) && ((g.ldb & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(g.a) & 15) == 0) &&
                         ((reinterpret_cast<uintptr_t>(g.b) & 15) == 0);
    // the staged kernels read whole 128-byte K stages: A must be zero past k
    const bool staged = aligned && ((g.k & 127) == 0 || g.a_zero_padded);
    if (staged && g.m <= 16) return launch_decode(g, kFused, stream);
    const TilePlan plan = plan_tiles(g.m, g.n, g.k);
    if (plan.n_main >= g.n) return launch_shape<kFused>(plan.main, g, aligned, staged, stream);
    GemmArgs head = g;
    head.n = plan.n_main;
    hipError_t e = launch_shape<kFused>(plan.main, head, aligned, staged, stream);
    if (e != hipSuccess) return e;
    // the remaining columns: every column operand moves by n_main (the weight
    // rows keep 16-byte alignment: n_main is a multiple of the tile width)
    GemmArgs tail = g;
    tail.n = g.n - plan.n_main;
    tail.b = g.b + plan.n_main * g.ldb;
    if (kFused) {
        tail.col_absmax = g.col_absmax + plan.n_main;
        if (g.bias) tail.bias = g.bias + plan.n_main;
        tail.out = g.out + plan.n_main;
    } else {
        tail.c = g.c + plan.n_main;
    }
    return launch_shape<kFused>(plan.tail, tail, aligned, staged, stream);
}

}  // namespace

hipError_t launch_gemm_i32(const GemmArgs& g, hipStream_t stream) { return launch_gemm<false>(g, stream); }
hipError_t launch_gemm_fused(const GemmArgs& g, hipStream_t stream) { return launch_gemm<true>(g, stream); }

}  // namespace i8mp

// extern "C" entry points of libi8mp.so: argument validation, workspace
// layout, launch sequencing.  Nothing here allocates, synchronizes or reads
// device memory; every launch goes to the caller's stream.
#include <atomic>
#include <cstring>
#include <mutex>

#include "common.h"
#include "backward.h"
#include "fp4.h"

using namespace i8mp;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

std::atomic<int> g_arch_ok[64];  // 0 unknown, 1 gfx950, -1 other

i8mp_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return I8MP_EDEVICE;
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return I8MP_OK;
    if (c == -1) return I8MP_EDEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return I8MP_EDEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? I8MP_OK : I8MP_EDEVICE;
}

i8mp_status launched(hipError_t e) { return e == hipSuccess ? I8MP_OK : I8MP_ELAUNCH; }

bool bad_k(int64_t k) { return k < 1; }
bool bad_ld(int64_t ld) { return ld > I8MP_MAX_LD; }

void forward_layout(int64_t m, int64_t k, int32_t cap, i8mp_linear_workspace* L) {
    std::memset(L, 0, sizeof(*L));
    L->ldq = round_up(k, 128);
    L->cap_pad = (int32_t)round_up(cap, 32);
    L->idx_len = round_up(k, 32);   // room for every column: the list is never cut
    size_t off = 0;
    L->scratch_offset = off;
    L->scratch_bytes = quant_scratch_bytes(k);
    off = align_up(off + L->scratch_bytes);
    L->bitmap_offset = off;
    off = align_up(off + (size_t)ceil_div(k, 32) * 4);
    L->idx_offset = off;
    off = align_up(off + (size_t)L->idx_len * 4);
    L->count_offset = off;
    off = align_up(off + 4);
    L->absmax_offset = off;
    off = align_up(off + (size_t)m * 4);
    L->q_offset = off;
    off = align_up(off + (size_t)m * (size_t)L->ldq);
    L->xo_offset = off;
    off = align_up(off + (size_t)m * (size_t)L->cap_pad * 2);
    L->bytes = off;
}

void backward_layout(int64_t m, int64_t n, int64_t k, int32_t cap, i8mp_backward_workspace* L) {
    std::memset(L, 0, sizeof(*L));
    L->ld_n = round_up(n > 0 ? n : 1, 128);
    L->ld_m = round_up(m > 0 ? m : 1, 128);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + (bytes > 0 ? bytes : 1));
        return at;
    };
    L->gq_offset = take((size_t)m * (size_t)L->ld_n);
    L->gs_offset = take((size_t)m * 4);
    L->wtq_offset = take((size_t)k * (size_t)L->ld_n);
    L->wts_offset = take((size_t)k * 4);
    L->gtq_offset = take((size_t)n * (size_t)L->ld_m);
    L->gts_offset = take((size_t)n * 4);
    L->xtq_offset = take((size_t)k * (size_t)L->ld_m);
    L->xts_offset = take((size_t)k * 4);
    // column maxima of the three column-wise quantizations (run one after the
    // other on the stream, so they share one buffer), then the fp32 sums of
    // the outlier columns of grad_w
    size_t colmax = colquant_scratch_bytes(n, k);
    if (colquant_scratch_bytes(m, n) > colmax) colmax = colquant_scratch_bytes(m, n);
    if (colquant_scratch_bytes(m, k) > colmax) colmax = colquant_scratch_bytes(m, k);
    L->scratch_offset = off;
    const size_t acc_at = align_up(colmax);
    L->scratch_bytes = acc_at + fix_part_bytes(m, n, cap);
    off = align_up(off + L->scratch_bytes);
    L->bytes = off;
}

}  // namespace

extern "C" {

const char* i8mp_status_string(i8mp_status s) {
    switch (s) {
        case I8MP_OK: return "ok";
        case I8MP_EINVAL: return "invalid argument (NULL pointer, size or leading dimension)";
        case I8MP_ERANGE: return "k exceeds the exact int32 accumulation limit (133144)";
        case I8MP_EWORKSPACE: return "workspace missing or too small";
        case I8MP_EDEVICE: return "no gfx950 device is current";
        case I8MP_ELAUNCH: return "kernel launch failed";
        case I8MP_ESCRATCH: return "the call needs more than the library's fixed scratch array holds";
        default: return "unknown status";
    }
}

int32_t i8mp_abi_version(void) { return (3 << 16) | 0; }

size_t i8mp_quant_workspace_bytes(int64_t m, int64_t k) {
    if (m <= 0 || k < 1 || k > I8MP_MAX_K) return 0;
    return quant_scratch_bytes(k);
}

i8mp_status i8mp_int8_vectorwise_quant(const void* x, int64_t m, int64_t k, int64_t ldx,
                                       float threshold, int8_t* q, int64_t ldq, float* absmax,
                                       uint32_t* outlier_bitmap, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    if (m < 0 || bad_k(k) || ldx < k || ldq < k) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m > 0 && (!x || !q || !absmax)) return I8MP_EINVAL;
    const bool detect = threshold > 0.0f;
    if (detect && m > 0 && (!workspace || workspace_bytes < quant_scratch_bytes(k))) return I8MP_EWORKSPACE;
    if (m == 0 && !outlier_bitmap) return I8MP_OK;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    QuantArgs a{};
    a.x = static_cast<const half_bits*>(x);
    a.m = m;
    a.k = k;
    a.ldx = ldx;
    a.threshold = threshold;
    a.partial = static_cast<uint32_t*>(workspace);
    a.words = ceil_div(k, 32);
    a.q = q;
    a.ldq = ldq;
    a.kpad = k;
    a.absmax = absmax;
    a.bitmap_out = outlier_bitmap;
    return launched(launch_quantize(a, stream));
}

i8mp_status i8mp_outlier_extract(const void* x, int64_t m, int64_t k, int64_t ldx,
                                 const uint32_t* outlier_bitmap, int32_t cap, int32_t* idx,
                                 int32_t* count, void* x_out, int64_t ldo, hipStream_t stream) {
    if (m < 0 || bad_k(k) || ldx < k || cap < 0) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (!outlier_bitmap || !count || (cap > 0 && !idx)) return I8MP_EINVAL;
    if (m > 0 && !x) return I8MP_EINVAL;
    if (x_out && ldo < cap) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    QuantArgs a{};
    a.x = static_cast<const half_bits*>(x);
    a.m = x_out ? m : 0;
    a.k = k;
    a.ldx = ldx;
    a.bitmap_in = outlier_bitmap;
    a.row_blocks = 1;
    a.words = ceil_div(k, 32);
    a.idx_out = cap > 0 ? idx : nullptr;
    a.count_out = count;
    a.cap = cap;
    a.idx_len = cap;
    a.x_out = static_cast<half_bits*>(x_out);
    a.ldo = ldo;
    a.xo_cols = cap;
    return launched(launch_quant_rows(a, stream));
}

i8mp_status i8mp_int8_linear_matmul(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                                    int64_t m, int64_t n, int64_t k, int32_t* c, int64_t ldc,
                                    hipStream_t stream) {
    if (m < 0 || n < 0 || bad_k(k) || lda < k || ldb < k || ldc < n) return I8MP_EINVAL;
    if (bad_ld(lda) || bad_ld(ldb) || bad_ld(ldc)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0 || n == 0) return I8MP_OK;
    if (!a || !b || !c) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    GemmArgs g{};
    g.a = a;
    g.lda = lda;
    g.b = b;
    g.ldb = ldb;
    g.m = m;
    g.n = n;
    g.k = k;
    g.c = c;
    g.ldc = ldc;
    return launched(launch_gemm_i32(g, stream));
}

i8mp_status i8mp_int8_mm_dequant(const int32_t* c, int64_t ldc, const float* row_absmax,
                                 const float* col_absmax, const void* bias, int64_t m, int64_t n,
                                 const void* x_out, int64_t ldo, const int32_t* idx,
                                 const int32_t* count, int32_t cap, const int8_t* b, int64_t ldb,
                                 int64_t k, void* out, int64_t ldout, hipStream_t stream) {
    if (m < 0 || n < 0 || ldc < n || ldout < n || cap < 0) return I8MP_EINVAL;
    const int outl = (x_out != nullptr) + (idx != nullptr) + (count != nullptr) + (b != nullptr);
    if (outl != 0 && outl != 4) return I8MP_EINVAL;
    if (outl == 4 && (ldo < cap || bad_k(k) || ldb < k)) return I8MP_EINVAL;
    if (outl == 4 && k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0 || n == 0) return I8MP_OK;
    if (!c || !row_absmax || !col_absmax || !out) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    DequantArgs d{};
    d.c = c;
    d.ldc = ldc;
    d.row_absmax = row_absmax;
    d.col_absmax = col_absmax;
    d.bias = static_cast<const half_bits*>(bias);
    d.m = m;
    d.n = n;
    d.x_out = outl ? static_cast<const half_bits*>(x_out) : nullptr;
    d.ldo = ldo;
    d.idx = idx;
    d.count = count;
    d.cap = cap;
    d.b = b;
    d.ldb = ldb;
    d.out = static_cast<half_bits*>(out);
    d.ldout = ldout;
    return launched(launch_dequant(d, stream));
}

i8mp_status i8mp_int8_vectorwise_dequant(const int8_t* q, int64_t ldq, int64_t m, int64_t k,
                                         const float* absmax, int32_t out_dtype, void* out, int64_t ldout,
                                         hipStream_t stream) {
    if (m < 0 || k < 0 || ldq < k || ldout < k || bad_ld(ldq) || bad_ld(ldout)) return I8MP_EINVAL;
    if (out_dtype != I8MP_DTYPE_F16 && out_dtype != I8MP_DTYPE_F32) return I8MP_EINVAL;
    if (m == 0 || k == 0) return I8MP_OK;
    if (!q || !absmax || !out) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    VecDequantArgs d{};
    d.q = q;
    d.ldq = ldq;
    d.m = m;
    d.k = k;
    d.absmax = absmax;
    d.out = out;
    d.ldout = ldout;
    d.half_out = out_dtype == I8MP_DTYPE_F16;
    return launched(launch_vectorwise_dequant(d, stream));
}

i8mp_status i8mp_linear_workspace_query(int64_t m, int64_t n, int64_t k, int32_t cap,
                                        i8mp_linear_workspace* layout) {
    if (!layout || m < 0 || n < 0 || bad_k(k) || cap < 0 || bad_ld(cap)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    forward_layout(m, k, cap, layout);
    return I8MP_OK;
}

namespace {

// Quantizer arguments writing codes, absmax, bitmap, index list, count and
// gathered outlier values of x into the forward workspace.
QuantArgs forward_quant_args(const void* x, int64_t m, int64_t k, int64_t ldx, float threshold, int32_t cap,
                             const i8mp_linear_workspace& L, char* ws) {
    QuantArgs a{};
    a.x = static_cast<const half_bits*>(x);
    a.m = m;
    a.k = k;
    a.ldx = ldx;
    a.threshold = threshold;
    a.partial = reinterpret_cast<uint32_t*>(ws + L.scratch_offset);
    a.words = ceil_div(k, 32);
    a.q = reinterpret_cast<int8_t*>(ws + L.q_offset);
    a.ldq = L.ldq;
    a.kpad = L.ldq;
    a.absmax = reinterpret_cast<float*>(ws + L.absmax_offset);
    a.bitmap_out = reinterpret_cast<uint32_t*>(ws + L.bitmap_offset);
    a.idx_out = reinterpret_cast<int32_t*>(ws + L.idx_offset);
    a.count_out = reinterpret_cast<int32_t*>(ws + L.count_offset);
    a.cap = cap;
    a.idx_len = (int32_t)L.idx_len;
    a.x_out = L.cap_pad > 0 ? reinterpret_cast<half_bits*>(ws + L.xo_offset) : nullptr;
    a.ldo = L.cap_pad;
    a.xo_cols = L.cap_pad;
    return a;
}

i8mp_status enqueue_quantize(const void* x, int64_t m, int64_t k, int64_t ldx, float threshold,
                             int32_t cap, const i8mp_linear_workspace& L, char* ws,
                             hipStream_t stream) {
    return launched(launch_quantize(forward_quant_args(x, m, k, ldx, threshold, cap, L, ws), stream));
}

// Arguments of the fused GEMM + dequant epilogue reading the forward workspace
// (and x itself for outlier slots past cap).
GemmArgs forward_gemm_args(const i8mp_linear_workspace& L, const char* ws, const void* x, int64_t ldx, int64_t m,
                           int64_t k, int32_t cap, const int8_t* w_q, int64_t ldw, const float* w_absmax, int64_t n,
                           const void* bias, void* out, int64_t ldout) {
    GemmArgs g{};
    g.a = reinterpret_cast<const int8_t*>(ws + L.q_offset);
    g.lda = L.ldq;
    g.a_zero_padded = true;
    g.b = w_q;
    g.ldb = ldw;
    g.m = m;
    g.n = n;
    g.k = k;
    g.row_absmax = reinterpret_cast<const float*>(ws + L.absmax_offset);
    g.col_absmax = w_absmax;
    g.bias = static_cast<const half_bits*>(bias);
    g.x_out = L.cap_pad > 0 ? reinterpret_cast<const half_bits*>(ws + L.xo_offset) : nullptr;
    g.ldo = L.cap_pad;
    g.idx = reinterpret_cast<const int32_t*>(ws + L.idx_offset);
    g.idx_len = (int32_t)L.idx_len;
    g.count = reinterpret_cast<const int32_t*>(ws + L.count_offset);
    g.cap = cap;
    g.x = static_cast<const half_bits*>(x);
    g.ldx = ldx;
    g.out = static_cast<half_bits*>(out);
    g.ldout = ldout;
    return g;
}

i8mp_status enqueue_matmul_dequant(const i8mp_linear_workspace& L, const char* ws, const void* x, int64_t ldx,
                                   int64_t m, int64_t k, int32_t cap, const int8_t* w_q, int64_t ldw,
                                   const float* w_absmax, int64_t n, const void* bias, void* out,
                                   int64_t ldout, hipStream_t stream) {
    return launched(launch_gemm_fused(
        forward_gemm_args(L, ws, x, ldx, m, k, cap, w_q, ldw, w_absmax, n, bias, out, ldout), stream));
}

}  // namespace

i8mp_status i8mp_linear_quantize(const void* x, int64_t m, int64_t k, int64_t ldx, float threshold,
                                 int32_t cap, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    if (m < 0 || bad_k(k) || ldx < k || cap < 0 || bad_ld(cap) || bad_ld(ldx)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0) return I8MP_OK;
    if (!x) return I8MP_EINVAL;
    i8mp_linear_workspace L;
    forward_layout(m, k, cap, &L);
    if (!workspace || workspace_bytes < L.bytes) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    return enqueue_quantize(x, m, k, ldx, threshold, cap, L, static_cast<char*>(workspace), stream);
}

i8mp_status i8mp_linear_matmul_dequant(const void* x, int64_t ldx, const void* workspace, size_t workspace_bytes,
                                       int64_t m, int64_t k, int32_t cap, const int8_t* w_q, int64_t ldw,
                                       const float* w_absmax, int64_t n, const void* bias, void* out,
                                       int64_t ldout, hipStream_t stream) {
    if (m < 0 || n < 0 || bad_k(k) || ldx < k || ldw < k || ldout < n || cap < 0) return I8MP_EINVAL;
    if (bad_ld(ldx) || bad_ld(ldw) || bad_ld(ldout) || bad_ld(cap)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0 || n == 0) return I8MP_OK;
    if (!x || !w_q || !w_absmax || !out) return I8MP_EINVAL;
    i8mp_linear_workspace L;
    forward_layout(m, k, cap, &L);
    if (!workspace || workspace_bytes < L.bytes) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    return enqueue_matmul_dequant(L, static_cast<const char*>(workspace), x, ldx, m, k, cap, w_q, ldw, w_absmax,
                                  n, bias, out, ldout, stream);
}

namespace {

// Checks shared by the forward entry points; I8MP_OK with *empty set when
// there is nothing to do.
i8mp_status check_forward_args(const void* x, int64_t m, int64_t k, int64_t ldx, const int8_t* w_q, int64_t ldw,
                               const float* w_absmax, int64_t n, int32_t cap, const void* out, int64_t ldout,
                               bool* empty) {
    *empty = false;
    if (m < 0 || n < 0 || bad_k(k) || ldx < k || ldw < k || ldout < n || cap < 0) return I8MP_EINVAL;
    if (bad_ld(ldx) || bad_ld(ldw) || bad_ld(ldout) || bad_ld(cap)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0 || n == 0) {
        *empty = true;
        return I8MP_OK;
    }
    if (!x || !w_q || !w_absmax || !out) return I8MP_EINVAL;
    return I8MP_OK;
}

// The forward's launches with its workspace at ws (layout L).
i8mp_status enqueue_forward(const void* x, int64_t m, int64_t k, int64_t ldx, const int8_t* w_q, int64_t ldw,
                            const float* w_absmax, int64_t n, const void* bias, float threshold, int32_t cap,
                            void* out, int64_t ldout, const i8mp_linear_workspace& L, char* ws,
                            hipStream_t stream) {
    // one or two rows: quantization inside the GEMV's workgroups, one launch
    const QuantArgs qa = forward_quant_args(x, m, k, ldx, threshold, cap, L, ws);
    const GemmArgs g = forward_gemm_args(L, ws, x, ldx, m, k, cap, w_q, ldw, w_absmax, n, bias, out, ldout);
    if (decode_forward_fits(qa, g)) return launched(launch_decode_forward(qa, g, stream));
    if (i8mp_status s = launched(launch_quantize(qa, stream)); s != I8MP_OK) return s;
    return launched(launch_gemm_fused(g, stream));
}

}  // namespace

i8mp_status i8mp_linear_forward(const void* x, int64_t m, int64_t k, int64_t ldx,
                                const int8_t* w_q, int64_t ldw, const float* w_absmax, int64_t n,
                                const void* bias, float threshold, int32_t cap, void* out,
                                int64_t ldout, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    bool empty = false;
    if (i8mp_status s = check_forward_args(x, m, k, ldx, w_q, ldw, w_absmax, n, cap, out, ldout, &empty);
        s != I8MP_OK || empty)
        return s;
    i8mp_linear_workspace L;
    forward_layout(m, k, cap, &L);
    if (!workspace || workspace_bytes < L.bytes) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    return enqueue_forward(x, m, k, ldx, w_q, ldw, w_absmax, n, bias, threshold, cap, out, ldout, L,
                           static_cast<char*>(workspace), stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The forward for callers that cannot allocate: its workspace is this
// file-scope device array, one per GPU, held until the process ends.  In host
// code the name `scratch` is a host-side stand-in, not device memory; the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device (with that device current) on the entry point's first call
// there, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[I8MP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of the scratch array.
i8mp_status scratch_on_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return I8MP_EDEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return I8MP_EDEVICE;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return I8MP_OK;
}

}  // namespace

extern "C" {

i8mp_status i8mp_linear_forward_noalloc(const void* x, int64_t m, int64_t k, int64_t ldx, const int8_t* w_q,
                                        int64_t ldw, const float* w_absmax, int64_t n, const void* bias,
                                        float threshold, int32_t cap, void* out, int64_t ldout,
                                        hipStream_t stream) {
    bool empty = false;
    if (i8mp_status s = check_forward_args(x, m, k, ldx, w_q, ldw, w_absmax, n, cap, out, ldout, &empty);
        s != I8MP_OK || empty)
        return s;
    i8mp_linear_workspace L;
    forward_layout(m, k, cap, &L);
    if (L.bytes > (size_t)I8MP_NOALLOC_SCRATCH_BYTES) return I8MP_ESCRATCH;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    void* ws = nullptr;
    if (i8mp_status s = scratch_on_current_device(&ws); s != I8MP_OK) return s;
    // every intermediate is written before it is read: nothing to clear
    return enqueue_forward(x, m, k, ldx, w_q, ldw, w_absmax, n, bias, threshold, cap, out, ldout, L,
                           static_cast<char*>(ws), stream);
}

size_t i8mp_colwise_quant_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 1) return 0;
    return colquant_scratch_bytes(rows, cols);
}

i8mp_status i8mp_int8_colwise_quant(const void* a, int64_t rows, int64_t cols, int64_t lda,
                                    const int32_t* zero_idx, const int32_t* zero_count, int32_t cap,
                                    int8_t* qt, int64_t ldqt, float* col_absmax, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    if (rows < 0 || cols < 0 || ldqt < rows || bad_ld(ldqt) || cap < 0) return I8MP_EINVAL;
    if (cols == 0) return I8MP_OK;
    if (lda < cols || !qt || !col_absmax || (rows > 0 && !a)) return I8MP_EINVAL;
    if (zero_idx && !zero_count) return I8MP_EINVAL;
    if (!workspace || workspace_bytes < colquant_scratch_bytes(rows, cols)) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    ColQuantArgs c{};
    c.x = static_cast<const half_bits*>(a);
    c.rows = rows;
    c.cols = cols;
    c.lda = lda;
    c.zero_idx = zero_idx;
    c.zero_count = zero_count;
    c.cap = cap;
    c.qt = qt;
    c.ldqt = ldqt;
    c.col_absmax = col_absmax;
    c.partial = static_cast<float*>(workspace);
    return launched(launch_colwise_quant(c, stream));
}

i8mp_status i8mp_linear_backward_workspace_query(int64_t m, int64_t n, int64_t k, int32_t cap,
                                                 i8mp_backward_workspace* layout) {
    if (!layout || m < 0 || n < 0 || bad_k(k) || cap < 0 || bad_ld(cap)) return I8MP_EINVAL;
    if (m > I8MP_MAX_K || n > I8MP_MAX_K) return I8MP_ERANGE;
    backward_layout(m, n, k, cap, layout);
    return I8MP_OK;
}

i8mp_status i8mp_linear_backward(const void* grad_out, int64_t ldg, const void* x, int64_t ldx,
                                 const void* w, int64_t ldw, int64_t m, int64_t n, int64_t k,
                                 int32_t cap, const void* fwd_workspace, size_t fwd_workspace_bytes,
                                 void* grad_x, int64_t ldgx, void* grad_w, int64_t ldgw,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (m < 0 || n < 0 || bad_k(k) || cap < 0 || bad_ld(cap) || ldg < n) return I8MP_EINVAL;
    if (grad_x && (ldw < k || ldgx < k || bad_ld(ldgx))) return I8MP_EINVAL;
    if (grad_w && (ldx < k || ldgw < k || bad_ld(ldgw))) return I8MP_EINVAL;
    if (m > I8MP_MAX_K || n > I8MP_MAX_K) return I8MP_ERANGE;
    const bool want_x = grad_x && m > 0;
    const bool want_w = grad_w && n > 0;
    if (!want_x && !want_w) return I8MP_OK;
    if (want_x && n > 0 && (!grad_out || !w)) return I8MP_EINVAL;
    if (want_w && m > 0 && (!grad_out || !x)) return I8MP_EINVAL;
    i8mp_backward_workspace L;
    backward_layout(m, n, k, cap, &L);
    if (!workspace || workspace_bytes < L.bytes) return I8MP_EWORKSPACE;
    i8mp_linear_workspace F;
    forward_layout(m, k, cap, &F);
    if (fwd_workspace && fwd_workspace_bytes < F.bytes) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    char* ws = static_cast<char*>(workspace);
    float* colmax = reinterpret_cast<float*>(ws + L.scratch_offset);
    const half_bits* g = static_cast<const half_bits*>(grad_out);

    if (want_x) {
        if (n == 0) {  // empty contraction
            if (i8mp_status s = launched(launch_fill_f16(static_cast<half_bits*>(grad_x), m, k, ldgx, stream));
                s != I8MP_OK)
                return s;
        } else {
            // g row-wise (threshold off), W column-wise (CBt), then the GEMM
            QuantArgs q{};
            q.x = g;
            q.m = m;
            q.k = n;
            q.ldx = ldg;
            q.threshold = 0.0f;
            q.words = ceil_div(n, 32);
            q.q = reinterpret_cast<int8_t*>(ws + L.gq_offset);
            q.ldq = L.ld_n;
            q.kpad = L.ld_n;
            q.absmax = reinterpret_cast<float*>(ws + L.gs_offset);
            if (i8mp_status s = launched(launch_quantize(q, stream)); s != I8MP_OK) return s;
            ColQuantArgs c{};
            c.x = static_cast<const half_bits*>(w);
            c.rows = n;
            c.cols = k;
            c.lda = ldw;
            c.qt = reinterpret_cast<int8_t*>(ws + L.wtq_offset);
            c.ldqt = L.ld_n;
            c.col_absmax = reinterpret_cast<float*>(ws + L.wts_offset);
            c.partial = colmax;
            if (i8mp_status s = launched(launch_colwise_quant(c, stream)); s != I8MP_OK) return s;
            GemmArgs G{};
            G.a = reinterpret_cast<const int8_t*>(ws + L.gq_offset);
            G.lda = L.ld_n;
            G.a_zero_padded = true;
            G.b = reinterpret_cast<const int8_t*>(ws + L.wtq_offset);
            G.ldb = L.ld_n;
            G.m = m;
            G.n = k;
            G.k = n;
            G.row_absmax = reinterpret_cast<const float*>(ws + L.gs_offset);
            G.col_absmax = reinterpret_cast<const float*>(ws + L.wts_offset);
            G.out = static_cast<half_bits*>(grad_x);
            G.ldout = ldgx;
            if (i8mp_status s = launched(launch_gemm_fused(G, stream)); s != I8MP_OK) return s;
        }
    }
    if (want_w) {
        if (m == 0) {  // empty contraction
            return launched(launch_fill_f16(static_cast<half_bits*>(grad_w), n, k, ldgw, stream));
        }
        const char* fws = static_cast<const char*>(fwd_workspace);
        // g and x column-wise, every outlier column of x zeroed (CAt), then
        // the GEMM; the pass over g also sums the fp16 outlier columns that
        // the forward gathered per row block, and the store after the GEMM
        // writes every outlier column of grad_w
        FixArgs f{};
        if (fws) {
            f.x_out = cap > 0 ? reinterpret_cast<const half_bits*>(fws + F.xo_offset) : nullptr;
            f.ldo = F.cap_pad;
            f.idx = reinterpret_cast<const int32_t*>(fws + F.idx_offset);
            f.idx_len = (int32_t)F.idx_len;
            f.count = reinterpret_cast<const int32_t*>(fws + F.count_offset);
            f.cap = cap;
            f.part = reinterpret_cast<float*>(ws + L.scratch_offset + (L.scratch_bytes - fix_part_bytes(m, n, cap)));
            f.grad_w = static_cast<half_bits*>(grad_w);
            f.ldgw = ldgw;
            f.g = g;
            f.ldg = ldg;
            f.x = static_cast<const half_bits*>(x);
            f.ldx = ldx;
        }
        ColQuantArgs c{};
        c.x = g;
        c.rows = m;
        c.cols = n;
        c.lda = ldg;
        c.qt = reinterpret_cast<int8_t*>(ws + L.gtq_offset);
        c.ldqt = L.ld_m;
        c.col_absmax = reinterpret_cast<float*>(ws + L.gts_offset);
        c.partial = colmax;
        c.fix = f;
        if (i8mp_status s = launched(launch_colwise_quant(c, stream)); s != I8MP_OK) return s;
        c.fix = FixArgs{};
        c.x = static_cast<const half_bits*>(x);
        c.cols = k;
        c.lda = ldx;
        c.zero_bitmap = fws ? reinterpret_cast<const uint32_t*>(fws + F.bitmap_offset) : nullptr;
        c.qt = reinterpret_cast<int8_t*>(ws + L.xtq_offset);
        c.col_absmax = reinterpret_cast<float*>(ws + L.xts_offset);
        if (i8mp_status s = launched(launch_colwise_quant(c, stream)); s != I8MP_OK) return s;
        GemmArgs G{};
        G.a = reinterpret_cast<const int8_t*>(ws + L.gtq_offset);
        G.lda = L.ld_m;
        G.a_zero_padded = true;
        G.b = reinterpret_cast<const int8_t*>(ws + L.xtq_offset);
        G.ldb = L.ld_m;
        G.m = n;
        G.n = k;
        G.k = m;
        G.row_absmax = reinterpret_cast<const float*>(ws + L.gts_offset);
        G.col_absmax = reinterpret_cast<const float*>(ws + L.xts_offset);
        G.out = static_cast<half_bits*>(grad_w);
        G.ldout = ldgw;
        if (i8mp_status s = launched(launch_gemm_fused(G, stream)); s != I8MP_OK) return s;
        if (i8mp_status s = launched(launch_outlier_store(f, m, n, stream)); s != I8MP_OK) return s;
    }
    return I8MP_OK;
}

namespace {
bool fp4_scales_ok(const float* absmax, const uint8_t* c8, const float* s2) {
    return absmax ? (!c8 && !s2) : (c8 && s2);
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
}  // namespace

i8mp_status i8mp_fp4_quantize(const void* w, int64_t n, int64_t k, int64_t ldw, uint8_t* codes, int64_t ldc,
                              float* absmax, hipStream_t stream) {
    if (n < 0 || k < 64 || k % 64 || ldw < k || ldc < k / 2) return I8MP_EINVAL;
    if (n == 0) return I8MP_OK;
    if (!w || !codes || !absmax) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    Fp4Args a{};
    a.w = static_cast<const half_bits*>(w);
    a.ldw = ldw;
    a.codes_out = codes;
    a.ldc = ldc;
    a.absmax_out = absmax;
    a.n = n;
    a.k = k;
    return launched(launch_fp4_quantize(a, stream));
}

i8mp_status i8mp_fp4_double_quant(const float* absmax, int64_t nb, uint8_t* c8, float* s2, hipStream_t stream) {
    if (nb < 0) return I8MP_EINVAL;
    if (nb == 0) return I8MP_OK;
    if (!absmax || !c8 || !s2) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    return launched(launch_fp4_double_quant(absmax, nb, c8, s2, stream));
}

i8mp_status i8mp_fp4_dequantize(const uint8_t* codes, int64_t ldc, int64_t n, int64_t k, const float* absmax,
                                const uint8_t* c8, const float* s2, int32_t out_dtype, void* out, int64_t ldout,
                                hipStream_t stream) {
    if (n < 0 || k < 64 || k % 64 || ldc < k / 2 || ldout < k) return I8MP_EINVAL;
    if (out_dtype != I8MP_DTYPE_F16 && out_dtype != I8MP_DTYPE_F32) return I8MP_EINVAL;
    if (n == 0) return I8MP_OK;
    if (!codes || !out || !fp4_scales_ok(absmax, c8, s2)) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    Fp4Args a{};
    a.codes = codes;
    a.ldc = ldc;
    a.absmax = absmax;
    a.c8 = c8;
    a.s2 = s2;
    a.out = out;
    a.ldout = ldout;
    a.half_out = out_dtype == I8MP_DTYPE_F16;
    a.n = n;
    a.k = k;
    return launched(launch_fp4_dequantize(a, stream));
}

i8mp_status i8mp_fp4_linear(const void* x, int64_t m, int64_t k, int64_t ldx, const uint8_t* codes, int64_t ldc,
                            const float* absmax, const uint8_t* c8, const float* s2, int64_t n, const void* bias,
                            void* out, int64_t ldout, hipStream_t stream) {
    if (m < 0 || n < 0 || k < 64 || k % 64 || ldx < k || ldx % 8 || ldc < k / 2 || ldc % 16 || ldout < n)
        return I8MP_EINVAL;
    if (m == 0 || n == 0) return I8MP_OK;
    if (!x || !codes || !out || !fp4_scales_ok(absmax, c8, s2)) return I8MP_EINVAL;
    if (!aligned16(x) || !aligned16(codes)) return I8MP_EINVAL;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    Fp4Args a{};
    a.x = static_cast<const half_bits*>(x);
    a.ldx = ldx;
    a.m = m;
    a.codes = codes;
    a.ldc = ldc;
    a.absmax = absmax;
    a.c8 = c8;
    a.s2 = s2;
    a.bias = static_cast<const half_bits*>(bias);
    a.out = out;
    a.ldout = ldout;
    a.n = n;
    a.k = k;
    return launched(launch_fp4_linear(a, stream));
}

}  // extern "C"

// extern "C" entry points of libi8mp.so: argument validation, workspace
// layout, launch sequencing.  Nothing here allocates, synchronizes or reads
// device memory; every launch goes to the caller's stream.
#include <atomic>
#include <cstring>

#include "common.h"

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
    size_t off = 0;
    L->scratch_offset = off;
    L->scratch_bytes = quant_scratch_bytes(k);
    off = align_up(off + L->scratch_bytes);
    L->bitmap_offset = off;
    off = align_up(off + (size_t)ceil_div(k, 32) * 4);
    L->idx_offset = off;
    off = align_up(off + (size_t)(L->cap_pad > 0 ? L->cap_pad : 1) * 4);
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
        default: return "unknown status";
    }
}

int32_t i8mp_abi_version(void) { return (2 << 16) | 0; }

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
    a.idx_len = L.cap_pad;
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

// Arguments of the fused GEMM + dequant epilogue reading the forward workspace.
GemmArgs forward_gemm_args(const i8mp_linear_workspace& L, const char* ws, int64_t m, int64_t k, int32_t cap,
                           const int8_t* w_q, int64_t ldw, const float* w_absmax, int64_t n,
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
    g.count = reinterpret_cast<const int32_t*>(ws + L.count_offset);
    g.cap = cap;
    g.out = static_cast<half_bits*>(out);
    g.ldout = ldout;
    return g;
}

i8mp_status enqueue_matmul_dequant(const i8mp_linear_workspace& L, const char* ws, int64_t m,
                                   int64_t k, int32_t cap, const int8_t* w_q, int64_t ldw,
                                   const float* w_absmax, int64_t n, const void* bias, void* out,
                                   int64_t ldout, hipStream_t stream) {
    return launched(launch_gemm_fused(
        forward_gemm_args(L, ws, m, k, cap, w_q, ldw, w_absmax, n, bias, out, ldout), stream));
}

}  // namespace

i8mp_status i8mp_linear_quantize(const void* x, int64_t m, int64_t k, int64_t ldx, float threshold,
                                 int32_t cap, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    if (m < 0 || bad_k(k) || ldx < k || cap < 0 || bad_ld(cap)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0) return I8MP_OK;
    if (!x) return I8MP_EINVAL;
    i8mp_linear_workspace L;
    forward_layout(m, k, cap, &L);
    if (!workspace || workspace_bytes < L.bytes) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    return enqueue_quantize(x, m, k, ldx, threshold, cap, L, static_cast<char*>(workspace), stream);
}

i8mp_status i8mp_linear_matmul_dequant(const void* workspace, size_t workspace_bytes, int64_t m,
                                       int64_t k, int32_t cap, const int8_t* w_q, int64_t ldw,
                                       const float* w_absmax, int64_t n, const void* bias, void* out,
                                       int64_t ldout, hipStream_t stream) {
    if (m < 0 || n < 0 || bad_k(k) || ldw < k || ldout < n || cap < 0) return I8MP_EINVAL;
    if (bad_ld(ldw) || bad_ld(ldout) || bad_ld(cap)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0 || n == 0) return I8MP_OK;
    if (!w_q || !w_absmax || !out) return I8MP_EINVAL;
    i8mp_linear_workspace L;
    forward_layout(m, k, cap, &L);
    if (!workspace || workspace_bytes < L.bytes) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    return enqueue_matmul_dequant(L, static_cast<const char*>(workspace), m, k, cap, w_q, ldw, w_absmax,
                                  n, bias, out, ldout, stream);
}

i8mp_status i8mp_linear_forward(const void* x, int64_t m, int64_t k, int64_t ldx,
                                const int8_t* w_q, int64_t ldw, const float* w_absmax, int64_t n,
                                const void* bias, float threshold, int32_t cap, void* out,
                                int64_t ldout, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    if (m < 0 || n < 0 || bad_k(k) || ldx < k || ldw < k || ldout < n || cap < 0) return I8MP_EINVAL;
    if (bad_ld(ldw) || bad_ld(ldout) || bad_ld(cap)) return I8MP_EINVAL;
    if (k > I8MP_MAX_K) return I8MP_ERANGE;
    if (m == 0 || n == 0) return I8MP_OK;
    if (!x || !w_q || !w_absmax || !out) return I8MP_EINVAL;
    i8mp_linear_workspace L;
    forward_layout(m, k, cap, &L);
    if (!workspace || workspace_bytes < L.bytes) return I8MP_EWORKSPACE;
    if (i8mp_status s = check_device(); s != I8MP_OK) return s;
    char* ws = static_cast<char*>(workspace);
    // one to four rows: quantization inside the GEMV's workgroups, one launch
    const QuantArgs qa = forward_quant_args(x, m, k, ldx, threshold, cap, L, ws);
    const GemmArgs g = forward_gemm_args(L, ws, m, k, cap, w_q, ldw, w_absmax, n, bias, out, ldout);
    if (decode_forward_fits(qa, g)) return launched(launch_decode_forward(qa, g, stream));
    if (i8mp_status s = launched(launch_quantize(qa, stream)); s != I8MP_OK) return s;
    return launched(launch_gemm_fused(g, stream));
}

}  // extern "C"

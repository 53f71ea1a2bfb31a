// api.cpp -- the C ABI of libw8a8 (declared in include/w8a8.h).
//
// Every argument is checked here, on the host, before anything is enqueued:
// a bad call returns a status and a per-thread message and never aborts
// (the review of "[Kernel] Add w8a8 CUTLASS kernels" asks that input
// validation never crash the caller and that dims and layout be checked,
// e.g. a B that is not column-major, the cause of its misaligned-address
// report). Nothing here allocates, frees or synchronises, so the calls can
// be captured into a HIP graph (the graph-capture failure reported on the
// same page).
#include <stdarg.h>
#include <stdio.h>

#include "../../include/w8a8.h"
#include "launch.hpp"

static_assert(W8A8_MAX_SHARDS == w8a8::kMaxShards, "shard limit of the C ABI and the kernels");

namespace {

thread_local char g_msg[512] = "";

w8a8_status fail(w8a8_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return s;
}

w8a8_status ok() {
    g_msg[0] = '\0';
    return W8A8_OK;
}

w8a8_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(W8A8_ERR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(w8a8_dtype t) { return t == W8A8_BF16 || t == W8A8_FP16 ? 2 : 4; }

bool valid_qtype(w8a8_qtype q) { return q == W8A8_Q_INT8 || q == W8A8_Q_FP8_E4M3FN; }

bool valid_in_dtype(w8a8_dtype t) { return t == W8A8_BF16 || t == W8A8_FP16 || t == W8A8_F32; }

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

// Shared checks of an [M, K] high-precision input and its [M, K] codes.
w8a8_status check_quant_io(const char* fn, const void* x, w8a8_dtype xt, int64_t M, int64_t K,
                           int64_t ldx, const void* q, w8a8_qtype qt, int64_t ldq) {
    if (!valid_in_dtype(xt)) return fail(W8A8_ERR_DTYPE, "%s: input type %d is not BF16, FP16 or F32", fn, xt);
    if (!valid_qtype(qt)) return fail(W8A8_ERR_DTYPE, "%s: code type %d is not INT8 or FP8_E4M3FN", fn, qt);
    if (M < 0 || K < 0) return fail(W8A8_ERR_SHAPE, "%s: negative size M=%lld K=%lld", fn, (long long)M, (long long)K);
    if (M > kMaxDim || K > kMaxDim) return fail(W8A8_ERR_UNSUPPORTED, "%s: M or K above 2^31-1", fn);
    if (ldx < K || ldq < K) return fail(W8A8_ERR_LAYOUT, "%s: leading dimensions ldx=%lld ldq=%lld must be >= K=%lld", fn, (long long)ldx, (long long)ldq, (long long)K);
    if (M == 0 || K == 0) return W8A8_OK;  // no element is read or written
    if (K % 16 || ldx % 16 || ldq % 16)
        return fail(W8A8_ERR_ALIGNMENT, "%s: K, ldx and ldq must be multiples of 16 (K=%lld ldx=%lld ldq=%lld)", fn, (long long)K, (long long)ldx, (long long)ldq);
    if (!x || !q) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL x or q", fn);
    if (!aligned16(x) || !aligned16(q)) return fail(W8A8_ERR_ALIGNMENT, "%s: x and q must be 16-byte aligned", fn);
    if (xt == W8A8_F32 && (reinterpret_cast<uintptr_t>(x) & 31u))
        return fail(W8A8_ERR_ALIGNMENT, "%s: float32 input must be 32-byte aligned", fn);
    const uint64_t units = static_cast<uint64_t>(M) * static_cast<uint64_t>((K + 2047) / 2048);
    if (units >= (uint64_t{1} << 31)) return fail(W8A8_ERR_UNSUPPORTED, "%s: tensor too large", fn);
    return W8A8_OK;
}

// Checks of a scaled product's arguments (host only, from the arguments).
static w8a8_status scaled_mm_check(const char* fn, void* out, w8a8_dtype ot, int64_t ldo,
                                   const void* a, int64_t lda, const void* b, int64_t ldb,
                                   w8a8_qtype qt, int64_t M, int64_t N, int64_t K,
                                   const float* a_scales, int64_t n_a, const float* b_scales,
                                   int64_t n_b) {
    if (!valid_qtype(qt)) return fail(W8A8_ERR_DTYPE, "%s: code type %d is not INT8 or FP8_E4M3FN", fn, qt);
    if (ot != W8A8_BF16 && ot != W8A8_FP16 && ot != W8A8_F32 && ot != W8A8_I32)
        return fail(W8A8_ERR_DTYPE, "%s: output type %d unknown", fn, ot);
    if (ot == W8A8_I32 && qt != W8A8_Q_INT8)
        return fail(W8A8_ERR_DTYPE, "%s: I32 output (raw accumulator) exists for int8 only", fn);
    if (ot == W8A8_I32 && (a_scales || b_scales))
        return fail(W8A8_ERR_INVALID_ARG, "%s: I32 output is the raw accumulator; scales must be NULL", fn);
    if (M < 0 || N < 0 || K < 0)
        return fail(W8A8_ERR_SHAPE, "%s: negative size M=%lld N=%lld K=%lld", fn, (long long)M, (long long)N, (long long)K);
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(W8A8_ERR_UNSUPPORTED, "%s: a size is above 2^31-1", fn);
    if (lda < K) return fail(W8A8_ERR_LAYOUT, "%s: lda=%lld < K=%lld", fn, (long long)lda, (long long)K);
    if (ldb < K)
        return fail(W8A8_ERR_LAYOUT, "%s: ldb=%lld < K=%lld: B must be K x N column-major (rows of an [N, K] weight)", fn, (long long)ldb, (long long)K);
    if (ldo < N) return fail(W8A8_ERR_LAYOUT, "%s: ldo=%lld < N=%lld", fn, (long long)ldo, (long long)N);
    if (a_scales && n_a != 1 && n_a != M)
        return fail(W8A8_ERR_SHAPE, "%s: a_scales has %lld entries; need 1 (per tensor) or M=%lld (per token)", fn, (long long)n_a, (long long)M);
    if (b_scales && n_b != 1 && n_b != N)
        return fail(W8A8_ERR_SHAPE, "%s: b_scales has %lld entries; need 1 (per tensor) or N=%lld (per channel)", fn, (long long)n_b, (long long)N);
    if (qt == W8A8_Q_INT8 && K > 131072)
        return fail(W8A8_ERR_UNSUPPORTED, "%s: int8 K=%lld could overflow the int32 accumulator (max 131072)", fn, (long long)K);
    if (K > 0 && (lda > (int64_t{1} << 23) || ldb > (int64_t{1} << 23)))
        return fail(W8A8_ERR_UNSUPPORTED, "%s: lda and ldb are limited to 2^23 bytes", fn);
    if (M == 0 || N == 0) return ok();
    if (!out) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL out", fn);
    if (K > 0 && (!a || !b)) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL a or b", fn);
    if (K % 16 || (K > 0 && (lda % 16 || ldb % 16)))
        return fail(W8A8_ERR_ALIGNMENT, "%s: K, lda and ldb must be multiples of 16 (K=%lld lda=%lld ldb=%lld)", fn, (long long)K, (long long)lda, (long long)ldb);
    if ((a && !aligned16(a)) || (b && !aligned16(b))) return fail(W8A8_ERR_ALIGNMENT, "%s: a and b must be 16-byte aligned", fn);
    if (reinterpret_cast<uintptr_t>(out) % elem_size(ot)) return fail(W8A8_ERR_ALIGNMENT, "%s: out is not aligned to its element size", fn);
    if ((a_scales && (reinterpret_cast<uintptr_t>(a_scales) & 3u)) || (b_scales && (reinterpret_cast<uintptr_t>(b_scales) & 3u)))
        return fail(W8A8_ERR_ALIGNMENT, "%s: scale arrays must be 4-byte aligned", fn);
    return ok();
}

static w8a8::GemmProblem make_problem(void* out, w8a8_dtype ot, int64_t ldo, const void* a,
                                      int64_t lda, const void* b, int64_t ldb, w8a8_qtype qt,
                                      int64_t M, int64_t N, int64_t K, const float* a_scales,
                                      int64_t n_a, const float* b_scales, int64_t n_b) {
    w8a8::GemmProblem p;
    p.out = out;
    p.ot = ot;
    p.ldo = ldo;
    p.a = static_cast<const uint8_t*>(a);
    p.lda = lda;
    p.b = static_cast<const uint8_t*>(b);
    p.ldb = ldb;
    p.qt = qt;
    p.M = M;
    p.N = N;
    p.K = K;
    p.sa = a_scales;
    p.sa_per_row = a_scales && n_a == M && M != 1;
    p.sb = b_scales;
    p.sb_per_col = b_scales && n_b == N && N != 1;
    return p;
}

static w8a8_status scaled_mm_impl(const char* fn, void* out, w8a8_dtype ot, int64_t ldo, const void* a,
                                  int64_t lda, const void* b, int64_t ldb, w8a8_qtype qt, int64_t M,
                                  int64_t N, int64_t K, const float* a_scales, int64_t n_a,
                                  const float* b_scales, int64_t n_b, hipStream_t stream) {
    w8a8_status s = scaled_mm_check(fn, out, ot, ldo, a, lda, b, ldb, qt, M, N, K, a_scales, n_a,
                                    b_scales, n_b);
    if (s != W8A8_OK || M == 0 || N == 0) return s;
    w8a8::GemmProblem p = make_problem(out, ot, ldo, a, lda, b, ldb, qt, M, N, K, a_scales, n_a,
                                       b_scales, n_b);
    return from_hip(w8a8::launch_scaled_mm(p, stream), fn);
}

}  // namespace

extern "C" {

const char* w8a8_version(void) { return "libw8a8 0.1 (gfx950)"; }

const char* w8a8_last_error(void) { return g_msg; }

const char* w8a8_status_string(w8a8_status s) {
    switch (s) {
        case W8A8_OK: return "W8A8_OK";
        case W8A8_ERR_INVALID_ARG: return "W8A8_ERR_INVALID_ARG";
        case W8A8_ERR_SHAPE: return "W8A8_ERR_SHAPE";
        case W8A8_ERR_LAYOUT: return "W8A8_ERR_LAYOUT";
        case W8A8_ERR_ALIGNMENT: return "W8A8_ERR_ALIGNMENT";
        case W8A8_ERR_DTYPE: return "W8A8_ERR_DTYPE";
        case W8A8_ERR_UNSUPPORTED: return "W8A8_ERR_UNSUPPORTED";
        case W8A8_ERR_HIP: return "W8A8_ERR_HIP";
    }
    return "W8A8_UNKNOWN_STATUS";
}

w8a8_status w8a8_quant_per_token(const void* x, w8a8_dtype xt, int64_t M, int64_t K, int64_t ldx,
                                 void* q, w8a8_qtype qt, int64_t ldq, float* scales,
                                 hipStream_t stream) {
    const char* fn = "w8a8_quant_per_token";
    w8a8_status s = check_quant_io(fn, x, xt, M, K, ldx, q, qt, ldq);
    if (s != W8A8_OK) return s;
    if (M == 0) return ok();
    if (!scales) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL scales", fn);
    if (reinterpret_cast<uintptr_t>(scales) & 3u) return fail(W8A8_ERR_ALIGNMENT, "%s: scales must be 4-byte aligned", fn);
    return from_hip(w8a8::launch_quant_per_token(xt, x, M, K, ldx, static_cast<uint8_t*>(q), qt, ldq, scales, stream), fn);
}

w8a8_status w8a8_quant_per_tensor(const void* x, w8a8_dtype xt, int64_t M, int64_t K, int64_t ldx,
                                  void* q, w8a8_qtype qt, int64_t ldq, float* scale, int dynamic,
                                  hipStream_t stream) {
    const char* fn = "w8a8_quant_per_tensor";
    if (dynamic != 0 && dynamic != 1) return fail(W8A8_ERR_INVALID_ARG, "%s: dynamic must be 0 or 1", fn);
    w8a8_status s = check_quant_io(fn, x, xt, M, K, ldx, q, qt, ldq);
    if (s != W8A8_OK) return s;
    if (dynamic && !scale) return fail(W8A8_ERR_INVALID_ARG, "%s: dynamic scaling needs a scale buffer", fn);
    if (scale && (reinterpret_cast<uintptr_t>(scale) & 3u)) return fail(W8A8_ERR_ALIGNMENT, "%s: scale must be 4-byte aligned", fn);
    if (M == 0 && !dynamic) return ok();
    return from_hip(w8a8::launch_quant_per_tensor(xt, x, M, K, ldx, static_cast<uint8_t*>(q), qt, ldq, scale, dynamic != 0, stream), fn);
}

w8a8_status w8a8_scaled_mm(void* out, w8a8_dtype ot, int64_t ldo, const void* a, int64_t lda,
                           const void* b, int64_t ldb, w8a8_qtype qt, int64_t M, int64_t N,
                           int64_t K, const float* a_scales, int64_t n_a, const float* b_scales,
                           int64_t n_b, hipStream_t stream) {
    return scaled_mm_impl("w8a8_scaled_mm", out, ot, ldo, a, lda, b, ldb, qt, M, N, K, a_scales, n_a,
                          b_scales, n_b, stream);
}

w8a8_status w8a8_quant_scaled_mm(void* out, w8a8_dtype ot, int64_t ldo, const void* x,
                                 w8a8_dtype xt, int64_t ldx, const void* b, int64_t ldb,
                                 w8a8_qtype qt, int64_t M, int64_t N, int64_t K,
                                 const float* b_scales, int64_t n_b, void* q, int64_t ldq,
                                 float* a_scales, hipStream_t stream) {
    const char* fn = "w8a8_quant_scaled_mm";
    if (ot == W8A8_I32) return fail(W8A8_ERR_DTYPE, "%s: the output is scaled: BF16, FP16 or F32", fn);
    w8a8_status s = check_quant_io(fn, x, xt, M, K, ldx, q, qt, ldq);
    if (s != W8A8_OK) return s;
    if (M > 0 && !a_scales) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL a_scales", fn);
    if (a_scales && (reinterpret_cast<uintptr_t>(a_scales) & 3u)) return fail(W8A8_ERR_ALIGNMENT, "%s: a_scales must be 4-byte aligned", fn);
    // The product's own checks, with the codes as A (a_scales per token).
    s = scaled_mm_check(fn, out, ot, ldo, q, ldq, b, ldb, qt, M, N, K, a_scales, M, b_scales, n_b);
    if (s != W8A8_OK) return s;
    if (M == 0) return ok();
    w8a8::GemmProblem p = make_problem(out, ot, ldo, q, ldq, b, ldb, qt, M, N, K, a_scales, M, b_scales, n_b);
    return from_hip(w8a8::launch_quant_scaled_mm(p, xt, x, ldx, static_cast<uint8_t*>(q), ldq, a_scales, stream), fn);
}

const char* w8a8_quant_scaled_mm_kernel(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return "";
    return w8a8::quant_scaled_mm_fused(M, N, K) ? "gemm_dynq_kernel" : "quant_rows_kernel+scaled_mm";
}

const char* w8a8_scaled_mm_kernel(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return "";
    return w8a8::scaled_mm_kernel_name(M, N, K, false);
}

const char* w8a8_scaled_mm_ws_kernel(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return "";
    return w8a8::scaled_mm_kernel_name(M, N, K, true);
}

int64_t w8a8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    return w8a8::plan_splitk(M, N, K).workspace_bytes;
}

w8a8_status w8a8_scaled_mm_ws(void* out, w8a8_dtype ot, int64_t ldo, const void* a, int64_t lda,
                              const void* b, int64_t ldb, w8a8_qtype qt, int64_t M, int64_t N,
                              int64_t K, const float* a_scales, int64_t n_a, const float* b_scales,
                              int64_t n_b, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream) {
    const char* fn = "w8a8_scaled_mm_ws";
    if (workspace_bytes < 0) return fail(W8A8_ERR_INVALID_ARG, "%s: negative workspace_bytes", fn);
    if (workspace_bytes > 0 && !workspace) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL workspace of %lld bytes", fn, (long long)workspace_bytes);
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return fail(W8A8_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", fn);
    w8a8_status s = scaled_mm_check(fn, out, ot, ldo, a, lda, b, ldb, qt, M, N, K, a_scales, n_a,
                                    b_scales, n_b);
    if (s != W8A8_OK || M == 0 || N == 0) return s;
    w8a8::GemmProblem p = make_problem(out, ot, ldo, a, lda, b, ldb, qt, M, N, K, a_scales, n_a,
                                       b_scales, n_b);
    p.workspace = workspace;
    p.workspace_bytes = workspace_bytes;
    return from_hip(w8a8::launch_scaled_mm(p, stream), fn);
}

w8a8_status w8a8_scaled_mm_noalloc(void* out, w8a8_dtype ot, int64_t ldo, const void* a,
                                   int64_t lda, const void* b, int64_t ldb, w8a8_qtype qt,
                                   int64_t M, int64_t N, int64_t K, const float* a_scales,
                                   int64_t n_a, const float* b_scales, int64_t n_b,
                                   hipStream_t stream) {
    const char* fn = "w8a8_scaled_mm_noalloc";
    w8a8_status s = scaled_mm_check(fn, out, ot, ldo, a, lda, b, ldb, qt, M, N, K, a_scales, n_a,
                                    b_scales, n_b);
    if (s != W8A8_OK || M == 0 || N == 0) return s;
    w8a8::GemmProblem p = make_problem(out, ot, ldo, a, lda, b, ldb, qt, M, N, K, a_scales, n_a,
                                       b_scales, n_b);
    int64_t needed = 0;
    const hipError_t e = w8a8::launch_scaled_mm_noalloc(p, stream, &needed);
    if (needed > 0)
        return fail(W8A8_ERR_UNSUPPORTED,
                    "%s: M=%lld N=%lld K=%lld needs %lld bytes of split-K scratch, the library "
                    "holds %lld", fn, (long long)M, (long long)N, (long long)K, (long long)needed,
                    (long long)w8a8::scaled_mm_noalloc_scratch_bytes());
    if (e == hipErrorInvalidDevice)
        return fail(W8A8_ERR_INVALID_ARG, "%s: the stream must belong to the current device (whose "
                    "scratch the call uses)", fn);
    return from_hip(e, fn);
}

w8a8_status kv_fp8_scaled_quant(const void* x, w8a8_dtype xt, int64_t n, uint8_t* q, float* scale,
                                int dynamic, hipStream_t stream) {
    const char* fn = "kv_fp8_scaled_quant";
    if (dynamic != 0 && dynamic != 1) return fail(W8A8_ERR_INVALID_ARG, "%s: dynamic must be 0 or 1", fn);
    if (n < 0) return fail(W8A8_ERR_SHAPE, "%s: negative n", fn);
    if (n % 16) return fail(W8A8_ERR_ALIGNMENT, "%s: n=%lld must be a multiple of 16", fn, (long long)n);
    // A flat tensor is one row of n elements.
    w8a8_status s = check_quant_io(fn, x, xt, n > 0 ? 1 : 0, n, n, q, W8A8_Q_FP8_E4M3FN, n);
    if (s != W8A8_OK) return s;
    if (dynamic && !scale) return fail(W8A8_ERR_INVALID_ARG, "%s: dynamic scaling needs a scale buffer", fn);
    if (scale && (reinterpret_cast<uintptr_t>(scale) & 3u)) return fail(W8A8_ERR_ALIGNMENT, "%s: scale must be 4-byte aligned", fn);
    if (n == 0 && !dynamic) return ok();
    return from_hip(w8a8::launch_quant_per_tensor(xt, x, n > 0 ? 1 : 0, n, n, q, W8A8_Q_FP8_E4M3FN, n, scale, dynamic != 0, stream), fn);
}

w8a8_status kv_fp8_scaled_dequant(const uint8_t* q, int64_t n, const float* scale, void* x,
                                  w8a8_dtype xt, hipStream_t stream) {
    const char* fn = "kv_fp8_scaled_dequant";
    if (!valid_in_dtype(xt)) return fail(W8A8_ERR_DTYPE, "%s: output type %d is not BF16, FP16 or F32", fn, xt);
    if (n < 0) return fail(W8A8_ERR_SHAPE, "%s: negative n", fn);
    if (n % 16) return fail(W8A8_ERR_ALIGNMENT, "%s: n=%lld must be a multiple of 16", fn, (long long)n);
    if (n == 0) return ok();
    if (!q || !x) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL q or x", fn);
    if (!aligned16(q) || !aligned16(x)) return fail(W8A8_ERR_ALIGNMENT, "%s: q and x must be 16-byte aligned", fn);
    if (scale && (reinterpret_cast<uintptr_t>(scale) & 3u)) return fail(W8A8_ERR_ALIGNMENT, "%s: scale must be 4-byte aligned", fn);
    return from_hip(w8a8::launch_kv_dequant(q, n, scale, x, xt, stream), fn);
}

w8a8_status w8a8_quant_per_token_azp(const void* x, w8a8_dtype xt, int64_t M, int64_t K, int64_t ldx,
                                     void* q, int64_t ldq, float* scales, int32_t* azp,
                                     hipStream_t stream) {
    const char* fn = "w8a8_quant_per_token_azp";
    w8a8_status s = check_quant_io(fn, x, xt, M, K, ldx, q, W8A8_Q_INT8, ldq);
    if (s != W8A8_OK || M == 0) return s;
    if (!scales || !azp) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL scales or azp", fn);
    if ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(azp)) & 3u)
        return fail(W8A8_ERR_ALIGNMENT, "%s: scales and azp must be 4-byte aligned", fn);
    return from_hip(w8a8::launch_quant_per_token_azp(xt, x, M, K, ldx, static_cast<uint8_t*>(q), ldq,
                                                     scales, azp, stream),
                    fn);
}

w8a8_status w8a8_quant_per_tensor_azp(const void* x, w8a8_dtype xt, int64_t M, int64_t K,
                                      int64_t ldx, void* q, int64_t ldq, float* scale,
                                      int32_t* azp, int dynamic, hipStream_t stream) {
    const char* fn = "w8a8_quant_per_tensor_azp";
    if (dynamic != 0 && dynamic != 1) return fail(W8A8_ERR_INVALID_ARG, "%s: dynamic must be 0 or 1", fn);
    w8a8_status s = check_quant_io(fn, x, xt, M, K, ldx, q, W8A8_Q_INT8, ldq);
    if (s != W8A8_OK) return s;
    if (dynamic && (!scale || !azp)) return fail(W8A8_ERR_INVALID_ARG, "%s: dynamic scaling needs scale and azp buffers", fn);
    if ((reinterpret_cast<uintptr_t>(scale) | reinterpret_cast<uintptr_t>(azp)) & 3u)
        return fail(W8A8_ERR_ALIGNMENT, "%s: scale and azp must be 4-byte aligned", fn);
    if (!dynamic && (M == 0 || K == 0)) return ok();
    return from_hip(w8a8::launch_quant_per_tensor_azp(xt, x, M, K, ldx, static_cast<uint8_t*>(q), ldq,
                                                      scale, azp, dynamic != 0, stream),
                    fn);
}

w8a8_status w8a8_colsum(const void* b, int64_t ldb, int64_t N, int64_t K, int32_t* colsum,
                        hipStream_t stream) {
    const char* fn = "w8a8_colsum";
    if (N < 0 || K < 0) return fail(W8A8_ERR_SHAPE, "%s: negative size N=%lld K=%lld", fn, (long long)N, (long long)K);
    if (N > kMaxDim || K > kMaxDim) return fail(W8A8_ERR_UNSUPPORTED, "%s: N or K above 2^31-1", fn);
    if (ldb < K) return fail(W8A8_ERR_LAYOUT, "%s: ldb=%lld < K=%lld", fn, (long long)ldb, (long long)K);
    if (K % 16 || ldb % 16) return fail(W8A8_ERR_ALIGNMENT, "%s: K and ldb must be multiples of 16", fn);
    if (N == 0) return ok();
    if (!colsum) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL colsum", fn);
    if (reinterpret_cast<uintptr_t>(colsum) & 3u) return fail(W8A8_ERR_ALIGNMENT, "%s: colsum must be 4-byte aligned", fn);
    if (K > 0 && !b) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL b", fn);
    if (b && !aligned16(b)) return fail(W8A8_ERR_ALIGNMENT, "%s: b must be 16-byte aligned", fn);
    return from_hip(w8a8::launch_colsum(static_cast<const uint8_t*>(b), ldb, N, K, colsum, stream), fn);
}

w8a8_status w8a8_scaled_mm_azp(void* out, w8a8_dtype ot, int64_t ldo, const void* a, int64_t lda,
                               const void* b, int64_t ldb, int64_t M, int64_t N, int64_t K,
                               const float* a_scales, int64_t n_a, const int32_t* azp, int64_t n_azp,
                               const int32_t* colsum, const float* b_scales, int64_t n_b,
                               hipStream_t stream) {
    const char* fn = "w8a8_scaled_mm_azp";
    w8a8_status s = scaled_mm_check(fn, out, ot, ldo, a, lda, b, ldb, W8A8_Q_INT8, M, N, K, a_scales,
                                    n_a, b_scales, n_b);
    if (s != W8A8_OK) return s;
    if (azp) {
        if (n_azp != 1 && n_azp != M)
            return fail(W8A8_ERR_SHAPE, "%s: azp has %lld entries; need 1 (per tensor) or M=%lld (per token)", fn, (long long)n_azp, (long long)M);
        if (!colsum) return fail(W8A8_ERR_INVALID_ARG, "%s: zero points need the weights' colsum", fn);
        if ((reinterpret_cast<uintptr_t>(azp) | reinterpret_cast<uintptr_t>(colsum)) & 3u)
            return fail(W8A8_ERR_ALIGNMENT, "%s: azp and colsum must be 4-byte aligned", fn);
        if (K > 65536)
            return fail(W8A8_ERR_UNSUPPORTED, "%s: K=%lld; with zero points the int32 accumulator holds K <= 65536", fn, (long long)K);
    }
    if (M == 0 || N == 0) return s;
    w8a8::GemmProblem p = make_problem(out, ot, ldo, a, lda, b, ldb, W8A8_Q_INT8, M, N, K, a_scales,
                                       n_a, b_scales, n_b);
    p.azp = azp;
    p.azp_per_row = azp && n_azp == M && M != 1;
    p.colsum = azp ? colsum : nullptr;
    return from_hip(w8a8::launch_scaled_mm(p, stream), fn);
}

static w8a8_status check_shards(const char* fn, const int64_t* rows, int64_t S, int64_t* N) {
    if (S < 1) return fail(W8A8_ERR_SHAPE, "%s: num_shards=%lld must be >= 1", fn, (long long)S);
    if (S > W8A8_MAX_SHARDS)
        return fail(W8A8_ERR_UNSUPPORTED, "%s: num_shards=%lld above %d", fn, (long long)S, W8A8_MAX_SHARDS);
    if (!rows) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL shard_rows", fn);
    int64_t n = 0;
    for (int64_t i = 0; i < S; ++i) {
        if (rows[i] < 0) return fail(W8A8_ERR_SHAPE, "%s: shard %lld has %lld rows", fn, (long long)i, (long long)rows[i]);
        n += rows[i];
        if (n > kMaxDim) return fail(W8A8_ERR_UNSUPPORTED, "%s: more than 2^31-1 rows", fn);
    }
    *N = n;
    return W8A8_OK;
}

w8a8_status w8a8_expand_shard_scales(const float* shard_scales, const int64_t* shard_rows,
                                     int64_t num_shards, float* b_scales, hipStream_t stream) {
    const char* fn = "w8a8_expand_shard_scales";
    int64_t N = 0;
    const w8a8_status e = check_shards(fn, shard_rows, num_shards, &N);
    if (e != W8A8_OK) return e;
    if (N == 0) return ok();
    if (!shard_scales || !b_scales) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL shard_scales or b_scales", fn);
    if ((reinterpret_cast<uintptr_t>(shard_scales) | reinterpret_cast<uintptr_t>(b_scales)) & 3u)
        return fail(W8A8_ERR_ALIGNMENT, "%s: scale arrays must be 4-byte aligned", fn);
    return from_hip(w8a8::launch_expand_shard_scales(shard_scales, shard_rows, num_shards, b_scales, stream), fn);
}

w8a8_status w8a8_requant_shared_scale(const void* w, int64_t ldw, w8a8_qtype qt, int64_t K,
                                      const int64_t* shard_rows, int64_t num_shards,
                                      const float* shard_scales, void* out, int64_t ldo,
                                      float* shared_scale, hipStream_t stream) {
    const char* fn = "w8a8_requant_shared_scale";
    if (!valid_qtype(qt)) return fail(W8A8_ERR_DTYPE, "%s: code type %d is not INT8 or FP8_E4M3FN", fn, qt);
    int64_t N = 0;
    const w8a8_status e = check_shards(fn, shard_rows, num_shards, &N);
    if (e != W8A8_OK) return e;
    if (K < 0) return fail(W8A8_ERR_SHAPE, "%s: negative K", fn);
    if (K > kMaxDim) return fail(W8A8_ERR_UNSUPPORTED, "%s: K above 2^31-1", fn);
    if (ldw < K || ldo < K)
        return fail(W8A8_ERR_LAYOUT, "%s: leading dimensions ldw=%lld ldo=%lld must be >= K=%lld", fn, (long long)ldw, (long long)ldo, (long long)K);
    if (K % 16 || ldw % 16 || ldo % 16)
        return fail(W8A8_ERR_ALIGNMENT, "%s: K, ldw and ldo must be multiples of 16", fn);
    if (!shard_scales || !shared_scale) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL shard_scales or shared_scale", fn);
    if ((reinterpret_cast<uintptr_t>(shard_scales) | reinterpret_cast<uintptr_t>(shared_scale)) & 3u)
        return fail(W8A8_ERR_ALIGNMENT, "%s: scale pointers must be 4-byte aligned", fn);
    if (N > 0 && K > 0) {
        if (!w || !out) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL w or out", fn);
        if (!aligned16(w) || !aligned16(out)) return fail(W8A8_ERR_ALIGNMENT, "%s: w and out must be 16-byte aligned", fn);
    }
    return from_hip(w8a8::launch_requant_shared_scale(static_cast<const uint8_t*>(w), ldw, qt, K, shard_rows,
                                                      num_shards, shard_scales, static_cast<uint8_t*>(out), ldo,
                                                      shared_scale, stream),
                    fn);
}

int64_t kv_fp8_attention_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seq_len) {
    // beyond the launch limits kv_fp8_decode_attention refuses the call (and
    // the product below could overflow)
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_seq_len < 0 || B > 65535 || Hq > 65535 || Hkv > 65535)
        return 0;
    const int splits = w8a8::attention_splits(B, Hkv, max_seq_len);
    return B * Hq * splits * (128 + 2) * 4;
}

namespace {

// The checks and arguments shared by the contiguous and the paged attention
// calls (everything but the row layout).
w8a8_status attention_common(const char* fn, void* out, const void* q, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t D, const uint8_t* k_cache,
                             const uint8_t* v_cache, int64_t rows, int64_t max_seq_len,
                             const float* k_scale, const float* v_scale, float sm_scale,
                             void* workspace, int64_t workspace_bytes, w8a8::AttnArgs& a) {
    if (B < 0 || Hq < 0 || Hkv < 0 || D < 0 || rows < 0 || max_seq_len < 0)
        return fail(W8A8_ERR_SHAPE, "%s: negative size", fn);
    if (B == 0 || Hq == 0) return ok();
    if (Hkv == 0 || Hq % Hkv) return fail(W8A8_ERR_SHAPE, "%s: Hq=%lld is not a multiple of Hkv=%lld", fn, (long long)Hq, (long long)Hkv);
    const int64_t G = Hq / Hkv;
    if (D != 128) return fail(W8A8_ERR_UNSUPPORTED, "%s: head dimension %lld (only 128)", fn, (long long)D);
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(W8A8_ERR_UNSUPPORTED, "%s: %lld query heads per KV head (1, 2, 4 or 8)", fn, (long long)G);
    if (B > 65535 || Hkv > 65535 || Hq > 65535 || max_seq_len > kMaxDim || rows > kMaxDim)
        return fail(W8A8_ERR_UNSUPPORTED, "%s: sizes beyond the launch limits", fn);
    if (!out || !q || !workspace) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL out, q or workspace", fn);
    if (rows > 0 && (!k_cache || !v_cache)) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL cache", fn);
    if (!aligned16(out) || !aligned16(q) || (k_cache && !aligned16(k_cache)) || (v_cache && !aligned16(v_cache)) ||
        !aligned16(workspace))
        return fail(W8A8_ERR_ALIGNMENT, "%s: out, q, caches and workspace must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3u)
        return fail(W8A8_ERR_ALIGNMENT, "%s: scales must be 4-byte aligned", fn);
    if (workspace_bytes < kv_fp8_attention_workspace_size(B, Hq, Hkv, max_seq_len))
        return fail(W8A8_ERR_INVALID_ARG, "%s: workspace of %lld bytes, %lld needed", fn, (long long)workspace_bytes,
                    (long long)kv_fp8_attention_workspace_size(B, Hq, Hkv, max_seq_len));
    a.out = static_cast<uint16_t*>(out);
    a.q = static_cast<const uint16_t*>(q);
    a.k = k_cache;
    a.v = v_cache;
    a.starts = nullptr;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.sm_scale = sm_scale != 0.0f ? sm_scale : 0.08838834764831845f;  // 1/sqrt(128)
    a.B = static_cast<int>(B);
    a.Hq = static_cast<int>(Hq);
    a.Hkv = static_cast<int>(Hkv);
    a.rows = rows;
    a.splits = w8a8::attention_splits(B, Hkv, max_seq_len);
    a.chunk = w8a8::attention_chunk(max_seq_len, a.splits);
    a.part = static_cast<float*>(workspace);
    return W8A8_OK;
}

}  // namespace

w8a8_status kv_fp8_decode_attention(void* out, const void* q, int64_t B, int64_t Hq, int64_t Hkv,
                                    int64_t D, const uint8_t* k_cache, const uint8_t* v_cache,
                                    int64_t rows, const int32_t* seq_starts, int64_t max_seq_len,
                                    const float* k_scale, const float* v_scale, float sm_scale,
                                    void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    const char* fn = "kv_fp8_decode_attention";
    w8a8::AttnArgs a;
    const w8a8_status s = attention_common(fn, out, q, B, Hq, Hkv, D, k_cache, v_cache, rows, max_seq_len,
                                           k_scale, v_scale, sm_scale, workspace, workspace_bytes, a);
    if (s != W8A8_OK || B == 0 || Hq == 0) return s;
    if (!seq_starts) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL seq_starts", fn);
    if (reinterpret_cast<uintptr_t>(seq_starts) & 3u) return fail(W8A8_ERR_ALIGNMENT, "%s: seq_starts must be 4-byte aligned", fn);
    a.starts = seq_starts;
    return from_hip(w8a8::launch_attention(a, stream), fn);
}

w8a8_status kv_fp8_paged_decode_attention(void* out, const void* q, int64_t B, int64_t Hq,
                                          int64_t Hkv, int64_t D, const uint8_t* k_cache,
                                          const uint8_t* v_cache, int64_t num_blocks,
                                          int64_t block_size, const int32_t* block_tables,
                                          int64_t table_stride, const int32_t* seq_lens,
                                          int64_t max_seq_len, const float* k_scale,
                                          const float* v_scale, float sm_scale, void* workspace,
                                          int64_t workspace_bytes, hipStream_t stream) {
    const char* fn = "kv_fp8_paged_decode_attention";
    if (num_blocks < 0 || table_stride < 0) return fail(W8A8_ERR_SHAPE, "%s: negative size", fn);
    if (block_size < 1 || block_size > 1024 || (block_size & (block_size - 1)))
        return fail(W8A8_ERR_UNSUPPORTED, "%s: block size %lld (a power of two, 1 .. 1024)", fn, (long long)block_size);
    if (num_blocks > kMaxDim / block_size) return fail(W8A8_ERR_UNSUPPORTED, "%s: cache beyond the launch limits", fn);
    w8a8::AttnArgs a;
    const w8a8_status s = attention_common(fn, out, q, B, Hq, Hkv, D, k_cache, v_cache, num_blocks * block_size,
                                           max_seq_len, k_scale, v_scale, sm_scale, workspace, workspace_bytes, a);
    if (s != W8A8_OK || B == 0 || Hq == 0) return s;
    if (!block_tables || !seq_lens) return fail(W8A8_ERR_INVALID_ARG, "%s: NULL block_tables or seq_lens", fn);
    if ((reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(seq_lens)) & 3u)
        return fail(W8A8_ERR_ALIGNMENT, "%s: block_tables and seq_lens must be 4-byte aligned", fn);
    if (table_stride * block_size < max_seq_len)
        return fail(W8A8_ERR_SHAPE, "%s: %lld table entries of %lld rows cannot cover max_seq_len %lld", fn,
                    (long long)table_stride, (long long)block_size, (long long)max_seq_len);
    if (table_stride > kMaxDim / B) return fail(W8A8_ERR_UNSUPPORTED, "%s: block table beyond the launch limits", fn);
    a.tables = block_tables;
    a.lens = seq_lens;
    a.table_stride = table_stride;
    a.bshift = __builtin_ctzll(static_cast<unsigned long long>(block_size));
    a.nblocks = num_blocks;
    return from_hip(w8a8::launch_attention(a, stream), fn);
}

}  // extern "C"

/*
 * oracle.c -- the plain, slow, CPU definition of the w8a8 scaled matrix
 * multiply and of the quantizers that feed it.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg do. It shares no code, header,
 * table or constant generator with the HIP library.
 *
 * What is computed, and where it is defined (the reference pages):
 *  - "[Kernel] Add w8a8 CUTLASS kernels" (vLLM issue/PR 4749), the bullet
 *    list of the PR description: D = a_scale * b_scale * (A_q . B_q) with
 *    symmetric int8 or fp8 e4m3 operands, activation scales per tensor or per
 *    token, weight scales per tensor or per output channel, bf16 or fp16
 *    output. The per_tensor_quantize snippet of the misaligned-address report
 *    on the same page fixes the quantisation recipe: divide by the scale,
 *    clamp to the e4m3 finite range, then cast.
 *  - "Enable scaled FP8 (e4m3fn) KV cache on ROCm" (vLLM issue 3290),
 *    "Scaling semantics": scale = absmax / 448 (the e4m3 max-norm),
 *    q = fp8_quant(x / scale), x' = fp8_dequant(q) * scale, per tensor; and
 *    the review answers on the same page: no scale given means scale 1.0.
 *  - "[Kernel] Add w8a8 CUTLASS kernels" again, its remark that the
 *    asymmetric int8 case needs small operations fused onto the GEMM: zero
 *    points per token or per tensor, the weights' code sums,
 *    D = s_a s_b (acc - z colsum) (the textbook asymmetric scheme).
 *  - "[Kernel] Support Fp8 Checkpoints (Dynamic + Static)" (vLLM PR 4332):
 *    merged layers (QKV, gate_up) whose shards carry their own weight
 *    scales; a review comment there proposes one shared scale max(s_i) with
 *    every shard rescaled by s_i / max(s_i).
 *
 * Readings taken where the pages are silent (listed with the reasons in the
 * design notes of the repository):
 *  - every float step is IEEE binary32 with round-to-nearest-even, including
 *    the division x / scale (a true division, not a reciprocal multiply);
 *  - int8 is symmetric: q = clamp(round_half_even(v), -127, 127);
 *  - absmax = 0 gives scale 1.0 (the pages' default scale);
 *  - NaN encodes to 0x7F (e4m3) and to 0 (int8); +-Inf saturate.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no fast-math: every double and
 * float operation below must be IEEE).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#define QT_INT8 0
#define QT_FP8 1

#define DT_BF16 0
#define DT_FP16 1
#define DT_F32 2
#define DT_I32 3
#define DT_F64 4

/* ---------------------------------------------------------------------- */
/* Rounding a non-negative double onto a binary floating-point grid.       */
/*                                                                          */
/* A format with p significand bits (the implicit one included) and        */
/* smallest normal exponent emin has, in the binade [2^E, 2^(E+1)), the    */
/* spacing 2^(E-p+1); below 2^emin the spacing stays 2^(emin-p+1)          */
/* (subnormals). The exponent is not bounded above here: the caller        */
/* decides what a result above the largest finite value means.             */
/* Rounding is to nearest, ties to the even multiple of the spacing.       */
/* ---------------------------------------------------------------------- */
static double round_to_grid(double a, int p, int emin) {
    if (a == 0.0) return 0.0;
    int e;
    frexp(a, &e);              /* a in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < emin) E = emin;
    double spacing = ldexp(1.0, E - (p - 1));
    /* a / spacing is exact (power-of-two scaling); nearbyint rounds ties to
       even in the default rounding mode. */
    return nearbyint(a / spacing) * spacing;
}

/* ---------------------------------------------------------------------- */
/* OCP fp8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3    */
/* mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448.   */
/* ---------------------------------------------------------------------- */
double oracle_e4m3_decode(uint8_t b) {
    int s = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9)            /* m/8 * 2^-6 */
                          : ldexp((double)(8 + m), e - 10); /* (1+m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* Clamp to [-448, 448], then round to nearest-even on the e4m3 grid. */
uint8_t oracle_e4m3_encode(float v) {
    if (isnan(v)) return 0x7F;
    double x = (double)v;
    if (x > 448.0) x = 448.0;
    if (x < -448.0) x = -448.0;
    int neg = signbit(x) ? 1 : 0;
    double r = round_to_grid(fabs(x), 4, -6);  /* r <= 448 since 448 is on the grid */
    uint8_t code;
    if (r == 0.0) {
        code = 0;
    } else {
        int e;
        frexp(r, &e);
        int E = e - 1;                          /* r in [2^E, 2^(E+1)) */
        if (E < -6) {                           /* subnormal: r = m * 2^-9 */
            code = (uint8_t)(r * 512.0);
        } else {                                /* r = (8 + m) * 2^(E-3) */
            int m = (int)(ldexp(r, 3 - E)) - 8;
            code = (uint8_t)(((E + 7) << 3) | m);
        }
    }
    return neg ? (uint8_t)(code | 0x80) : code;
}

/* Symmetric int8: round half to even, clamp to [-127, 127]. */
int8_t oracle_int8_encode(float v) {
    if (isnan(v)) return 0;
    double r = nearbyint((double)v);
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (int8_t)r;
}

/* ---------------------------------------------------------------------- */
/* bfloat16 (8 significand bits, emin -126) and IEEE half (11 bits, emin   */
/* -14): decode, and round-to-nearest-even from a double.                  */
/* ---------------------------------------------------------------------- */
float oracle_bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

double oracle_fp16_to_double(uint16_t h) {
    int s = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp((double)(1024 + m), e - 25);
    return s ? -mag : mag;
}

uint16_t oracle_bf16_from_double(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double r = round_to_grid(fabs(v), 8, -126);
    const double bf16_max = ldexp(255.0, 120);  /* (2 - 2^-7) * 2^127 */
    if (r > bf16_max) return (uint16_t)(sign | 0x7F80);
    float f = (float)r;                         /* exact: the bf16 grid is in the fp32 grid */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

uint16_t oracle_fp16_from_double(double v) {
    if (isnan(v)) return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double r = round_to_grid(fabs(v), 11, -14);
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00);
    uint16_t bits;
    if (r == 0.0) {
        bits = 0;
    } else {
        int e;
        frexp(r, &e);
        int E = e - 1;
        if (E < -14) {
            bits = (uint16_t)(r * 16777216.0);  /* r = m * 2^-24 */
        } else {
            int m = (int)(ldexp(r, 10 - E)) - 1024;
            bits = (uint16_t)(((E + 15) << 10) | m);
        }
    }
    return (uint16_t)(sign | bits);
}

/* ---------------------------------------------------------------------- */
/* Element access for the high-precision inputs.                            */
/* ---------------------------------------------------------------------- */
static float load_x(const void* x, int xtype, int64_t i) {
    if (xtype == DT_BF16) return oracle_bf16_to_float(((const uint16_t*)x)[i]);
    if (xtype == DT_FP16) return (float)oracle_fp16_to_double(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

static void store_x(void* x, int xtype, int64_t i, float v) {
    if (xtype == DT_BF16) ((uint16_t*)x)[i] = oracle_bf16_from_double((double)v);
    else if (xtype == DT_FP16) ((uint16_t*)x)[i] = oracle_fp16_from_double((double)v);
    else ((float*)x)[i] = v;
}

static float qmax_of(int qtype) { return qtype == QT_FP8 ? 448.0f : 127.0f; }

/* The scale of a group: absmax / Qmax in binary32; absmax 0 gives 1.0. */
float oracle_scale_from_absmax(float absmax, int qtype) {
    if (absmax == 0.0f) return 1.0f;
    return absmax / qmax_of(qtype);
}

/* One code: q = enc(fl32(x / s)). */
static uint8_t quant_one(float x, float s, int qtype) {
    float t = x / s;
    if (qtype == QT_FP8) return oracle_e4m3_encode(t);
    return (uint8_t)oracle_int8_encode(t);
}

/* Per-token (per-row) dynamic quantisation of x [M, K] (row stride ldx):
   scales[m] = absmax of row m / Qmax, q[m, k] = enc(x[m, k] / scales[m]).
   The same routine, run on a weight [N, K], gives per-output-channel
   weight quantisation. */
void oracle_quant_per_token(const void* x, int xtype, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, int qtype, int64_t ldq, float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(load_x(x, xtype, m * ldx + k));
            if (a > amax) amax = a;
        }
        float s = oracle_scale_from_absmax(amax, qtype);
        scales[m] = s;
        for (int64_t k = 0; k < K; ++k)
            q[m * ldq + k] = quant_one(load_x(x, xtype, m * ldx + k), s, qtype);
    }
}

/* Absmax over a whole [M, K] tensor. */
static float absmax_tensor(const void* x, int xtype, int64_t M, int64_t K, int64_t ldx) {
    float amax = 0.0f;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(load_x(x, xtype, m * ldx + k));
            if (a > amax) amax = a;
        }
    return amax;
}

/* Per-tensor quantisation. dynamic != 0: *scale is computed from the
   tensor's absmax and written. dynamic == 0: *scale is read (a static,
   calibrated scale); scale == NULL means 1.0. */
void oracle_quant_per_tensor(const void* x, int xtype, int64_t M, int64_t K, int64_t ldx,
                             uint8_t* q, int qtype, int64_t ldq, float* scale, int dynamic) {
    float s;
    if (dynamic) {
        s = oracle_scale_from_absmax(absmax_tensor(x, xtype, M, K, ldx), qtype);
        *scale = s;
    } else {
        s = scale ? *scale : 1.0f;
    }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            q[m * ldq + k] = quant_one(load_x(x, xtype, m * ldx + k), s, qtype);
}

/* Scaled fp8 KV cache, flat tensor of n elements, one scale per tensor. */
void oracle_kv_quant(const void* x, int xtype, int64_t n, uint8_t* q, float* scale, int dynamic) {
    oracle_quant_per_tensor(x, xtype, 1, n, n, q, QT_FP8, n, scale, dynamic);
}

/* x' = dequant(q) * scale in binary32, then rounded to the output type. */
void oracle_kv_dequant(const uint8_t* q, int64_t n, const float* scale, void* x, int xtype) {
    float s = scale ? *scale : 1.0f;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float d = (float)oracle_e4m3_decode(q[i]);   /* exact */
        store_x(x, xtype, i, d * s);
    }
}

/* ---------------------------------------------------------------------- */
/* Asymmetric int8 activations ("[Kernel] Add w8a8 CUTLASS kernels": the   */
/* asymmetric int8 case brings small operations to fuse onto the GEMM; the */
/* pages give no formula, so the textbook one is taken). Per row:          */
/*   lo = min(0, min_k x), hi = max(0, max_k x) (0 stays representable),  */
/*   s = fl32(hi - lo) / 255 in binary32 (1.0 when hi == lo, i.e. x == 0), */
/*   z = clamp(rint(fl32(-128 - fl32(lo / s))), -128, 127) (int32),       */
/*   q = clamp(rint(fl32(x / s)) + z, -128, 127),                          */
/* so that x ~ (q - z) * s. Every rint rounds half to even.                */
/* ---------------------------------------------------------------------- */
void oracle_quant_per_token_azp(const void* x, int xtype, int64_t M, int64_t K, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* scales, int32_t* azp) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = load_x(x, xtype, m * ldx + k);
            if (v > hi) hi = v;
            if (v < lo) lo = v;
        }
        const float d = hi - lo;
        const float s = d == 0.0f ? 1.0f : d / 255.0f;
        float zf = rintf(-128.0f - lo / s);
        if (zf < -128.0f) zf = -128.0f;
        if (zf > 127.0f) zf = 127.0f;
        scales[m] = s;
        azp[m] = (int32_t)zf;
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(load_x(x, xtype, m * ldx + k) / s) + zf;
            if (r < -128.0f) r = -128.0f;
            if (r > 127.0f) r = 127.0f;
            q[m * ldq + k] = (uint8_t)(int8_t)(int)r;
        }
    }
}

/* The same scheme with one scale and zero point for the whole tensor.     */
/* dynamic: lo and hi over every element (0 included), written to *scale   */
/* and *azp; static (calibrated): *scale and *azp are read (NULL: 1.0, 0). */
void oracle_quant_per_tensor_azp(const void* x, int xtype, int64_t M, int64_t K, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* scale, int32_t* azp,
                                 int dynamic) {
    float s = 1.0f, zf = 0.0f;
    if (dynamic) {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k) {
                float v = load_x(x, xtype, m * ldx + k);
                if (v > hi) hi = v;
                if (v < lo) lo = v;
            }
        const float d = hi - lo;
        s = d == 0.0f ? 1.0f : d / 255.0f;
        zf = rintf(-128.0f - lo / s);
        if (zf < -128.0f) zf = -128.0f;
        if (zf > 127.0f) zf = 127.0f;
        *scale = s;
        *azp = (int32_t)zf;
    } else {
        if (scale) s = *scale;
        if (azp) zf = (float)*azp;
    }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(load_x(x, xtype, m * ldx + k) / s) + zf;
            if (r < -128.0f) r = -128.0f;
            if (r > 127.0f) r = 127.0f;
            q[m * ldq + k] = (uint8_t)(int8_t)(int)r;
        }
}

/* Sum of each int8 weight row's codes, colsum[n] = sum_k b[n, k]. */
void oracle_colsum(const uint8_t* b, int64_t ldb, int64_t N, int64_t K, int32_t* out) {
    for (int64_t n = 0; n < N; ++n) {
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k) acc += (int8_t)b[n * ldb + k];
        out[n] = (int32_t)acc;
    }
}

/* The product with zero points: acc[m, n] = sum_k (a[m, k] - z[m or 0]) * b[n, k]
 * (exact in int64), then D = acc * a_scale * b_scale in fp64, rounded once
 * (DT_I32 stores acc itself). A NULL azp means zero points of 0. */
void oracle_scaled_mm_azp(void* out, int otype, int64_t ldo, const uint8_t* a, int64_t lda,
                          const uint8_t* b, int64_t ldb, int64_t M, int64_t N, int64_t K,
                          const float* sa, int64_t n_a, const int32_t* azp, int64_t n_azp,
                          const float* sb, int64_t n_b) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            const int64_t z = azp ? azp[n_azp == 1 ? 0 : m] : 0;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += ((int64_t)(int8_t)a[m * lda + k] - z) * (int64_t)(int8_t)b[n * ldb + k];
            if (otype == DT_I32) {
                ((int32_t*)out)[m * ldo + n] = (int32_t)acc;
                continue;
            }
            const double s_a = sa ? (double)sa[n_a == 1 ? 0 : m] : 1.0;
            const double s_b = sb ? (double)sb[n_b == 1 ? 0 : n] : 1.0;
            const double d = (double)acc * s_a * s_b;
            if (otype == DT_BF16) ((uint16_t*)out)[m * ldo + n] = oracle_bf16_from_double(d);
            else if (otype == DT_FP16) ((uint16_t*)out)[m * ldo + n] = oracle_fp16_from_double(d);
            else if (otype == DT_F64) ((double*)out)[m * ldo + n] = d;
            else ((float*)out)[m * ldo + n] = (float)d;
        }
}

/* ---------------------------------------------------------------------- */
/* Merged layers: a weight made of S shards stacked along N (QKV, gate_up), */
/* shard i holding n_i consecutive rows and its own per-tensor scale s_i    */
/* ("[Kernel] Support Fp8 Checkpoints (Dynamic + Static)": the loader must  */
/* handle merged layers whose shards do not share one weight scale).        */
/* ---------------------------------------------------------------------- */

/* Per-output-channel form of the shard scales: b_scales[n] = s_i for every
 * row n of shard i, so that one scaled product with per-channel weight
 * scales covers the whole merged layer. */
void oracle_expand_shard_scales(const float* shard_scales, const int64_t* rows, int64_t S,
                                float* out) {
    int64_t n = 0;
    for (int64_t i = 0; i < S; ++i)
        for (int64_t r = 0; r < rows[i]; ++r) out[n++] = shard_scales[i];
}

/* One shared scale (the review comment on the same page): s = max_i s_i,
 * and every code c of shard i is rescaled by the shard's ratio to it,
 * w' = (s_i / s) * w. Read literally, in binary32 with round-to-nearest-
 * even at each step: the ratio t_i = fl32(s_i / s) first, then the value
 * v = fl32(dec(c) * t_i), then the usual encode of v (saturating RNE for
 * e4m3, round-half-even and clamp to +-127 for int8). w is [N, K] with row
 * stride ldw (N = sum of rows), out likewise with stride ldo; *shared = s. */
void oracle_requant_shared_scale(const uint8_t* w, int64_t ldw, int qtype, int64_t K,
                                 const int64_t* rows, int64_t S, const float* shard_scales,
                                 uint8_t* out, int64_t ldo, float* shared) {
    float smax = shard_scales[0];
    for (int64_t i = 1; i < S; ++i)
        if (shard_scales[i] > smax) smax = shard_scales[i];
    *shared = smax;
    int64_t n0 = 0;
    for (int64_t i = 0; i < S; ++i) {
        const float t = shard_scales[i] / smax;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows[i]; ++r)
            for (int64_t k = 0; k < K; ++k) {
                const uint8_t c = w[(n0 + r) * ldw + k];
                const float d = qtype == QT_FP8 ? (float)oracle_e4m3_decode(c) : (float)(int8_t)c;
                const float v = d * t;
                out[(n0 + r) * ldo + k] =
                    qtype == QT_FP8 ? oracle_e4m3_encode(v) : (uint8_t)oracle_int8_encode(v);
            }
        n0 += rows[i];
    }
}

/* ---------------------------------------------------------------------- */
/* The scaled matrix multiply.                                              */
/*                                                                          */
/* a: codes [M, K], row stride lda. b: codes [N, K], row stride ldb (the   */
/* bytes of a K x N column-major matrix). acc[m, n] = sum_k a[m,k] b[n,k]   */
/* is exact: int32 for int8 (|acc| <= 127^2 K < 2^31 for K < 133,144), an  */
/* fp64 sum for e4m3 (every product is a multiple of 2^-18 below 2^18, so  */
/* the sum stays exact while K < 2^17).                                     */
/* D[m, n] = acc * a_scale[m or 0] * b_scale[n or 0] in fp64, then rounded */
/* once to bf16 or fp16. A NULL scale array means 1.0.                     */
/* otype DT_F32 stores the fp64 value rounded to binary32, DT_F64 the fp64 */
/* value itself; DT_I32 (int8 only) stores the raw accumulator.            */
/* ---------------------------------------------------------------------- */
static void mm_one(void* out, int otype, int64_t ldo, int64_t orow, const uint8_t* a, int64_t lda,
                   const uint8_t* b, int64_t ldb, int qtype, int64_t m, int64_t n, int64_t K,
                   const float* sa, int64_t n_a, const float* sb, int64_t n_b) {
    double acc;
    int64_t iacc = 0;
    if (qtype == QT_INT8) {
        const int8_t* ar = (const int8_t*)(a + m * lda);
        const int8_t* br = (const int8_t*)(b + n * ldb);
        for (int64_t k = 0; k < K; ++k) iacc += (int64_t)ar[k] * (int64_t)br[k];
        acc = (double)iacc;
    } else {
        const uint8_t* ar = a + m * lda;
        const uint8_t* br = b + n * ldb;
        acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += oracle_e4m3_decode(ar[k]) * oracle_e4m3_decode(br[k]);
    }
    if (otype == DT_I32) {
        ((int32_t*)out)[orow * ldo + n] = (int32_t)iacc;
        return;
    }
    double s_a = sa ? (double)sa[n_a == 1 ? 0 : m] : 1.0;
    double s_b = sb ? (double)sb[n_b == 1 ? 0 : n] : 1.0;
    double d = acc * s_a * s_b;
    if (otype == DT_BF16) ((uint16_t*)out)[orow * ldo + n] = oracle_bf16_from_double(d);
    else if (otype == DT_FP16) ((uint16_t*)out)[orow * ldo + n] = oracle_fp16_from_double(d);
    else if (otype == DT_F64) ((double*)out)[orow * ldo + n] = d;
    else ((float*)out)[orow * ldo + n] = (float)d;
}

void oracle_scaled_mm(void* out, int otype, int64_t ldo, const uint8_t* a, int64_t lda,
                      const uint8_t* b, int64_t ldb, int qtype, int64_t M, int64_t N, int64_t K,
                      const float* sa, int64_t n_a, const float* sb, int64_t n_b) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            mm_one(out, otype, ldo, m, a, lda, b, ldb, qtype, m, n, K, sa, n_a, sb, n_b);
}

/* The same definition evaluated only on the rows listed in rows[0..nrows):
   output row i of out holds row rows[i] of D. */
void oracle_scaled_mm_rows(void* out, int otype, int64_t ldo, const int64_t* rows, int64_t nrows,
                           const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int qtype,
                           int64_t N, int64_t K, const float* sa, int64_t n_a,
                           const float* sb, int64_t n_b) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < nrows; ++i)
        for (int64_t n = 0; n < N; ++n)
            mm_one(out, otype, ldo, i, a, lda, b, ldb, qtype, rows[i], n, K, sa, n_a, sb, n_b);
}

/* Threads the OpenMP loops above use. */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Vector helpers for the tests. */
void oracle_e4m3_encode_n(const float* v, int64_t n, uint8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) q[i] = oracle_e4m3_encode(v[i]);
}
void oracle_int8_encode_n(const float* v, int64_t n, int8_t* q) {
    for (int64_t i = 0; i < n; ++i) q[i] = oracle_int8_encode(v[i]);
}
void oracle_e4m3_decode_n(const uint8_t* q, int64_t n, double* v) {
    for (int64_t i = 0; i < n; ++i) v[i] = oracle_e4m3_decode(q[i]);
}
void oracle_bf16_from_double_n(const double* v, int64_t n, uint16_t* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = oracle_bf16_from_double(v[i]);
}
void oracle_fp16_from_double_n(const double* v, int64_t n, uint16_t* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = oracle_fp16_from_double(v[i]);
}

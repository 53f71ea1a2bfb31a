/*
 * w8a8.h -- C ABI of libw8a8: the w8a8 scaled matrix multiply for MI355X
 * (gfx950) and the quantizers that feed it.
 *
 * Definitions come from the reference pages:
 *  [P1] "[Kernel] Add w8a8 CUTLASS kernels" (vLLM issue/PR 4749): the
 *       PR description's bullet list (symmetric int8 / fp8 e4m3 operands,
 *       per-tensor or per-token activation scales, per-tensor or
 *       per-output-channel weight scales, bf16 or fp16 output); the
 *       misaligned-address report (B must be column-major, the
 *       per_tensor_quantize recipe: divide, clamp, cast); the review
 *       comments (check dims and layout, never crash on bad input,
 *       submatrices with leading-dimension strides are allowed, the op must
 *       work under graph capture).
 *  [P2] "[Kernel] Support Fp8 Checkpoints (Dynamic + Static)" (vLLM PR
 *       4332): static (calibrated) and dynamic activation scales.
 *  [P3] "Enable scaled FP8 (e4m3fn) KV cache on ROCm" (vLLM issue 3290),
 *       "Scaling semantics": scale = absmax / 448, q = fp8(x / scale),
 *       x' = fp8_dequant(q) * scale; and its review answers: no scale means
 *       scale 1.0.
 *
 * Conventions shared by every call
 *  - All data pointers are DEVICE pointers on the current HIP device; scale
 *    arrays are device float32 arrays. The caller owns and allocates every
 *    buffer. The library never allocates, frees or synchronises, and keeps no
 *    global state (besides the static device array that w8a8_scaled_mm_noalloc
 *    uses instead of a workspace), so each call can be captured into a HIP
 *    graph. Work is enqueued on `stream` (0 = the null stream) and runs
 *    asynchronously.
 *  - Inputs are validated on the host from the arguments alone (device data
 *    is never read). A bad argument returns an error status and never aborts
 *    the process; w8a8_last_error() then holds a message (per thread).
 *    Faults inside a kernel surface asynchronously, at a later HIP call.
 *  - Matrices are row-major with a leading dimension (row stride, in
 *    elements) >= the row length, so submatrices are accepted. Rows must be
 *    16-byte aligned: data pointers 16-byte aligned, K and every leading
 *    dimension a multiple of 16 (W8A8_ERR_ALIGNMENT otherwise).
 *  - e4m3fn is the OCP fp8 E4M3 format (max 448, no infinities, 0x7F/0xFF
 *    NaN). Quantisation is q = enc(x / s) with an IEEE binary32 division and
 *    round-to-nearest-even; fp8 saturates at +-448 (NaN -> 0x7F), int8 is
 *    symmetric, clamp(round_half_even(.), -127, 127) (NaN -> 0).
 *  - A dynamic scale is absmax / Qmax with Qmax = 448 (fp8) or 127 (int8),
 *    computed in binary32; an all-zero group gets scale 1.0.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w8a8_status {
    W8A8_OK = 0,
    W8A8_ERR_INVALID_ARG = 1, /* NULL pointer, bad flag, scales where none are allowed */
    W8A8_ERR_SHAPE = 2,       /* negative or incompatible sizes, bad scale length */
    W8A8_ERR_LAYOUT = 3,      /* leading dimension smaller than the row (e.g. B not column-major) */
    W8A8_ERR_ALIGNMENT = 4,   /* pointer, K or leading dimension not 16-byte aligned */
    W8A8_ERR_DTYPE = 5,       /* unknown or unsupported element type combination */
    W8A8_ERR_UNSUPPORTED = 6, /* valid request outside what the kernels handle (e.g. int8 K > 131072) */
    W8A8_ERR_HIP = 7          /* a HIP runtime call (launch) failed */
} w8a8_status;

/* 8-bit code type of quantised operands. */
typedef enum w8a8_qtype {
    W8A8_Q_INT8 = 0,        /* symmetric int8, codes -127..127 */
    W8A8_Q_FP8_E4M3FN = 1,  /* OCP fp8 E4M3 */
    /* Range markers, never valid arguments: they give the type the range of
     * a 32-bit int, so that any int a caller passes is a value of the type
     * and is rejected by the validation (W8A8_ERR_DTYPE). Without them a
     * C++ compiler may take the type to hold only 0 and 1. */
    W8A8_QTYPE_RANGE_MIN = -2147483647 - 1,
    W8A8_QTYPE_RANGE_MAX = 2147483647
} w8a8_qtype;

/* Element type of high-precision tensors (inputs of quantizers, outputs). */
typedef enum w8a8_dtype {
    W8A8_BF16 = 0,
    W8A8_FP16 = 1,
    W8A8_F32 = 2,   /* float32 */
    W8A8_I32 = 3,   /* int32: raw int8 accumulator output of w8a8_scaled_mm only */
    /* Range markers, never valid arguments (as for w8a8_qtype). */
    W8A8_DTYPE_RANGE_MIN = -2147483647 - 1,
    W8A8_DTYPE_RANGE_MAX = 2147483647
} w8a8_dtype;

/*
 * Dynamic per-token quantisation [P1 bullet list: per-token activations;
 * P2: dynamic activation scales; scale rule of P3 "Scaling semantics"].
 * For each row m of x [M, K] (row stride ldx elements, type xt in
 * BF16/FP16/F32): scales[m] = absmax(x[m, :]) / Qmax (1.0 if the row is all
 * zeros), q[m, k] = enc(x[m, k] / scales[m]) with row stride ldq bytes.
 * Run on a weight [N, K] it gives per-output-channel weight quantisation.
 * q: device, M*ldq bytes. scales: device float32 [M], written.
 * M == 0 is a no-op. K == 0 writes scales of 1.0.
 */
w8a8_status w8a8_quant_per_token(const void* x, w8a8_dtype xt, int64_t M, int64_t K, int64_t ldx,
                                 void* q, w8a8_qtype qt, int64_t ldq, float* scales,
                                 hipStream_t stream);

/*
 * Per-tensor quantisation [P1 per_tensor_quantize recipe; P2 static
 * act_scale and dynamic per-tensor scaling; P3 scale rule].
 * dynamic == 0 (static, calibrated): s = *scale (scale == NULL means 1.0,
 *   the pages' default); *scale is not written.
 * dynamic == 1: s = absmax(x) / Qmax is computed and written to *scale
 *   (scale must not be NULL). This takes three kernels on `stream`; until the
 *   last one ends, the last (at most 4 KB of) codes of q hold intermediate
 *   values (partial maxima).
 * q[m, k] = enc(x[m, k] / s), row strides ldx (elements) and ldq (bytes).
 */
w8a8_status w8a8_quant_per_tensor(const void* x, w8a8_dtype xt, int64_t M, int64_t K, int64_t ldx,
                                  void* q, w8a8_qtype qt, int64_t ldq, float* scale, int dynamic,
                                  hipStream_t stream);

/*
 * The scaled matrix multiply [P1: cutlass_scaled_mm_dq, its bullet list and
 * the layout rule from the misaligned-address report]:
 *   D[m, n] = a_scale[m or 0] * b_scale[n or 0] * sum_k A[m, k] * B[k, n]
 * A: codes [M, K] row-major, row stride lda bytes.
 * B: codes K x N COLUMN-major, i.e. the bytes of a row-major [N, K] weight
 *    (row n = output channel n), column stride ldb bytes (ldb >= K; a
 *    smaller ldb means B is not column-major: W8A8_ERR_LAYOUT).
 * A and B share the code type qt. Accumulation is int32 (exact) for int8 and
 * float32 for fp8.
 * a_scales: device float32, n_a == 1 (per tensor) or n_a == M (per token).
 * b_scales: device float32, n_b == 1 (per tensor) or n_b == N (per channel).
 * A NULL scale array means 1.0 (n_a / n_b are then ignored).
 * out: [M, N] row-major, row stride ldo elements, type ot:
 *   BF16 / FP16: the scaled result, rounded to nearest even;
 *   F32: the scaled result in float32;
 *   I32: the raw int32 accumulator (int8 only; both scale arrays must be NULL).
 * M == 0 or N == 0 is a no-op; K == 0 writes zeros.
 */
w8a8_status w8a8_scaled_mm(void* out, w8a8_dtype ot, int64_t ldo, const void* a, int64_t lda,
                           const void* b, int64_t ldb, w8a8_qtype qt, int64_t M, int64_t N,
                           int64_t K, const float* a_scales, int64_t n_a, const float* b_scales,
                           int64_t n_b, hipStream_t stream);

/*
 * Bytes of device workspace with which w8a8_scaled_mm_ws splits K for an
 * M x N x K problem (0: it would not split, and needs none). Host-only.
 * Splitting pays for decode problems with 16 < M <= 64 on weights too
 * narrow to occupy the GPU: K >= 8192 and N < 16321, or K >= 4096 and
 * N <= 1024. Up to 4 splits of fp32 (int32 for int8) partial sums, at most
 * 16*M*N bytes.
 */
int64_t w8a8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * w8a8_scaled_mm with an optional caller workspace [P1: the same operation].
 * When workspace_bytes >= w8a8_scaled_mm_workspace_size(M, N, K) > 0, two to
 * four workgroups share each column block along K (four per 16 columns on
 * weights of at most 2048 rows; on wider ones as many per 64 columns as
 * fill one round of the GPU's workgroup slots), write their partial sums to
 * the workspace, and a second kernel adds them in a fixed split order and
 * applies the scales: results are deterministic, and equal to
 * w8a8_scaled_mm's up to the fp8 summation order (bit-identical for int8).
 * Otherwise this is w8a8_scaled_mm. The workspace needs no initialisation
 * and holds nothing between calls; calls that share one must not overlap.
 * workspace: device memory, 256-byte aligned (may be NULL with 0 bytes).
 */
w8a8_status w8a8_scaled_mm_ws(void* out, w8a8_dtype ot, int64_t ldo, const void* a, int64_t lda,
                              const void* b, int64_t ldb, w8a8_qtype qt, int64_t M, int64_t N,
                              int64_t K, const float* a_scales, int64_t n_a, const float* b_scales,
                              int64_t n_b, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream);

/*
 * w8a8_scaled_mm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc. Same operation, arguments and results as w8a8_scaled_mm_ws
 * given a large enough workspace, with the split-K partial sums kept in a
 * static device array of the library (16 MiB, held on each GPU the library
 * runs on until the process ends) instead of a caller workspace. The call
 * allocates and frees nothing and does not synchronise. Every split plan
 * fits the array; a problem that needed more would be refused with
 * W8A8_ERR_UNSUPPORTED. Calls share the current device's array: calls that
 * overlap on one GPU (several streams or threads at once) race on it, so the
 * caller orders them; the array needs no clearing between calls (every
 * partial sum read was written by the same call). `stream` must belong to
 * the current device (else W8A8_ERR_INVALID_ARG).
 */
w8a8_status w8a8_scaled_mm_noalloc(void* out, w8a8_dtype ot, int64_t ldo, const void* a,
                                   int64_t lda, const void* b, int64_t ldb, w8a8_qtype qt,
                                   int64_t M, int64_t N, int64_t K, const float* a_scales,
                                   int64_t n_a, const float* b_scales, int64_t n_b,
                                   hipStream_t stream);

/*
 * Dynamic per-token quantisation followed by the scaled matrix multiply, the
 * decode step of a w8a8 linear layer [P1 bullet list: per-token activation
 * scales with per-channel weight scales; P2: dynamic activation scales]:
 *   w8a8_quant_per_token(x -> q, a_scales), then
 *   w8a8_scaled_mm(out, q, B, a_scales (per token), b_scales).
 * Same arguments and rules as those two calls: x [M, K] (row stride ldx
 * elements, type xt in BF16/FP16/F32), q [M, ldq] codes and a_scales [M]
 * (device, written: the caller can reuse them), B and b_scales as in
 * w8a8_scaled_mm, out of type BF16/FP16/F32 (I32 is refused). Results are
 * identical to the two calls (codes and scales bit for bit, out up to the
 * fp8 accumulation order). M == 1 with K <= 15360 and N < 16321 runs as one
 * kernel that quantises the row in every workgroup; other sizes run the two
 * kernels (w8a8_quant_scaled_mm_kernel names which).
 */
w8a8_status w8a8_quant_scaled_mm(void* out, w8a8_dtype ot, int64_t ldo, const void* x,
                                 w8a8_dtype xt, int64_t ldx, const void* b, int64_t ldb,
                                 w8a8_qtype qt, int64_t M, int64_t N, int64_t K,
                                 const float* b_scales, int64_t n_b, void* q, int64_t ldq,
                                 float* a_scales, hipStream_t stream);

/*
 * Scaled fp8 KV-cache quantisation of one flat, contiguous tensor of n
 * elements (e.g. one layer's K or V cache) [P3 "Scaling semantics": per
 * tensor scale = absmax / 448, q = fp8(x / scale)].
 * dynamic == 1: *scale = absmax / 448 is computed and written (as in
 * w8a8_quant_per_tensor, three kernels, the tail of q holding intermediate
 * values until the last ends). dynamic == 0: the given *scale is used
 * (NULL: 1.0).
 * q: device, n bytes of e4m3fn codes. n must be a multiple of 16.
 */
w8a8_status kv_fp8_scaled_quant(const void* x, w8a8_dtype xt, int64_t n, uint8_t* q, float* scale,
                                int dynamic, hipStream_t stream);

/*
 * Scaled fp8 KV-cache dequantisation [P3: x' = fp8_dequant(q) * scale]:
 * x[i] = round(e4m3_value(q[i]) * s) with the product in float32, then
 * rounded to nearest even into xt (BF16/FP16/F32). s = *scale, NULL: 1.0.
 * n must be a multiple of 16.
 */
w8a8_status kv_fp8_scaled_dequant(const uint8_t* q, int64_t n, const float* scale, void* x,
                                  w8a8_dtype xt, hipStream_t stream);

/*
 * Asymmetric int8 activations [P1: the asymmetric int8 case brings a few
 * small operations that are fused onto the GEMM instead of sweeping the
 * output again; the pages give no formula, the textbook scheme is used].
 * Per row m of x [M, K] (BF16/FP16/F32, row stride ldx elements):
 *   lo = min(0, min x), hi = max(0, max x)   (0 is representable),
 *   s = (hi - lo) / 255 (1.0 for an all-zero row),
 *   z = clamp(rint(-128 - lo / s), -128, 127),
 *   q = clamp(rint(x / s) + z, -128, 127),
 * in binary32 with correctly rounded divisions and round-half-even rint, so
 * that x ~ (q - z) * s. Writes q [M, ldq] int8 codes, scales [M] and
 * azp [M] (int32), all device memory. Same layout rules as
 * w8a8_quant_per_token.
 */
w8a8_status w8a8_quant_per_token_azp(const void* x, w8a8_dtype xt, int64_t M, int64_t K, int64_t ldx,
                                     void* q, int64_t ldq, float* scales, int32_t* azp,
                                     hipStream_t stream);

/*
 * Asymmetric int8 activations per tensor [P1: zero points per tensor or per
 * token for the asymmetric int8 case]: the scheme of
 * w8a8_quant_per_token_azp with one scale and zero point for the whole
 * tensor x [M, K].
 * dynamic == 1: lo and hi over every element (0 included), s and z as
 *   above, written to *scale and *azp (both required). Three kernels on
 *   `stream`; until the last one ends, the last (at most 8 KB of) codes of q
 *   hold intermediate values (partial ranges).
 * dynamic == 0 (static, calibrated): s = *scale and z = *azp are read
 *   (NULL: 1.0 and 0).
 * q = clamp(rint(x / s) + z, -128, 127). Feeds w8a8_scaled_mm_azp with
 * n_a = n_azp = 1. Same layout rules as w8a8_quant_per_token.
 */
w8a8_status w8a8_quant_per_tensor_azp(const void* x, w8a8_dtype xt, int64_t M, int64_t K,
                                      int64_t ldx, void* q, int64_t ldq, float* scale,
                                      int32_t* azp, int dynamic, hipStream_t stream);

/*
 * colsum[n] = sum_k b[n, k] over int8 weight codes b [N, K] (row stride ldb
 * bytes; the K x N column-major B of the product), int32, device. Computed
 * once per weight. K and ldb multiples of 16, b 16-byte aligned.
 */
w8a8_status w8a8_colsum(const void* b, int64_t ldb, int64_t N, int64_t K, int32_t* colsum,
                        hipStream_t stream);

/*
 * The int8 scaled product with activation zero points:
 *   D[m, n] = a_scale[m or 0] * b_scale[n or 0] * sum_k (A[m, k] - z) B[k, n]
 * with z = azp[m] (n_azp == M) or azp[0] (n_azp == 1), computed as
 * acc - z * colsum[n] in the epilogue of the int8 kernels. Arguments and
 * rules as w8a8_scaled_mm with qt = INT8; I32 output stores the corrected
 * accumulator. azp == NULL gives the symmetric product. With zero points K
 * is limited to 65536 (the corrected int32 sum stays exact).
 */
w8a8_status w8a8_scaled_mm_azp(void* out, w8a8_dtype ot, int64_t ldo, const void* a, int64_t lda,
                               const void* b, int64_t ldb, int64_t M, int64_t N, int64_t K,
                               const float* a_scales, int64_t n_a, const int32_t* azp, int64_t n_azp,
                               const int32_t* colsum, const float* b_scales, int64_t n_b,
                               hipStream_t stream);

/*
 * Merged layers [P2: the loader must handle merged QKV / gate_up layers
 * whose shards carry their own weight scales; a review comment on the same
 * page proposes one shared scale]. A merged weight stacks S shards along N:
 * shard i holds shard_rows[i] consecutive rows (host array, >= 0 each, at
 * most W8A8_MAX_SHARDS shards) and has the per-tensor weight scale
 * shard_scales[i] (device, positive).
 */
#define W8A8_MAX_SHARDS 64

/*
 * Per-channel form: b_scales[n] = shard_scales[i] for every row n of shard
 * i (device output, N = sum of shard_rows entries). Exact: one
 * w8a8_scaled_mm with per-channel b_scales then computes every shard as its
 * own per-tensor product would. N == 0 is a no-op.
 */
w8a8_status w8a8_expand_shard_scales(const float* shard_scales, const int64_t* shard_rows,
                                     int64_t num_shards, float* b_scales, hipStream_t stream);

/*
 * Shared-scale form: *shared_scale = s = max_i shard_scales[i], and every
 * code c of shard i is rescaled by the shard's ratio to it, in binary32
 * with round-to-nearest-even at each step: t_i = s_i / s, v = dec(c) * t_i,
 * code = enc(v) (e4m3: saturating RNE, NaN codes stay NaN 0x7F; int8: round
 * half to even, clamp to +-127). Lossy by one rounding per code; the shard
 * holding the maximum keeps its codes. w and out: [N, K] codes with row
 * strides ldw and ldo bytes (device; out may be w itself with ldo == ldw,
 * other overlaps are undefined). K, ldw, ldo multiples of 16; w and out
 * 16-byte aligned. The scale is written even when N or K is 0.
 */
w8a8_status w8a8_requant_shared_scale(const void* w, int64_t ldw, w8a8_qtype qt, int64_t K,
                                      const int64_t* shard_rows, int64_t num_shards,
                                      const float* shard_scales, void* out, int64_t ldo,
                                      float* shared_scale, hipStream_t stream);

/*
 * Decode attention over an e4m3fn KV cache, the cache dequantised with its
 * per-tensor scales as it is read [P3: the paged-attention kernel reads the
 * fp8 cache with the KV scale; "Scaling semantics": x' = fp8_dequant(q) *
 * scale]. One query token per sequence:
 *   out[b, h] = sum_t softmax_t(s) * dec(v[t, g]) * v_scale,
 *   s_t = sm_scale * q[b, h] . (dec(k[t, g]) * k_scale),  g = h / (Hq / Hkv),
 * over the cache rows t = seq_starts[b] .. seq_starts[b+1]-1 (contiguous
 * rows per sequence; no block table). An empty sequence gives zeros.
 *   out, q: device bf16 [B, Hq, D], contiguous.
 *   k_cache, v_cache: device e4m3fn codes [rows, Hkv, D], contiguous (the
 *     layout kv_fp8_scaled_quant writes for a [rows, Hkv, D] tensor).
 *   seq_starts: device int32 [B + 1], non-decreasing; every sequence at most
 *     max_seq_len rows (host value sizing the row splits; rows past it are
 *     not read). Rows outside 0 .. rows-1 are never read (they count as
 *     absent), so bad device offsets cannot fault.
 *   k_scale, v_scale: device float32 scalars, NULL: 1.0. sm_scale: host
 *     float, 0: 1/sqrt(D).
 *   workspace: device memory of at least
 *     kv_fp8_attention_workspace_size(B, Hq, Hkv, max_seq_len) bytes
 *     (partial results of the row splits; no initialisation needed).
 * D must be 128 and Hq / Hkv one of 1, 2, 4, 8 (UNSUPPORTED otherwise). All
 * arithmetic is float32 (exp by the hardware's exponential), the output
 * rounded once to bf16. Two kernels; nothing allocated or synchronised.
 */
int64_t kv_fp8_attention_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seq_len);

w8a8_status kv_fp8_decode_attention(void* out, const void* q, int64_t B, int64_t Hq, int64_t Hkv,
                                    int64_t D, const uint8_t* k_cache, const uint8_t* v_cache,
                                    int64_t rows, const int32_t* seq_starts, int64_t max_seq_len,
                                    const float* k_scale, const float* v_scale, float sm_scale,
                                    void* workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * Decode attention over a paged e4m3fn KV cache [P3: the paged-attention
 * kernel reads the fp8 cache through its block table and dequantises it
 * with the KV scale]. The same operation and arguments as
 * kv_fp8_decode_attention, with the cache cut into blocks of block_size
 * consecutive rows and each sequence's rows found through its block table:
 *   k_cache, v_cache: device e4m3fn codes [num_blocks * block_size, Hkv, D].
 *   block_tables: device int32 [B, table_stride]; logical row t of sequence b
 *     is cache row block_tables[b * table_stride + t / block_size] *
 *     block_size + t % block_size. Entries outside 0 .. num_blocks-1 make
 *     their rows absent (never read, no weight).
 *   seq_lens: device int32 [B], rows per sequence (at most max_seq_len; rows
 *     past it are not read). table_stride * block_size >= max_seq_len, so a
 *     sequence's rows never index past its table row.
 *   block_size: a power of two, 1 .. 1024 (else W8A8_ERR_UNSUPPORTED).
 * Blocks may be shared between sequences (a common prefix). The workspace
 * is kv_fp8_attention_workspace_size(B, Hq, Hkv, max_seq_len) bytes.
 */
w8a8_status kv_fp8_paged_decode_attention(void* out, const void* q, int64_t B, int64_t Hq,
                                          int64_t Hkv, int64_t D, const uint8_t* k_cache,
                                          const uint8_t* v_cache, int64_t num_blocks,
                                          int64_t block_size, const int32_t* block_tables,
                                          int64_t table_stride, const int32_t* seq_lens,
                                          int64_t max_seq_len, const float* k_scale,
                                          const float* v_scale, float sm_scale, void* workspace,
                                          int64_t workspace_bytes, hipStream_t stream);

/*
 * Name of the kernel configuration w8a8_scaled_mm runs for an M x N x K
 * problem, such as "gemm_decode_kernel<16x16>" or
 * "gemm_tile_kernel<256x256>" (a static string; "" for negative sizes), so
 * that profiles can be matched to calls. Host-only.
 */
const char* w8a8_scaled_mm_kernel(int64_t M, int64_t N, int64_t K);

/* The same for w8a8_scaled_mm_ws given enough workspace. */
const char* w8a8_scaled_mm_ws_kernel(int64_t M, int64_t N, int64_t K);

/*
 * The same for w8a8_quant_scaled_mm: "gemm_dynq_kernel" for the fused
 * one-token kernel, else "quant_rows_kernel+scaled_mm" (host-only).
 */
const char* w8a8_quant_scaled_mm_kernel(int64_t M, int64_t N, int64_t K);

/* Name of a status code (static string). */
const char* w8a8_status_string(w8a8_status s);

/* Message of the last failing call on this thread ("" if none). */
const char* w8a8_last_error(void);

/* Library version string. */
const char* w8a8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */

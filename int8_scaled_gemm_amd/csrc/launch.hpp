// launch.hpp -- host-side launchers of the libw8a8 kernels. Arguments are
// validated by the C ABI layer (api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

hipError_t launch_quant_per_token(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int qt, int64_t ldq, float* scales, hipStream_t st);

hipError_t launch_quant_per_tensor(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* q, int qt, int64_t ldq, float* scale, bool dynamic,
                                   hipStream_t st);

hipError_t launch_kv_dequant(const uint8_t* q, int64_t n, const float* scale, void* x, int xt,
                             hipStream_t st);

// Asymmetric int8 per-token quantisation (codes, scales, zero points) and
// the per-row code sums of int8 weights.
hipError_t launch_quant_per_token_azp(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* scales, int32_t* azp,
                                      hipStream_t st);
hipError_t launch_colsum(const uint8_t* b, int64_t ldb, int64_t N, int64_t K, int32_t* colsum,
                         hipStream_t st);
// Asymmetric int8 per tensor: one scale and zero point, from the whole
// tensor's range (dynamic: written to *scale and *azp) or given (static).
hipError_t launch_quant_per_tensor_azp(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                       uint8_t* q, int64_t ldq, float* scale, int32_t* azp,
                                       bool dynamic, hipStream_t st);

// Merged layers: the most shards one call takes (their row ends travel as
// kernel arguments).
constexpr int kMaxShards = 64;

// b_scales[n] = s[i] for every row n of shard i (rows[i] rows each).
hipError_t launch_expand_shard_scales(const float* s, const int64_t* rows, int64_t S, float* out,
                                      hipStream_t st);

// Codes of a merged [N, K] weight rescaled to the shared scale max(s):
// out may be w itself (ldo == ldw); *shared receives max(s).
hipError_t launch_requant_shared_scale(const uint8_t* w, int64_t ldw, int qt, int64_t K,
                                       const int64_t* rows, int64_t S, const float* s, uint8_t* out,
                                       int64_t ldo, float* shared, hipStream_t st);

struct GemmProblem {
    void* out;
    int ot;
    int64_t ldo;
    const uint8_t* a;
    int64_t lda;
    const uint8_t* b;
    int64_t ldb;
    int qt;
    int64_t M, N, K;
    const float* sa;  // NULL: 1.0
    bool sa_per_row;
    const float* sb;  // NULL: 1.0
    bool sb_per_col;
    void* workspace = nullptr;    // optional: room for split-K partial sums
    int64_t workspace_bytes = 0;
    // asymmetric int8: zero points (1 or M entries) and the weights' code sums
    const int32_t* azp = nullptr;
    bool azp_per_row = false;
    const int32_t* colsum = nullptr;
};

// How a decode problem splits K when given a workspace (splits == 1: no
// split): the split count, the K stages each split walks, the bytes of the
// partial sums, and the decode kernel configuration that runs split.
struct SplitPlan {
    int splits;
    int stages_per_split;
    int64_t workspace_bytes;
    int config;
};
SplitPlan plan_splitk(int64_t M, int64_t N, int64_t K);

hipError_t launch_scaled_mm(const GemmProblem& p, hipStream_t st);

// launch_scaled_mm with split K through the library's static device scratch
// (no caller workspace, no allocation); *needed is set to the scratch bytes
// a problem would need when it is more than the scratch holds.
hipError_t launch_scaled_mm_noalloc(const GemmProblem& p, hipStream_t st, int64_t* needed);
int64_t scaled_mm_noalloc_scratch_bytes();

// Dynamic per-token quantisation of x [M, K] into q / a_scales, then the
// scaled product with p's B and b scales (p.a, p.lda, p.sa are ignored).
// Problems with quant_scaled_mm_fused() run as one fused kernel.
hipError_t launch_quant_scaled_mm(const GemmProblem& p, int xt, const void* x, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* a_scales, hipStream_t st);
bool quant_scaled_mm_fused(int64_t M, int64_t N, int64_t K);

// Name of the kernel configuration a problem runs with.
const char* scaled_mm_kernel_name(int64_t M, int64_t N, int64_t K, bool workspace);

// Decode attention over an e4m3fn KV cache (attention.hip).
struct AttnArgs {
    uint16_t* out;           // [B, Hq, 128] bf16
    const uint16_t* q;       // [B, Hq, 128] bf16
    const uint8_t* k;        // [rows, Hkv, 128] e4m3fn
    const uint8_t* v;
    const int32_t* starts;   // [B + 1] (device)
    const float* k_scale;    // NULL: 1.0
    const float* v_scale;
    float sm_scale;
    int B, Hq, Hkv;
    int64_t rows;            // cache rows (reads past them are skipped)
    int splits, chunk;       // row splits per sequence, rows per split (multiple of 32)
    float* part;             // [B, Hq, splits, 130] partial sums, maxima and weights
    // Paged layout (tables != NULL): sequence b has lens[b] rows; its logical
    // row t is cache row tables[b * table_stride + t / 2^bshift] * 2^bshift +
    // t % 2^bshift (blocks of 2^bshift rows); entries outside 0 .. nblocks-1
    // and rows past table_stride blocks are absent. starts is unused.
    const int32_t* tables = nullptr;
    const int32_t* lens = nullptr;
    int64_t table_stride = 0;
    int bshift = 0;
    int64_t nblocks = 0;
};
int attention_splits(int64_t B, int64_t Hkv, int64_t max_rows);
int attention_chunk(int64_t max_rows, int splits);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

}  // namespace w8a8

// attention.hip -- decode attention over an e4m3fn KV cache, the cache
// dequantised with its per-tensor scales as it is read ("Enable scaled FP8
// (e4m3fn) KV cache on ROCm": the paged-attention kernel reads the fp8 cache
// and dequantises it with the KV scale, x' = fp8_dequant(q) * scale).
//
// One query token per sequence, D = 128, grouped-query heads (query head h
// reads KV head h / G). Sequence b owns cache rows starts[b] .. starts[b+1]-1
// of K and V [rows, Hkv, D]. The cache is read once (1 byte per element);
// the scores run on the matrix cores, the rest in fp32 on the vector units:
//  - attn_split_kernel: workgroup (split s, KV head g, sequence b), one wave
//    per query head of the group, over the split's rows in blocks of 64.
//    K and V blocks are staged in LDS (each loaded once for the G heads),
//    the next block's bytes held in registers while the current one is
//    consumed. The block's scores for all G heads are bf16 MFMAs (codes
//    converted exactly to bf16, the query's own bf16 values, float32
//    sums), scaled by sm_scale * k_scale; lane t of wave w then holds row
//    t's score for head w. The softmax runs online (running max m and sum l
//    per wave), and lane l accumulates output dims 8 (l % 16) .. +7 over
//    rows 16 (l / 16) .. +15 of each block (the weights through LDS); the
//    four row groups are added once per split. Writes (o, m, l) per split.
//  - attn_combine_kernel: per (sequence, head), the splits' partial sums
//    rescaled to the common maximum (kept as a running maximum in one pass
//    over the splits), divided by the total weight, times v_scale, rounded
//    to bf16.
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace w8a8 {

namespace {

constexpr int kD = 128;        // head dimension
constexpr int kRows = 64;      // cache rows per block (one per lane)
constexpr int kChunks = 2 * kRows * kD / 16;  // 16-byte pieces of one K + V block
constexpr int kMaxSplits = 1024;  // row splits per sequence at most

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int G, bool PAGED>
__global__ __launch_bounds__(G * 64) void attn_split_kernel(AttnArgs p) {
    constexpr int NT = G * 64;
    constexpr int PER = kChunks / NT;  // pieces per thread per block
    static_assert(kChunks % NT == 0, "block pieces per thread");
    __shared__ __attribute__((aligned(16))) float ss[G][kRows];  // scores of the block
    __shared__ __attribute__((aligned(16))) float ps[G][kRows];
    __shared__ __attribute__((aligned(16))) uint8_t kb[kRows * kD];
    __shared__ __attribute__((aligned(16))) uint8_t vb[kRows * kD];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = g * G + w;
    const int first = PAGED ? 0 : p.starts[b];
    const int len = max(PAGED ? p.lens[b] : p.starts[b + 1] - first, 0);
    // Cache row of the sequence's logical row t (t < len), or -1 when it is
    // absent: outside the cache, or (paged) a block entry outside the cache
    // or past the table's row.
    auto cache_row = [&](int t) -> int64_t {
        if constexpr (PAGED) {
            const int64_t j = t >> p.bshift;
            if (j >= p.table_stride) return -1;
            const int blk = p.tables[static_cast<int64_t>(b) * p.table_stride + j];
            if (blk < 0 || blk >= p.nblocks) return -1;
            return (static_cast<int64_t>(blk) << p.bshift) + (t & ((1 << p.bshift) - 1));
        } else {
            const int64_t row = static_cast<int64_t>(first) + t;
            return row >= 0 && row < p.rows ? row : -1;
        }
    };
    const int r0 = s * p.chunk, r1 = min(len, r0 + p.chunk);
    float* dst = p.part + ((static_cast<int64_t>(b) * p.Hq + h) * p.splits + s) * (kD + 2);
    if (r0 >= r1) {  // past the end of the sequence: no weight
        if (lane == 0) {
            dst[kD] = -INFINITY;
            dst[kD + 1] = 0.0f;
        }
        return;
    }
    const float qscale = p.sm_scale * (p.k_scale ? *p.k_scale : 1.0f);
    // The group's queries as the second operand of 16 x 16 x 32 bf16 MFMAs:
    // lane l holds query head l % 16 of the group (zeros past G), dims
    // 32 ks + 8 (l / 16) .. +7 for ks = 0..3, the query's own bf16 values.
    u32x4 qf[kD / 32];
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
        qf[ks] = u32x4{0, 0, 0, 0};
        if ((lane & 15) < G)
            qf[ks] = *reinterpret_cast<const u32x4*>(
                p.q + (static_cast<int64_t>(b) * p.Hq + g * G + (lane & 15)) * kD + 32 * ks + 8 * (lane >> 4));
    }
    // Piece i of a block: K (i < kChunks/2) or V, row (i % 512) / 8, 16-byte
    // chunk i % 8. Rows past the split, the sequence or the cache read zero.
    const int64_t rstride = static_cast<int64_t>(p.Hkv) * kD;
    auto fetch = [&](int base, u32x4* v) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = threadIdx.x + NT * j;
            const int half = i / (kChunks / 2), k = i % (kChunks / 2);
            const int t = base + k / 8;
            const int64_t row = t < r1 ? cache_row(t) : -1;
            v[j] = u32x4{0, 0, 0, 0};
            if (row >= 0)
                v[j] = *reinterpret_cast<const u32x4*>((half ? p.v : p.k) + row * rstride +
                                                       static_cast<int64_t>(g) * kD + 16 * (k % 8));
        }
    };
    // K row t keeps chunk c at slot c ^ (t % 8): the 64 lanes, one row each,
    // then read 8 different slots per group of 8 rows. V row t keeps it at
    // slot c ^ (t / 16), so that the four 16-row groups read apart.
    auto stash = [&](const u32x4* v) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = threadIdx.x + NT * j;
            const int half = i / (kChunks / 2), k = i % (kChunks / 2);
            const int t = k / 8, c = k % 8;
            uint8_t* dst = half ? vb + t * kD + 16 * (c ^ (t >> 4)) : kb + t * kD + 16 * (c ^ (t & 7));
            *reinterpret_cast<u32x4*>(dst) = v[j];
        }
    };

    const int grp = lane >> 4, d0 = 8 * (lane & 15);  // value rows grp, grp+4, ...; dims d0..d0+7
    float m = -INFINITY, l = 0.0f;
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    u32x4 nxt[PER];
    fetch(r0, nxt);
    for (int base = r0; base < r1; base += kRows) {
        __syncthreads();  // the previous block is consumed
        stash(nxt);
        __syncthreads();
        if (base + kRows < r1) fetch(base + kRows, nxt);  // in flight during this block
        // Scores of the block's 64 rows for the G heads: 16-row tiles, each
        // dec(K) [16 x 128] . Q^T [128 x 16] as four bf16 MFMAs (the e4m3
        // codes convert exactly to bf16; the products are exact in float32).
        // Lane l of a tile reads row l % 16, dims 32 ks + 8 (l / 16) .. +7.
        for (int tile = w; tile < kRows / 16; tile += G) {
            f32x4 acc = f32x4{0, 0, 0, 0};
            const int r = 16 * tile + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) {
                const int c = 2 * ks + (lane >> 5);
                const u32x2 raw = *reinterpret_cast<const u32x2*>(
                    kb + r * kD + 16 * (c ^ (r & 7)) + 8 * ((lane >> 4) & 1));
                const f32x2 x[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(raw[0], false),
                                    __builtin_amdgcn_cvt_pk_f32_fp8(raw[0], true),
                                    __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], false),
                                    __builtin_amdgcn_cvt_pk_f32_fp8(raw[1], true)};
                u32x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a[e] = (__float_as_uint(x[e][0]) >> 16) | (__float_as_uint(x[e][1]) & 0xFFFF0000u);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, qf[ks]), acc,
                                                              0, 0, 0);
            }
            // lane l holds rows 16 tile + 4 (l / 16) + i of head l % 16
            if ((lane & 15) < G) {
#pragma unroll
                for (int i = 0; i < 4; ++i) ss[lane & 15][16 * tile + 4 * (lane >> 4) + i] = acc[i];
            }
        }
        __syncthreads();
        const float sc = ss[w][lane] * qscale;  // score of row base + lane for head h
        const bool valid = base + lane < r1 && cache_row(base + lane) >= 0;  // absent rows: no weight
        const float mn = fmaxf(m, wave_max(valid ? sc : -INFINITY));
        // A block with no row inside the cache leaves mn = m = -inf: nothing
        // to add (and -inf - -inf must not reach the exponential).
        const float alpha = mn == -INFINITY ? 1.0f : __expf(m - mn);  // 0 on the first block
        const float pt = valid ? __expf(sc - mn) : 0.0f;
        l = l * alpha + wave_sum(pt);
        ps[w][lane] = pt;  // read back by the lanes of this wave only
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
        for (int i4 = 0; i4 < kRows / 16; i4 += 1) {
            // rows t = 16 grp + 4 i4 .. +3 of the block
            const int t0 = 16 * grp + 4 * i4;
            const f32x4 pw = *reinterpret_cast<const f32x4*>(&ps[w][t0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + r;
                const u32x2 vv = *reinterpret_cast<const u32x2*>(
                    vb + t * kD + 16 * ((d0 >> 4) ^ grp) + (d0 & 15));
                const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(vv[0], false);
                const f32x2 b2 = __builtin_amdgcn_cvt_pk_f32_fp8(vv[0], true);
                const f32x2 c2 = __builtin_amdgcn_cvt_pk_f32_fp8(vv[1], false);
                const f32x2 d2 = __builtin_amdgcn_cvt_pk_f32_fp8(vv[1], true);
                o[0] = fmaf(pw[r], a[0], o[0]);
                o[1] = fmaf(pw[r], a[1], o[1]);
                o[2] = fmaf(pw[r], b2[0], o[2]);
                o[3] = fmaf(pw[r], b2[1], o[3]);
                o[4] = fmaf(pw[r], c2[0], o[4]);
                o[5] = fmaf(pw[r], c2[1], o[5]);
                o[6] = fmaf(pw[r], d2[0], o[6]);
                o[7] = fmaf(pw[r], d2[1], o[7]);
            }
        }
        __builtin_amdgcn_wave_barrier();  // ps is rewritten by the next block
        m = mn;
    }
    // add the four row groups (lanes l, l+16, l+32, l+48 hold the same dims)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[e] += __shfl_xor(o[e], 16, 64);
        o[e] += __shfl_xor(o[e], 32, 64);
    }
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[d0 + e] = o[e];
    }
    if (lane == 0) {
        dst[kD] = m;
        dst[kD + 1] = l;
    }
}

__global__ __launch_bounds__(kD) void attn_combine_kernel(AttnArgs p) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const float* part = p.part + (static_cast<int64_t>(b) * p.Hq + h) * p.splits * (kD + 2);
    // One pass with a running maximum: the sums so far and each split's are
    // rescaled to the larger of the two maxima as they are added. Splits with
    // no weight are skipped (their partial sums may be unset).
    float mx = -INFINITY, tot = 0.0f, acc = 0.0f;
#pragma unroll 8
    for (int s = 0; s < p.splits; ++s) {
        const float* ps = part + s * (kD + 2);
        const float ms = ps[kD], ls = ps[kD + 1], v = ps[d];
        const bool live = ls > 0.0f;
        const float mn = live ? fmaxf(mx, ms) : mx;
        const float a = live ? __expf(mx - mn) : 1.0f;  // 0 while nothing is summed
        const float f = live ? __expf(ms - mn) : 0.0f;
        tot = live ? fmaf(ls, f, tot * a) : tot;
        acc = live ? fmaf(v, f, acc * a) : acc;
        mx = mn;
    }
    const float vs = p.v_scale ? *p.v_scale : 1.0f;
    const float o = tot > 0.0f ? acc / tot * vs : 0.0f;  // an empty sequence gives zeros
    p.out[(static_cast<int64_t>(b) * p.Hq + h) * kD + d] = to_bf16_bits(o);
}

}  // namespace

int attention_splits(int64_t B, int64_t Hkv, int64_t max_rows) {
    // At least 256 rows per split, and enough workgroups for eight per CU
    // (sequences shorter than the longest leave their later splits empty).
    const int64_t by_rows = (max_rows + 255) / 256;
    const int64_t by_grid = (2048 + B * Hkv - 1) / (B * Hkv);
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(std::min(by_rows, by_grid), kMaxSplits)));
}

int attention_chunk(int64_t max_rows, int splits) {
    const int64_t c = (max_rows + splits - 1) / splits;
    return static_cast<int>(std::max<int64_t>(kRows, (c + kRows - 1) / kRows * kRows));
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
    const dim3 grid(a.splits, a.Hkv, a.B);
#define W8A8_ATTN(PG)                                                                                 \
    switch (a.Hq / a.Hkv) {                                                                           \
        case 1: hipLaunchKernelGGL((attn_split_kernel<1, PG>), grid, dim3(64), 0, st, a); break;     \
        case 2: hipLaunchKernelGGL((attn_split_kernel<2, PG>), grid, dim3(128), 0, st, a); break;    \
        case 4: hipLaunchKernelGGL((attn_split_kernel<4, PG>), grid, dim3(256), 0, st, a); break;    \
        default: hipLaunchKernelGGL((attn_split_kernel<8, PG>), grid, dim3(512), 0, st, a); break;   \
    }
    if (a.tables) {
        W8A8_ATTN(true)
    } else {
        W8A8_ATTN(false)
    }
#undef W8A8_ATTN
    hipLaunchKernelGGL(attn_combine_kernel, dim3(a.Hq, a.B), dim3(kD), 0, st, a);
    return hipGetLastError();
}

}  // namespace w8a8

// attention.hip -- decode attention over an e4m3fn KV cache, the cache
// dequantised with its per-tensor scales as it is read ("Enable scaled FP8
// (e4m3fn) KV cache on ROCm": the paged-attention kernel reads the fp8 cache
// and dequantises it with the KV scale, x' = fp8_dequant(q) * scale).
//
// One query token per sequence, D = 128, grouped-query heads (query head h
// reads KV head h / G). Sequence b owns cache rows starts[b] .. starts[b+1]-1
// of K and V [rows, Hkv, D], or (paged) the rows its block table names. The
// cache is read once (1 byte per element):
//  - attn_split_kernel: one wave per (row split s, KV head g, sequence b),
//    all G query heads of the group at once, over the split's rows in
//    steps of 32 staged in a wave-private LDS ring by direct global -> LDS
//    loads (no barrier). Scores are bf16 MFMAs (codes converted exactly to
//    bf16, the query's own bf16 values, float32 sums) scaled by
//    sm_scale * k_scale; the online softmax keeps a running maximum and
//    weight sum per head; the weights, as fp16 hi + lo parts, and the value
//    codes, converted exactly to fp16 and read transposed from LDS, make the
//    output sums on fp16 MFMAs. Writes (o, m, l) per head and split.
//  - attn_combine_kernel: per (sequence, head), the splits' partial sums
//    rescaled to the common maximum (32 splits at a time, all their loads in
//    flight together, with a running maximum across batches), divided by the
//    total weight, times v_scale, rounded to bf16.
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace w8a8 {

namespace {

constexpr int kD = 128;        // head dimension
constexpr int kStep = 32;      // cache rows per wave step
constexpr int kMaxSplits = 1024;  // row splits per sequence at most
constexpr int kStages = 2;        // steps in a wave's LDS ring
constexpr int64_t kMinWaves = 1024;  // waves the split rule aims for at least
constexpr int kCombineBatch = 32;    // splits whose partial sums the combine requests together

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// Eight value codes of one head dimension from eight consecutive block rows,
// through the LDS transpose read: within each 16-lane group, lane i names 8
// bytes (row 8q + i / 2 of the group's eight rows, dims 8 (i % 2) .. +7 of a
// 16-dim tile), and lane i gets byte i % 8 of the pieces named by lanes
// 2b + i / 8, b = 0..7: dim i of the tile, rows 8q .. 8q + 7 in order.
__device__ __forceinline__ u32x2 read_tr8(const uint8_t* lds) {
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)(const_cast<uint8_t*>(lds)));
    return __builtin_bit_cast(u32x2, r);
}

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight e4m3 codes as eight fp16 (bf16) values, two per conversion with
// scale 1 (exact: every e4m3 value is an fp16 and a bf16 value).
__device__ __forceinline__ h16x8 e4m3x8_to_f16(u32x2 raw) {
    u32x4 h;
    h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[0], 1.0f, false));
    h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[0], 1.0f, true));
    h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[1], 1.0f, false));
    h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[1], 1.0f, true));
    return __builtin_bit_cast(h16x8, h);
}
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4 h;
    h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    return __builtin_bit_cast(bf16x8, h);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Loaded in place of the cache bytes of a row outside the split, the
// sequence or the cache (zeros), and of a block-table entry past the
// table's row (-1: absent), so that every wave issues the same loads per
// step whatever its rows.
__device__ __attribute__((aligned(16))) uint8_t kZeroPiece[16];
__device__ __attribute__((aligned(16))) int32_t kAbsentEntry[4] = {-1, -1, -1, -1};

typedef __attribute__((address_space(3))) uint8_t* lds_ptr;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(p))));
}

// Direct global -> LDS loads: lane q of the wave writes the 16 (4) bytes at
// src to LDS byte address lds + 16 q (+ 4 q); lds is wave-uniform. They have
// no register result and retire in issue order with the wave's other vector
// memory loads; the waits for them are explicit (wait_loads), so that the
// loads of the next steps stay in flight while a step is computed. The
// cache pieces (16 bytes per lane) are read once: non-temporal, which took
// the call on a Llama-3-8B layer from 25.5 to 23.4 us; the block-table
// entries (4 bytes per lane), which every KV head's waves read, are cached.
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void load_lds4(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}

// Wait until at most n (one of the listed counts) of the wave's vector
// memory loads are in flight; an n not listed waits for all (safe: it only
// waits longer).
__device__ __forceinline__ void wait_loads(int n) {
    switch (n) {
        case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
        case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
        case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// Value row t (0..31) of a step keeps its 16-byte chunk c at slot
// c ^ vswz(t): the eight rows that one 16-lane group of the transposed value
// reads names (4q + i and 16 + 4q + i, i < 4) then sit in eight different
// slots. Key row t keeps chunk c at slot c ^ (t % 8), for the score reads
// (eight consecutive rows at one chunk per eight lanes).
__device__ __forceinline__ int vswz(int t) { return (t & 3) | ((t >> 2) & 4); }

// One wave per workgroup, sequence b, KV head g, row split s; the wave runs
// over the split's rows in steps of 32 through a private NS-slot LDS ring
// (K rows, V rows, and for a paged cache the rows' block-table entries),
// NS - 1 steps ahead of the one being computed, with no barrier. All G
// query heads of the group are computed together: the scores of the step's
// 32 rows are two 16 x 16 bf16 MFMA tiles, rows x heads (lane l: head l % 16,
// rows 16 t + 4 (l / 16) + i), and the same registers, as fp16 hi + lo parts,
// are the second operand of O^T [128 dims x 16 heads] += V^T P^T on fp16
// MFMAs (16 x 16 x 32): contraction slot 8 (l / 16) + b of lane l is row
// 16 (b / 4) + 4 (l / 16) + b % 4, and the transposed LDS read gives each
// lane those rows of its dim. Lane l thus keeps dims 16 tile + 4 (l / 16) + i
// of head l % 16, rescaled by its own head's factor; the running maximum is
// shared by the head's four lanes (two exchanges per step), the weight sums
// are added over them once at the end.
template <int G, bool PAGED, int NS>
__global__ __launch_bounds__(64) void attn_split_kernel(AttnArgs p) {
    constexpr int kSlot = 2 * kStep * kD;  // K then V rows of a step
    __shared__ __attribute__((aligned(16))) uint8_t ring[NS][kSlot];
    // Paged: the block-table entries of step k's rows in ent[k % 8], loaded
    // 2 NS - 2 steps ahead, before the pieces of the step whose wait covers
    // them.
    constexpr int kAhead = 2 * NS - 2;
    static_assert(kAhead + 1 <= 8, "entry ring");
    __shared__ __attribute__((aligned(16))) int32_t ent[PAGED ? 8 : 1][64];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int q4 = lane >> 4, n16 = lane & 15;
    const int first = PAGED ? 0 : p.starts[b];
    const int len = max(PAGED ? p.lens[b] : p.starts[b + 1] - first, 0);
    const int r0 = s * p.chunk, r1 = min(len, r0 + p.chunk);
    // partial results of head g G + hd: [B, Hq, splits, 130]
    auto part = [&](int hd) {
        return p.part + ((static_cast<int64_t>(b) * p.Hq + g * G + hd) * p.splits + s) * (kD + 2);
    };
    if (r0 >= r1) {  // past the end of the sequence: no weight
        if (lane < G) {
            part(lane)[kD] = -INFINITY;
            part(lane)[kD + 1] = 0.0f;
        }
        return;
    }
    const int nst = (r1 - r0 + kStep - 1) / kStep;
    const float qscale = p.sm_scale * (p.k_scale ? *p.k_scale : 1.0f);
    // The queries as the second operand of the score MFMAs (16 x 16 x 32
    // bf16, four per 16-row tile): lane l holds head l % 16 (zeros past G),
    // dims 32 (l / 16) + 8 ks .. +7 for ks = 0..3, the query's own bf16 values.
    u32x4 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        qf[ks] = u32x4{0, 0, 0, 0};
        if (n16 < G)
            qf[ks] = *reinterpret_cast<const u32x4*>(
                p.q + (static_cast<int64_t>(b) * p.Hq + g * G + n16) * kD + 32 * q4 + 8 * ks);
    }
    const int64_t rstride = static_cast<int64_t>(p.Hkv) * kD;
    const int64_t goff = static_cast<int64_t>(g) * kD;
    // Paged: the block-table entries of step k's rows into ent[k % 8] (lane
    // t < 32: row r0 + 32 k + t).
    auto fetch_entries = [&](int k) {
        const int t = r0 + kStep * k + lane;
        const int64_t j = static_cast<int64_t>(t) >> p.bshift;
        const void* src = lane < kStep && t < r1 && j < p.table_stride
                              ? static_cast<const void*>(p.tables + static_cast<int64_t>(b) * p.table_stride + j)
                              : static_cast<const void*>(kAbsentEntry);
        load_lds4(src, lds_addr(&ent[k & 7][0]));
    };
    // Cache row of the split's row r0 + 32 k + t, or -1 when it is absent.
    auto cache_row = [&](int k, int t) -> int64_t {
        const int lt = r0 + kStep * k + t;
        if (lt >= r1) return -1;
        if constexpr (PAGED) {
            const int blk = ent[k & 7][t];
            if (blk < 0 || blk >= p.nblocks) return -1;
            return (static_cast<int64_t>(blk) << p.bshift) + (lt & ((1 << p.bshift) - 1));
        } else {
            const int64_t row = static_cast<int64_t>(first) + lt;
            return row < p.rows ? row : -1;
        }
    };
    // Step k's 8 KB into slot: instruction j writes pieces 64 j + lane; K
    // pieces (j < 4) and V pieces (j >= 4) of row (64 (j % 4) + lane) / 8.
    // Contiguous rows all inside the split and the cache: piece 64 j + lane
    // of step k is row r0 + 32 k + 8 j + lane / 8, chunk (lane % 8) ^ (the
    // row's swizzle, which for V depends on j only through j >= 2).
    const int64_t lane_off = (static_cast<int64_t>(first) + r0 + lane / 8) * rstride + goff;
    const int kch = 16 * ((lane & 7) ^ (lane >> 3));
    const int vch0 = 16 * ((lane & 7) ^ ((lane >> 3) & 3)), vch1 = 16 * ((lane & 7) ^ (((lane >> 3) & 3) | 4));
    auto fetch = [&](int k, int slot) {
        if (!PAGED && r0 + kStep * (k + 1) <= r1 && static_cast<int64_t>(first) + r0 + kStep * (k + 1) <= p.rows) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t rows_off = (static_cast<int64_t>(kStep) * k + 8 * (j & 3)) * rstride;
                const uint8_t* src = j < 4 ? p.k + lane_off + rows_off + kch
                                           : p.v + lane_off + rows_off + ((j & 3) < 2 ? vch0 : vch1);
                load_lds16(src, lds_addr(&ring[slot][(j < 4 ? 0 : kStep * kD) + 16 * 64 * (j & 3)]));
            }
            return;
        }
        // The rows of the lane's four K and four V pieces first (a paged row
        // reads its block entry from LDS; read between the loads, whose asm
        // orders memory, each would be waited for in turn).
        int64_t row[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) row[j] = cache_row(k, (64 * j + lane) / 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = 64 * (j & 3) + lane;
            const int t = i / 8, sl = i % 8;
            const int c = sl ^ (j < 4 ? (t & 7) : vswz(t));
            const uint8_t* src =
                row[j & 3] >= 0 ? (j < 4 ? p.k : p.v) + row[j & 3] * rstride + goff + 16 * c : kZeroPiece;
            load_lds16(src, lds_addr(&ring[slot][(j < 4 ? 0 : kStep * kD) + 16 * 64 * (j & 3)]));
        }
    };
    // Loads issued at step u, in issue order: (paged) the entries of step
    // u + kAhead, then the pieces of step u + NS - 1. Those issued after the
    // pieces of step k (issued at step k - NS + 1):
    auto issued_after = [&](int k) {
        int n = 0;
#pragma unroll
        for (int v = 1; v <= NS - 2; ++v) {
            n += k + v < nst ? 8 : 0;
            if constexpr (PAGED) n += k + NS - 1 + v < nst ? 1 : 0;
        }
        return n;
    };

    f32x4 acc[kD / 16];  // O^T tiles: dims 16 tile + 4 q4 + i, head n16
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) acc[t] = f32x4{0, 0, 0, 0};
    float m = -INFINITY, l = 0.0f;  // running maximum (shared by the head's lanes), own weight sum

    if constexpr (PAGED) {  // the entries of the first kAhead steps
#pragma unroll
        for (int k = 0; k < kAhead; ++k)
            if (k < nst) fetch_entries(k);
        wait_loads(0);
    }
#pragma unroll
    for (int k = 0; k < NS - 1; ++k)
        if (k < nst) fetch(k, k);
    for (int k = 0; k < nst; ++k) {
        const int slot = k % NS;
        wait_loads(issued_after(k));  // step k's pieces (and the entries of step k + NS - 1) are in LDS
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slot (k - 1) % NS and ent[(k - 2) % 8] are read
        if constexpr (PAGED) {
            if (k + kAhead < nst) fetch_entries(k + kAhead);
        }
        if (k + NS - 1 < nst) fetch(k + NS - 1, (k + NS - 1) % NS);
        const uint8_t* kb = ring[slot];
        const uint8_t* vb = ring[slot] + kStep * kD;
        // scores: tile t, lane l: row 16 t + l % 16, dims 32 q4 .. +31
        f32x4 sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = 16 * t + n16;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(kb + r * kD + 16 * ((2 * q4) ^ (r & 7)));
            const u32x4 hi = *reinterpret_cast<const u32x4*>(kb + r * kD + 16 * ((2 * q4 + 1) ^ (r & 7)));
            sc[t] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4& src = ks < 2 ? lo : hi;
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    e4m3x8_to_bf16(src[2 * (ks & 1)], src[2 * (ks & 1) + 1]), __builtin_bit_cast(bf16x8, qf[ks]),
                    sc[t], 0, 0, 0);
            }
        }
        // lane l: rows 16 t + 4 q4 + i of head n16
        bool valid[2][4];
        float bmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                valid[t][i] = cache_row(k, 16 * t + 4 * q4 + i) >= 0;
                sc[t][i] *= qscale;
                if (valid[t][i]) bmax = fmaxf(bmax, sc[t][i]);
            }
        }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const float mn = fmaxf(m, bmax);
        // A step with no row inside the cache leaves mn = m = -inf: nothing
        // to add (and -inf - -inf must not reach the exponential).
        const float alpha = mn == -INFINITY ? 1.0f : __expf(m - mn);  // 0 on the first step
        u32x4 ph, pl;  // weights as fp16 hi and lo, contraction slots b = 0..7
        float lsum = 0.0f;
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const float pt = valid[bb / 4][bb % 4] ? __expf(sc[bb / 4][bb % 4] - mn) : 0.0f;
            lsum += pt;
            const _Float16 h = static_cast<_Float16>(pt);
            const _Float16 lo = static_cast<_Float16>(pt - static_cast<float>(h));
            const uint32_t hb = __builtin_bit_cast(uint16_t, h), lb = __builtin_bit_cast(uint16_t, lo);
            if (bb & 1) {
                ph[bb / 2] |= hb << 16;
                pl[bb / 2] |= lb << 16;
            } else {
                ph[bb / 2] = hb;
                pl[bb / 2] = lb;
            }
        }
        l = l * alpha + lsum;
        m = mn;
        // The sums change scale only where some head's maximum rose.
        const bool rescale = __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0;
        // V^T operand, dim tile t: the 16-lane group q4 names rows
        // 16 (b / 4) + 4 q4 + b % 4 (b = i / 2 for lane i of the group) at
        // dims 16 t + 8 (i % 2) .. +7.
        const int vr = 16 * ((n16 >> 1) >> 2) + 4 * q4 + ((n16 >> 1) & 3);
        const uint8_t* vrow = vb + vr * kD + 8 * (n16 & 1);
        const int vz = vswz(vr);
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) {
            const h16x8 vt = e4m3x8_to_f16(read_tr8(vrow + 16 * (t ^ vz)));
            if (rescale) acc[t] *= alpha;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vt, __builtin_bit_cast(h16x8, ph), acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vt, __builtin_bit_cast(h16x8, pl), acc[t], 0, 0, 0);
        }
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (n16 < G) {
        float* dst = part(n16);
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t + 4 * q4) = acc[t];
        if (q4 == 0) {
            dst[kD] = m;
            dst[kD + 1] = l;
        }
    }
}

__global__ __launch_bounds__(kD) void attn_combine_kernel(AttnArgs p) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x, lane = threadIdx.x & (kCombineBatch - 1);
    const float* part = p.part + (static_cast<int64_t>(b) * p.Hq + h) * p.splits * (kD + 2);
    // Only the splits that start inside the sequence were written. They are
    // taken kCombineBatch at a time, every load of a batch issued before the
    // first is used (past the last split a batch re-reads it, unused): lane j
    // (mod 32) holds split j's maximum and weight, and every thread its
    // dim of each split's sums. The batch's largest maximum over the splits
    // with weight, each split's sums scaled to the larger of it and the
    // running maximum, added to the running sums rescaled likewise. A split
    // with no weight (every row absent) adds nothing.
    const int len = max(p.tables ? p.lens[b] : p.starts[b + 1] - p.starts[b], 0);
    const int live = min(p.splits, (len + p.chunk - 1) / p.chunk);
    float mx = -INFINITY, tot = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < live; s0 += kCombineBatch) {
        const float* pl = part + min(s0 + lane, live - 1) * (kD + 2);
        const float mj = pl[kD], lj = pl[kD + 1];
        float v[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) v[j] = part[min(s0 + j, live - 1) * (kD + 2) + d];
        const bool wj = s0 + lane < live && lj > 0.0f;
        float mb = wj ? mj : -INFINITY;
#pragma unroll
        for (int m = kCombineBatch / 2; m >= 1; m >>= 1) mb = fmaxf(mb, __shfl_xor(mb, m, 64));
        const float mn = fmaxf(mx, mb);  // -inf while no split so far has weight
        const float a = mn == -INFINITY ? 1.0f : __expf(mx - mn);  // 0 while nothing is summed
        const float fj = wj ? __expf(mj - mn) : 0.0f;
        float tb = lj * fj;
#pragma unroll
        for (int m = kCombineBatch / 2; m >= 1; m >>= 1) tb += __shfl_xor(tb, m, 64);
        float ab = 0.0f;
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            ab = fmaf(v[j], __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fj), j)), ab);
        tot = fmaf(tot, a, tb);
        acc = fmaf(acc, a, ab);
        mx = mn;
    }
    const float vs = p.v_scale ? *p.v_scale : 1.0f;
    const float o = tot > 0.0f ? acc / tot * vs : 0.0f;  // an empty sequence gives zeros
    p.out[(static_cast<int64_t>(b) * p.Hq + h) * kD + d] = to_bf16_bits(o);
}

}  // namespace

int attention_splits(int64_t B, int64_t Hkv, int64_t max_rows) {
    // 128 rows (four steps) per wave, fewer (down to 64) while the grid
    // would have under kMinWaves waves, more where the longest sequence
    // would need over kMaxSplits splits (sequences shorter than the longest
    // leave their later splits empty).
    int64_t c = 128;
    while (c > 64 && B * Hkv * ((max_rows + c - 1) / c) < kMinWaves) c /= 2;
    const int64_t need = (max_rows + kMaxSplits - 1) / kMaxSplits;
    c = std::max<int64_t>(c, (need + kStep - 1) / kStep * kStep);
    return static_cast<int>(std::max<int64_t>(1, (max_rows + c - 1) / c));
}

int attention_chunk(int64_t max_rows, int splits) {
    const int64_t c = (max_rows + splits - 1) / splits;
    return static_cast<int>(std::max<int64_t>(kStep, (c + kStep - 1) / kStep * kStep));
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
    const dim3 grid(a.splits, a.Hkv, a.B);
#define W8A8_ATTN(PG)                                                                                 \
    switch (a.Hq / a.Hkv) {                                                                           \
        case 1: hipLaunchKernelGGL((attn_split_kernel<1, PG, kStages>), grid, dim3(64), 0, st, a); break;  \
        case 2: hipLaunchKernelGGL((attn_split_kernel<2, PG, kStages>), grid, dim3(64), 0, st, a); break;  \
        case 4: hipLaunchKernelGGL((attn_split_kernel<4, PG, kStages>), grid, dim3(64), 0, st, a); break;  \
        default: hipLaunchKernelGGL((attn_split_kernel<8, PG, kStages>), grid, dim3(64), 0, st, a); break; \
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

// gemm.hip -- the w8a8 scaled matrix multiply on gfx950 MFMA.
//
//   D[m, n] = a_scale[m|0] * b_scale[n|0] * sum_k A[m, k] * B[n, k]
//
// ("[Kernel] Add w8a8 CUTLASS kernels": the PR description's bullet list
// fixes the operation and its scale granularities; the misaligned-address
// report fixes B as K x N column-major, i.e. rows of an [N, K] weight.)
//
// The contraction runs on the CDNA4 matrix cores, fp32 accumulation for fp8
// e4m3 (format 0 of the f8f6f4 MFMAs) and exact int32 for int8:
//  - gemm_tile_kernel (M > 64): block tiles of 256x256 down to 64x64 with
//    32 x 32 MFMAs (v_mfma_f32_32x32x64_f8f6f4, v_mfma_i32_32x32x32_i8),
//    operands staged in LDS by direct global -> LDS loads.
//  - gemm_decode_kernel (M <= 64, bound by the weight stream): 16 x 16 MFMAs
//    (v_mfma_f32_16x16x128_f8f6f4, v_mfma_i32_16x16x64_i8) on a block of
//    16 or 64 output columns, weights streamed once through an LDS ring;
//    above 16 rows, with a caller workspace, on weights too narrow to
//    occupy the GPU, split along K, the partial sums added by
//    splitk_reduce_kernel.
//  - gemm_dynq_kernel (M == 1): the per-token quantisation of the one row
//    and the product in one kernel.
// Each MFMA lane holds a run of contiguous K bytes of one row of each
// operand; the order of K inside a fragment differs from memory order, but A
// and B always share it, so the sum is the same.
// The epilogue is fused: scales applied in fp32 and the result rounded to
// nearest even into bf16/fp16 in registers, then stored once (the tile
// kernel through LDS, as whole rows).

#include <atomic>
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace w8a8 {

namespace {

struct GemmArgs {
    void* out;
    int64_t ldo;
    const uint8_t* a;
    int64_t lda;
    const uint8_t* b;
    int64_t ldb;
    int M, N, K;
    const float* sa;
    int sa_per_row;
    const float* sb;
    int sb_per_col;
    int tiles_m, tiles_n;
    int vec_out;  // out and ldo allow 4-element vector stores
    int vec_row;  // out and ldo allow 16-byte stores
    // split-K decode: splits > 1 workgroups per column block, each over
    // stages_per_split K stages, writing fp32 (int32 for int8) partial sums
    // [splits][M][N] to part; a second kernel adds them
    void* part;
    int splits, stages_per_split;
    int split_config;  // the decode configuration that runs split
    // asymmetric int8 activations: zero points (1 or M entries) and the
    // weights' code sums; NULL azp: symmetric
    const int32_t* azp;
    int azp_per_row;
    const int32_t* colsum;
};

template <int QT>
struct AccOf;
template <>
struct AccOf<Q_FP8> {
    typedef f32x4 type;
};
template <>
struct AccOf<Q_INT8> {
    typedef i32x4 type;
};

// c += A_frag . B_frag over one 128-byte K slice.
template <int QT>
__device__ __forceinline__ void mma(typename AccOf<QT>::type& c, const i32x8& a, const i32x8& b) {
    if constexpr (QT == Q_FP8) {
        // Zero scale operands select the unscaled instruction.
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    } else {
        const i32x4 alo = {a[0], a[1], a[2], a[3]}, ahi = {a[4], a[5], a[6], a[7]};
        const i32x4 blo = {b[0], b[1], b[2], b[3]}, bhi = {b[4], b[5], b[6], b[7]};
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi, c, 0, 0, 0);
    }
}

__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
    return i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                 static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                 static_cast<int>(hi[2]), static_cast<int>(hi[3])};
}

// Scale, round and store one accumulator element (bounds already checked).
// Asymmetric int8 activations: the accumulator of (a - z) . b is
// acc - z[m] * colsum[n], exact in int32 while K <= 65536 (|a - z| <= 255).
// Float accumulators (fp8) have no zero points.
template <typename T>
__device__ __forceinline__ T azp_fix(const GemmArgs& p, int m, int n, T acc) {
    if constexpr (std::is_integral<T>::value) {
        if (p.azp) return acc - p.azp[p.azp_per_row ? m : 0] * p.colsum[n];
    }
    return acc;
}

template <int OT, typename T>
__device__ __forceinline__ void store_out(const GemmArgs& p, int m, int n, T acc) {
    acc = azp_fix(p, m, n, acc);
    if constexpr (OT == D_I32) {
        static_cast<int32_t*>(p.out)[static_cast<int64_t>(m) * p.ldo + n] = static_cast<int32_t>(acc);
    } else {
        const float sa = p.sa ? p.sa[p.sa_per_row ? m : 0] : 1.0f;
        const float sb = p.sb ? p.sb[p.sb_per_col ? n : 0] : 1.0f;
        const float d = static_cast<float>(acc) * sa * sb;
        const int64_t o = static_cast<int64_t>(m) * p.ldo + n;
        if constexpr (OT == D_BF16) static_cast<uint16_t*>(p.out)[o] = to_bf16_bits(d);
        else if constexpr (OT == D_FP16) static_cast<uint16_t*>(p.out)[o] = to_fp16_bits(d);
        else static_cast<float*>(p.out)[o] = d;
    }
}

// store_out with the row's scale given in a register.
template <int OT, typename T>
__device__ __forceinline__ void store_scaled(const GemmArgs& p, int m, int n, T acc, float sa) {
    const float sb = p.sb ? p.sb[p.sb_per_col ? n : 0] : 1.0f;
    const float d = static_cast<float>(acc) * sa * sb;
    const int64_t o = static_cast<int64_t>(m) * p.ldo + n;
    if constexpr (OT == D_BF16) static_cast<uint16_t*>(p.out)[o] = to_bf16_bits(d);
    else if constexpr (OT == D_FP16) static_cast<uint16_t*>(p.out)[o] = to_fp16_bits(d);
    else static_cast<float*>(p.out)[o] = d;
}

// Block id -> (tile_m, tile_n). Consecutive logical tiles share an XCD, and
// the walk goes down groups of 8 row-tiles before moving to the next column.
__device__ __forceinline__ bool tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int rpid = (pid % 8) * per_xcd + pid / 8;
    if (rpid >= total) return false;
    constexpr int kGroup = 8;
    const int in_group = kGroup * tiles_n;
    const int first_m = (rpid / in_group) * kGroup;
    const int gsz = min(tiles_m - first_m, kGroup);
    const int r = rpid % in_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
    return true;
}

constexpr int kBK = 128;  // K bytes per slice (one MFMA depth for fp8)

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (buffer_load_dwordx4 ... lds): lane q of the
// issuing wave writes its 16 bytes at lds + 16 * q; an offset at or beyond the
// resource's byte count reads as zero, which masks the tile edges.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint32_t* lds_u32p;
__device__ void raw_buffer_load_lds(i32x4 rsrc, lds_u32p lds, int size, int voffset, int soffset,
                                    int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

constexpr int kOutOfRange = 0x7FFFFFF0;

// The same load written as inline asm, for the ring loops that wait for
// their stages themselves: the compiler does not see these loads, so it
// neither waits for all of them before each barrier (its workgroup fence
// otherwise covers every direct-to-LDS load in flight, which keeps only one
// stage in flight whatever the ring depth) nor before each LDS read. Every
// wait for them is an explicit s_waitcnt vmcnt (wait_stages); loads retire
// in issue order. No register result.
template <bool NT>
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, const void* lds, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u32p)(const_cast<void*>(lds)))));
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                     :
                     : "v"(voffset), "s"(rsrc), "s"(m0)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :
                     : "v"(voffset), "s"(rsrc), "s"(m0)
                     : "memory", "m0");
}

__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t nbytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = static_cast<int>(static_cast<uint32_t>(a));
    r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu);  // stride 0
    r[2] = static_cast<int>(nbytes);
    r[3] = 0x00020000;  // raw buffer, 32-bit data format
    return r;
}

// LDS layout of a tile stage: every operand row keeps its 128 K bytes in
// one 128-byte LDS row, 32-row groups of 4 KB one after another. The 16-byte
// chunk c of row r sits at slot c ^ ((r / 2) % 8), so that the 32 x 32
// fragment reads below (lanes 0..31 on rows 0..31 at one chunk, lanes
// 32..63 two chunks further) meet every LDS bank once per 16 lanes. One
// wave-wide direct load fills 8 rows x 128 bytes: whole cache lines.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

template <int QT>
struct Acc32Of;
template <>
struct Acc32Of<Q_FP8> {
    typedef f32x16 type;
};
template <>
struct Acc32Of<Q_INT8> {
    typedef i32x16 type;
};

// The 32-byte fragment of K half h (bytes 64h .. 64h+63) for one 32-row
// group: lane l takes row l % 32, K bytes 64h + 32 (l / 32) .. +31 (the
// operand layout of v_mfma_f32_32x32x64_f8f6f4).
__device__ __forceinline__ i32x8 frag32(const uint8_t* group, int h, int lane) {
    const int r = lane & 31, sw = (r >> 1) & 7;
    const int c = 4 * h + 2 * (lane >> 5);
    const uint8_t* row = group + r * 128;
    return join(*reinterpret_cast<const u32x4*>(row + 16 * (c ^ sw)),
                *reinterpret_cast<const u32x4*>(row + 16 * ((c + 1) ^ sw)));
}

// c += W_frag . X_frag over one 64-byte K half: the weight fragment is the
// first operand, so the result's 32 x 32 tile has output columns (n) along
// its rows and output rows (m) along lanes. int8 splits the half into two
// 32-deep products over the fragment's two 16-byte words; both operands
// take the same words, so the integer sum is unchanged.
template <int QT>
__device__ __forceinline__ void mma32(typename Acc32Of<QT>::type& c, const i32x8& w, const i32x8& x) {
    if constexpr (QT == Q_FP8) {
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, c, 0, 0, 0, 0, 0, 0);
    } else {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{w[0], w[1], w[2], w[3]},
                                                  i32x4{x[0], x[1], x[2], x[3]}, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{w[4], w[5], w[6], w[7]},
                                                  i32x4{x[4], x[5], x[6], x[7]}, c, 0, 0, 0);
    }
}

// Scale, round and store the 4 consecutive columns n..n+3 of row m.
template <int OT, typename Acc>
__device__ __forceinline__ void store4(const GemmArgs& p, int m, int n, const Acc& acc, int base,
                                       bool vec) {
    if (m >= p.M) return;
    typedef typename std::remove_cv<typename std::remove_reference<decltype(acc[0])>::type>::type E;
    E v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = azp_fix(p, m, min(n + r, p.N - 1), static_cast<E>(acc[base + r]));
    if constexpr (OT == D_I32) {
        int32_t* o = static_cast<int32_t*>(p.out) + static_cast<int64_t>(m) * p.ldo + n;
        if (vec && n + 3 < p.N) {
            *reinterpret_cast<i32x4*>(o) =
                i32x4{static_cast<int>(v[0]), static_cast<int>(v[1]),
                      static_cast<int>(v[2]), static_cast<int>(v[3])};
        } else {
            for (int r = 0; r < 4; ++r)
                if (n + r < p.N) o[r] = static_cast<int32_t>(v[r]);
        }
    } else {
        const float sa = p.sa ? p.sa[p.sa_per_row ? m : 0] : 1.0f;
        float d[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float sb = p.sb ? p.sb[p.sb_per_col ? min(n + r, p.N - 1) : 0] : 1.0f;
            d[r] = static_cast<float>(v[r]) * sa * sb;
        }
        const int64_t o = static_cast<int64_t>(m) * p.ldo + n;
        if constexpr (OT == D_F32) {
            float* out = static_cast<float*>(p.out) + o;
            if (vec && n + 3 < p.N) {
                *reinterpret_cast<f32x4*>(out) = f32x4{d[0], d[1], d[2], d[3]};
            } else {
                for (int r = 0; r < 4; ++r)
                    if (n + r < p.N) out[r] = d[r];
            }
        } else {
            uint16_t h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[r] = (OT == D_BF16) ? to_bf16_bits(d[r]) : to_fp16_bits(d[r]);
            uint16_t* out = static_cast<uint16_t*>(p.out) + o;
            if (vec && n + 3 < p.N) {
                *reinterpret_cast<u32x2*>(out) = u32x2{h[0] | (static_cast<uint32_t>(h[1]) << 16),
                                                       h[2] | (static_cast<uint32_t>(h[3]) << 16)};
            } else {
                for (int r = 0; r < 4; ++r)
                    if (n + r < p.N) out[r] = h[r];
            }
        }
    }
}

// Wait until at most `pending` (<= P) stages of L loads each are still in
// flight; loads retire in issue order.
template <int P, int L>
__device__ __forceinline__ void wait_stages(int pending) {
    if constexpr (P == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        if (pending >= P) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(P * L) : "memory");
        else wait_stages<P - 1, L>(pending);
    }
}

// BM x BN block tile; WGM x WGN waves, each owning a (BM/WGM) x (BN/WGN)
// wave tile of 32 x 32 MFMA tiles. K is walked in 128-byte stages through an
// ST-slot LDS ring filled by direct loads: while stage k is consumed the
// loads of stages k+1 .. k+ST-1 are in flight, one barrier per stage (small
// tiles do little work per stage, so they keep more stages in flight to
// cover the memory latency). Inside a stage the fragments of the next
// 64-byte half are read from LDS while the MFMAs of the current half run
// (two register sets, interleaved by the scheduler hints below).
template <int QT, int OT, int BM, int BN, int WGM, int WGN, int ST>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_tile_kernel(GemmArgs p) {
    typedef typename Acc32Of<QT>::type Acc;
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int kGroup = 32 * kBK;          // one 32-row group of a stage
    constexpr int kStage = (BM + BN) * kBK;
    constexpr int kLoads = (BM + BN) / 8;     // 1 KB wave-wide loads per stage
    constexpr int kLPW = kLoads / NW;
    constexpr int kMfma = TM * TN * (QT == Q_FP8 ? 1 : 2), kReads = 2 * (TM + TN);
    constexpr int kReadsPerMfma = (kReads + kMfma - 1) / kMfma;
    static_assert(TM >= 1 && TN >= 1 && kLoads % NW == 0, "tile shape");
    static_assert(ST >= 2 && kLPW * (ST - 2) <= 63, "loads in flight");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * kStage];
    __shared__ float scl[BM + BN];  // the tile's row scales, then its column scales
    __shared__ int32_t zcs[QT == Q_INT8 ? BM + BN : 1];  // its zero points, then its code sums
    static_assert(NW * 64 >= BM + BN, "one thread per row and column scale");

    int tm, tn;
    if (!tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn)) return;
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;

    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
    const i32x4 ra = buffer_rsrc(p.a + static_cast<int64_t>(m0) * p.lda,
                                 static_cast<uint32_t>((rows_a - 1) * p.lda + p.K));
    const i32x4 rb = buffer_rsrc(p.b + static_cast<int64_t>(n0) * p.ldb,
                                 static_cast<uint32_t>((rows_b - 1) * p.ldb + p.K));

    // Load j of this wave: 8 rows x 128 bytes; lane q reads row 8 (i % 4) + q / 8
    // of 32-row group i / 4, the 16-byte chunk that lands at slot q % 8.
    int base_off[kLPW], kin[kLPW];
#pragma unroll
    for (int j = 0; j < kLPW; ++j) {
        const int i = wave + NW * j;
        const bool is_a = i < BM / 8;
        const int ii = is_a ? i : i - BM / 8;
        const int r = 8 * (ii & 3) + (lane >> 3);
        const int row = 32 * (ii >> 2) + r;
        kin[j] = 16 * ((lane & 7) ^ ((r >> 1) & 7));
        base_off[j] = (row < (is_a ? rows_a : rows_b))
                          ? row * static_cast<int>(is_a ? p.lda : p.ldb) + kin[j]
                          : kOutOfRange;
    }
    auto issue = [&](int kt, int buf) {
        uint8_t* st = smem + buf * kStage;
#pragma unroll
        for (int j = 0; j < kLPW; ++j) {
            const int i = wave + NW * j;
            const bool is_a = i < BM / 8;
            const bool ok = base_off[j] != kOutOfRange && kt * kBK + kin[j] < p.K;
            const int off = ok ? base_off[j] + kt * kBK : kOutOfRange;
            buffer_load_lds16<false>(is_a ? ra : rb, st + (is_a ? 0 : BM * kBK) + (is_a ? i : i - BM / 8) * 1024,
                                     off);
        }
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    i32x8 xa[TM], wa[TN], xb[TM], wb[TN];  // two fragment sets
    auto read = [&](i32x8* x, i32x8* w, int buf, int h) {
        const uint8_t* sa = smem + buf * kStage;
        const uint8_t* sb = sa + BM * kBK;
#pragma unroll
        for (int i = 0; i < TM; ++i) x[i] = frag32(sa + (wm * TM + i) * kGroup, h, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) w[j] = frag32(sb + (wn * TN + j) * kGroup, h, lane);
    };
    auto mfmas = [&](const i32x8* x, const i32x8* w) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) mma32<QT>(acc[i][j], w[j], x[i]);
    };
    // Scheduler hint: alternate one MFMA with a few LDS reads.
    auto interleave = [&]() {
#pragma unroll
        for (int t = 0; t < kMfma; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, kReadsPerMfma, 0);
        }
    };

    // The 2-byte-output epilogue's scales (and for asymmetric int8 the zero
    // points and code sums), one per thread (rows and columns past the
    // matrix clamped), loaded now and kept in registers through the main
    // loop, so that the epilogue does not start with a memory round trip
    // (measured on MI355X: 8192 x 28672 x 4096 763 -> 754 us, 2048 x 6144 x
    // 4096 53.2 -> 51.7 us).
    float scale_pre = 1.0f;
    int32_t zcs_pre = 0;
    if constexpr (OT == D_BF16 || OT == D_FP16) {
        const int t = threadIdx.x;
        const bool azp = QT == Q_INT8 && p.azp;
        if (t < BM) {
            const int m = min(m0 + t, p.M - 1);
            scale_pre = p.sa ? p.sa[p.sa_per_row ? m : 0] : 1.0f;
            if (azp) zcs_pre = p.azp[p.azp_per_row ? m : 0];
        } else if (t < BM + BN) {
            const int n = min(n0 + t - BM, p.N - 1);
            scale_pre = p.sb ? p.sb[p.sb_per_col ? n : 0] : 1.0f;
            if (azp) zcs_pre = p.colsum[n];
        }
    }
    const int KT = (p.K + kBK - 1) / kBK;
    if (KT > 0) {
        issue(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int s = 1; s < ST; ++s)
            if (s < KT) issue(s, s);
        read(xa, wa, 0, 0);
        int cur = 0;
        for (int kt = 0; kt + 1 < KT; ++kt) {
            const int nxt = cur + 1 == ST ? 0 : cur + 1;
            read(xb, wb, cur, 1);  // half 1 of stage kt, while half 0 runs
            mfmas(xa, wa);
            interleave();
            // stage kt+1 has landed once at most the stages issued after it
            // (kt+2 .. min(KT-1, kt+ST-1)) are pending
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            wait_stages<ST - 2, kLPW>(min(KT - 2 - kt, ST - 2));
            __syncthreads();  // ... in every wave; every wave is done reading stage kt
            if (kt + ST < KT) issue(kt + ST, cur);
            read(xa, wa, nxt, 0);  // half 0 of stage kt+1, while half 1 of kt runs
            mfmas(xb, wb);
            interleave();
            cur = nxt;
        }
        read(xb, wb, cur, 1);
        mfmas(xa, wa);
        interleave();
        mfmas(xb, wb);
    }

    // Fused epilogue. In a 32 x 32 tile lane l holds, for q = 0..3, output
    // row m = l % 32 and the 4 consecutive columns n = 8q + 4 (l / 32) + 0..3.
    if constexpr (OT == D_BF16 || OT == D_FP16) {
        // 2-byte outputs are scaled and rounded into a BM x BN tile in the
        // (now idle) LDS ring, then stored as whole rows, 16 bytes per lane:
        // direct stores of the fragments would write 32 partial cache lines
        // per instruction. Chunk c (8 columns) of tile row r sits at slot
        // c ^ (r % (BN / 8)).
        constexpr int kChunks = BN / 8;
        constexpr int kRowsPerAccess = 64 / kChunks;
        static_assert(BM * BN * 2 <= ST * kStage, "the output tile fits the LDS ring");
        if (threadIdx.x < BM + BN) {
            scl[threadIdx.x] = scale_pre;
            if constexpr (QT == Q_INT8) zcs[threadIdx.x] = zcs_pre;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();  // every wave is done reading the ring; scl is written
        // The lane's TM row scales (and zero points) are read once; its 16
        // column scales (and code sums) of each 32-column group j just
        // before that group is written, so that few stay live at a time.
        float sav[TM];
        int zv[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            sav[i] = scl[wm * WM + i * 32 + (lane & 31)];
            zv[i] = 0;
            if constexpr (QT == Q_INT8)
                if (p.azp) zv[i] = zcs[wm * WM + i * 32 + (lane & 31)];
        }
        // The tile into LDS; the zero-point term is compiled in only where used.
        auto write_tile = [&](auto with_azp) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                float sbv[16];
                int csv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int col = wn * WN + j * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    sbv[e] = scl[BM + col];
                    csv[e] = 0;
                    if constexpr (decltype(with_azp)::value) csv[e] = zcs[BM + col];
                }
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int row = wm * WM + i * 32 + (lane & 31);
                    const float sa = sav[i];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = wn * WN + j * 32 + 8 * q + 4 * (lane >> 5);
                        uint16_t h[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            auto a = acc[i][j][4 * q + r];
                            if constexpr (decltype(with_azp)::value) a -= zv[i] * csv[4 * q + r];
                            const float d = static_cast<float>(a) * sa * sbv[4 * q + r];
                            h[r] = (OT == D_BF16) ? to_bf16_bits(d) : to_fp16_bits(d);
                        }
                        const int slot = (col >> 3) ^ (row % kChunks);
                        *reinterpret_cast<u32x2*>(smem + row * (BN * 2) + slot * 16 + (col & 7) * 2) =
                            u32x2{h[0] | (static_cast<uint32_t>(h[1]) << 16),
                                  h[2] | (static_cast<uint32_t>(h[3]) << 16)};
                    }
                }
            }
        };
        if (QT == Q_INT8 && p.azp) write_tile(std::true_type{});
        else write_tile(std::false_type{});
        __syncthreads();
        const bool vec = p.vec_row;
#pragma unroll 4
        for (int r0 = wave * kRowsPerAccess; r0 < BM; r0 += NW * kRowsPerAccess) {
            const int row = r0 + lane / kChunks, c = lane % kChunks;
            const u32x4 v = *reinterpret_cast<const u32x4*>(smem + row * (BN * 2) + 16 * (c ^ (row % kChunks)));
            const int m = m0 + row, n = n0 + 8 * c;
            if (m >= p.M || n >= p.N) continue;
            uint16_t* out = static_cast<uint16_t*>(p.out) + static_cast<int64_t>(m) * p.ldo + n;
            if (vec && n + 7 < p.N) {
                // non-temporal: the tile is written once and not read back here;
                // normal stores leave the L2 full of dirty lines that hold up
                // the acknowledgements (measured 12% slower on 8192 x 28672)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out));
            } else {
                for (int e = 0; e < 8 && n + e < p.N; ++e)
                    out[e] = static_cast<uint16_t>(v[e >> 1] >> (16 * (e & 1)));
            }
        }
    } else {
        const bool vec = p.vec_out;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm * WM + i * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * (lane >> 5);
                    if (n < p.N) store4<OT>(p, m, n, acc[i][j], 4 * q, vec);
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode kernel, M <= 16*MT <= 64 rows: the weight stream from HBM bounds it.
// A workgroup (4 waves) owns CB output columns (16 or 64) over all of K. K is
// walked in stages of CH bytes through an ST-deep LDS ring; a stage holds the
// CB weight rows and the 16*MT activation rows, filled by direct global -> LDS
// loads in which each wave-wide load reads 1 KB of contiguous bytes (1024/CH
// whole row segments). The 16-byte chunk c of row r is stored at slot
// c ^ (r % 16), so the 16-row fragment reads of the MFMAs spread over all LDS
// banks. Weight loads are non-temporal: they are read once.
//  - CB = 64: wave w computes columns 16w .. 16w+15 over every K slice.
//  - CB = 16: wave w computes the block's 16 columns over the stage's K slices
//    w, w+4, ...; the four partial sums are added through LDS in a fixed order.
// Activation rows past M read as zeros; their results are never stored.
// ---------------------------------------------------------------------------
constexpr int kNonTemporal = 2;  // cache-policy operand of the buffer load: nt

template <int QT, int OT, int CB, int MT, int CH, int ST>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs p) {
    typedef typename AccOf<QT>::type Acc;
    constexpr int AROWS = 16 * MT;
    constexpr int STAGE = (CB + AROWS) * CH;
    constexpr int WL = CB * CH / 4096, AL = AROWS * CH / 4096;  // loads per wave per stage
    constexpr int LPW = WL + AL;
    constexpr int SL = CH / kBK;  // 128-byte K slices per stage
    constexpr int NCG = CB / 16, WPG = 4 / NCG;  // 16-column groups; waves per group
    static_assert(CB == 16 || CB == 32 || CB == 64, "columns per workgroup");
    static_assert(CH % 256 == 0 && WL >= 1 && AL >= 1, "stage shape");
    static_assert(SL % WPG == 0, "slices per wave");
    static_assert(ST >= 2 && LPW * (ST - 2) <= 63, "loads in flight");
    static_assert(ST * STAGE >= 4 * MT * 64 * 16, "room for the wave reduction");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = p.splits > 1 ? p.splits : 1;
    const int sp = blockIdx.x % S;
    const int n0 = (blockIdx.x / S) * CB;
    const int nst_all = (p.K + CH - 1) / CH;
    const int s0 = S > 1 ? sp * p.stages_per_split : 0;  // this workgroup's K stages
    const int s1 = S > 1 ? min(nst_all, s0 + p.stages_per_split) : nst_all;
    const int nst = max(s1 - s0, 0);
    const int kend = min(p.K, s1 * CH);
    const int mt = (p.M + 15) / 16;
    const int wrows = min(CB, p.N - n0);
    const int lda = static_cast<int>(p.lda), ldb = static_cast<int>(p.ldb);
    const i32x4 rb = buffer_rsrc(p.b + static_cast<int64_t>(n0) * p.ldb,
                                 static_cast<uint32_t>((wrows - 1) * ldb + p.K));
    const i32x4 ra = buffer_rsrc(p.a, static_cast<uint32_t>((p.M - 1) * lda + p.K));
    // Workgroups walk their K stages from different starting points: with
    // all of them at the same K offset, weight rows 4096 * j bytes apart land
    // on the same few HBM channels at once (a pure stream of 28672 x 4096
    // weights: 5.2 -> 6.1 TB/s). Measured per configuration on MI355X: a
    // 4-9% gain with one 16-row activation tile; with four (64 tokens) the
    // activation reads spread out and it is neutral to 18% slower, so those
    // keep the common order. The start is 5 x the block index (mod the stage
    // count) rather than the block index itself: 0.5-1% faster on the
    // 28672 x 4096 and 57344 x 8192 weights (A/B, repeated in one process).
    const int rot = (MT == 1 && ldb % 4096 == 0 && nst > 0) ? ((blockIdx.x / S) * 5) % nst : 0;

    auto issue = [&](int st, int buf) {
        const int ls = st + rot < nst ? st + rot : st + rot - nst;
        const int k0 = (s0 + ls) * CH;
        uint8_t* base = smem + buf * STAGE;
#pragma unroll
        for (int j = 0; j < WL + AL; ++j) {
            const bool is_w = j < WL;
            const int t = wave + 4 * (is_w ? j : j - WL);  // 1 KB piece of the operand's tile
            const int o = t * 1024 + 16 * lane;
            const int r = o / CH, c = ((o % CH) >> 4) ^ (r & 15);
            const int k = k0 + 16 * c;
            const bool ok = r < (is_w ? wrows : p.M) && k < kend;
            const int off = ok ? r * (is_w ? ldb : lda) + k : kOutOfRange;
            if (is_w)
                buffer_load_lds16<true>(rb, base + t * 1024, off);
            else
                buffer_load_lds16<false>(ra, base + CB * CH + t * 1024, off);
        }
    };

    Acc acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = Acc{0, 0, 0, 0};

#pragma unroll
    for (int st = 0; st < ST - 1; ++st)
        if (st < nst) issue(st, st);
    const int g = lane >> 4, r16 = lane & 15;
    for (int st = 0; st < nst; ++st) {
        // Wait for this stage's loads; later stages' loads stay in flight.
        wait_stages<ST - 2, LPW>(min(nst - 1 - st, ST - 2));
        __syncthreads();  // every wave's loads of this stage have landed
        if (st + ST - 1 < nst) issue(st + ST - 1, (st + ST - 1) % ST);  // slot freed last step
        const uint8_t* wb = smem + (st % ST) * STAGE;
        const uint8_t* ab = wb + CB * CH;
        const uint8_t* wrow = wb + (16 * (wave / WPG) + r16) * CH;
#pragma unroll
        for (int uu = 0; uu < SL / WPG; ++uu) {
            const int u = WPG * uu + wave % WPG;
            // lane's fragment: K bytes 32g .. 32g+31 of slice u (chunks 8u+2g, 8u+2g+1)
            const int c0 = (8 * u + 2 * g) ^ r16, c1 = (8 * u + 2 * g + 1) ^ r16;
            const i32x8 wf = join(*reinterpret_cast<const u32x4*>(wrow + 16 * c0),
                                  *reinterpret_cast<const u32x4*>(wrow + 16 * c1));
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if (i >= mt) break;
                const uint8_t* arow = ab + (16 * i + r16) * CH;
                const i32x8 af = join(*reinterpret_cast<const u32x4*>(arow + 16 * c0),
                                      *reinterpret_cast<const u32x4*>(arow + 16 * c1));
                mma<QT>(acc[i], af, wf);
            }
        }
    }

    // In a 16 x 16 tile lane l holds rows 4 (l / 16) + r, r < 4, of column l % 16.
    // Each result goes out scaled (no split) or as a plain partial sum of this
    // workgroup's K range (split K). The scales (and zero-point operands) of
    // a tile's four outputs are all loaded before the first store, at
    // clamped indices: loads under each store's own bounds check were waited
    // for one at a time.
    typedef typename std::conditional<QT == Q_FP8, float, int32_t>::type Part;
    Part* part = static_cast<Part*>(p.part) + static_cast<int64_t>(sp) * p.M * p.N;
    auto put4 = [&](int i, int n, const Acc& v) {
        const int m0 = 16 * i + 4 * g;
        if (S > 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (m0 + r < p.M && n < p.N) part[static_cast<int64_t>(m0 + r) * p.N + n] = static_cast<Part>(v[r]);
            return;
        }
        const int nc = min(n, p.N - 1);
        const float sb = p.sb ? p.sb[p.sb_per_col ? nc : 0] : 1.0f;
        float sa[4];
        int32_t z[4] = {0, 0, 0, 0};
        int32_t cs = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int mc = min(m0 + r, p.M - 1);
            sa[r] = p.sa ? p.sa[p.sa_per_row ? mc : 0] : 1.0f;
            if constexpr (QT == Q_INT8)
                if (p.azp) z[r] = p.azp[p.azp_per_row ? mc : 0];
        }
        if constexpr (QT == Q_INT8)
            if (p.azp) cs = p.colsum[nc];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + r;
            if (m < p.M && n < p.N) {
                auto acc_r = v[r];
                if constexpr (QT == Q_INT8)
                    if (p.azp) acc_r -= z[r] * cs;
                const int64_t o = static_cast<int64_t>(m) * p.ldo + n;
                if constexpr (OT == D_I32) {
                    static_cast<int32_t*>(p.out)[o] = static_cast<int32_t>(acc_r);
                } else {
                    const float d = static_cast<float>(acc_r) * sa[r] * sb;
                    if constexpr (OT == D_BF16) static_cast<uint16_t*>(p.out)[o] = to_bf16_bits(d);
                    else if constexpr (OT == D_FP16) static_cast<uint16_t*>(p.out)[o] = to_fp16_bits(d);
                    else static_cast<float*>(p.out)[o] = d;
                }
            }
        }
    };
    if constexpr (WPG == 1) {
        const int n = n0 + 16 * wave + r16;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i >= mt) break;
            put4(i, n, acc[i]);
        }
    } else {
        // The WPG waves of a column group hold sums over disjoint K slices:
        // added through LDS in wave order, a fixed order.
        __syncthreads();  // the ring is free
        Acc* red = reinterpret_cast<Acc*>(smem);
#pragma unroll
        for (int i = 0; i < MT; ++i) red[(wave * MT + i) * 64 + lane] = acc[i];
        __syncthreads();
        const int cg = wave / WPG, first = cg * WPG;
        const int n = n0 + 16 * cg + r16;
        for (int i = wave % WPG; i < mt; i += WPG) {
            Acc sum = red[(first * MT + i) * 64 + lane];
#pragma unroll
            for (int w = 1; w < WPG; ++w) sum += red[((first + w) * MT + i) * 64 + lane];
            put4(i, n, sum);
        }
    }
}

// ---------------------------------------------------------------------------
// One-token decode with the activation quantised in place (M == 1): dynamic
// per-token quantisation of x followed by the scaled product, in one kernel.
// Every workgroup (4 waves, 16 output columns) quantises the whole row x
// itself (a few KB, L2-resident once the first workgroups have read it) with
// the per-token quantizer's arithmetic: the same maximum, scale and
// correctly rounded division, so codes and scale are bit-identical to
// w8a8_quant_per_token. The codes stay in LDS; workgroup 0 also writes them
// and the scale to memory at the end. The weight rows stream through a
// 4-slot LDS ring in chunks of 16 rows x 1 KB, three chunks in flight. The
// row x is requested before the weights: loads retire in issue order, so the
// quantisation then waits only for x (the first chunks are compiler-visible
// loads, which it counts; the later ones are the inline-asm loads with
// explicit waits, and the barriers carry no fence, so that no wait drains
// the ring). Weight chunk c of row r sits at slot c ^ (r % 16).
// ---------------------------------------------------------------------------
constexpr int kDynqChunk = 1024;       // K bytes of weight per chunk
constexpr int kDynqSlots = 4;          // chunks in the LDS ring
constexpr int kDynqMaxK = 15360;       // longest row quantised in LDS (two workgroups per CU)

template <int XT, int QT, int OT>
__global__ __launch_bounds__(256) void gemm_dynq_kernel(GemmArgs p, const void* __restrict__ x,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ x_scale) {
    typedef typename AccOf<QT>::type Acc;
    constexpr int CH = kDynqChunk;
    constexpr int WL = 16 * CH / 4096;  // weight loads per wave per chunk
    constexpr int SW = CH / kBK / 4;    // slices per wave per chunk
    constexpr int kGroups = (kDynqMaxK + 2047) / 2048;  // 8-element groups of x per thread
    constexpr int NB = kDynqSlots;
    __shared__ __attribute__((aligned(1024))) uint8_t wbuf[NB][16 * CH];
    __shared__ __attribute__((aligned(16))) uint8_t arow[kDynqMaxK];
    __shared__ float part[4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16;
    const int K = p.K;
    const int nch = (K + CH - 1) / CH;
    const int wrows = min(16, p.N - n0);
    const int ldb = static_cast<int>(p.ldb);
    const i32x4 rb = buffer_rsrc(p.b + static_cast<int64_t>(n0) * p.ldb,
                                 static_cast<uint32_t>((wrows - 1) * ldb + K));
    // chunk order rotated per workgroup, as in the decode kernel
    const int rot = (ldb % 4096 == 0 && nch > 0) ? blockIdx.x % nch : 0;
    auto chunk_k = [&](int ci) { return (ci + rot < nch ? ci + rot : ci + rot - nch) * CH; };
    auto chunk = [&](int ci, int buf, bool visible) {
        const int kc = chunk_k(ci);
#pragma unroll
        for (int j = 0; j < WL; ++j) {
            const int t = wave + 4 * j;
            const int o = t * 1024 + 16 * lane;
            const int r = o / CH, c = ((o % CH) >> 4) ^ (r & 15);
            const int k = kc + 16 * c;
            const int off = (r < wrows && k < K) ? r * ldb + k : kOutOfRange;
            if (visible)
                raw_buffer_load_lds(rb, (lds_u32p)(wbuf[buf] + t * 1024), 16, off, 0, 0, kNonTemporal);
            else
                buffer_load_lds16<true>(rb, wbuf[buf] + t * 1024, off);
        }
    };
    // A barrier without the workgroup fence of __syncthreads (which would
    // wait for every direct load in flight): LDS stores are waited for here,
    // the ring's loads by their explicit waits.
    auto barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    // x first, then the first weight chunks.
    // All of the thread's loads of x are issued, unconditionally and
    // before the first is used, so that the compiler's wait for them counts
    // the weight loads issued after them (groups past K load the row's first
    // 8 elements, one cache line, and are not used).
    u32x4 raw[kGroups][2];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const int k = 8 * threadIdx.x + 2048 * j;
        load8_raw<XT>(x, k < K ? k : 0, raw[j]);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ci = 0; ci < NB - 1; ++ci)
        if (ci < nch) chunk(ci, ci, true);

    // The row's maximum |x|, its scale and its codes (into LDS).
    float v[kGroups][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        if (2048 * j >= K) break;
        widen8<XT>(raw[j], v[j]);
        if (8 * static_cast<int>(threadIdx.x) + 2048 * j < K)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
    amax = wave_max(amax);
    if (lane == 0) part[wave] = amax;
    barrier();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float s = scale_from_absmax<QT>(amax);
    const double rcp = 1.0 / static_cast<double>(s);
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const int k = 8 * threadIdx.x + 2048 * j;
        if (k < K) *reinterpret_cast<u32x2*>(arow + k) = quant8<QT>(v[j], rcp);
    }

    const int g = lane >> 4, r16 = lane & 15;
    const u32x4 z = {0, 0, 0, 0};
    Acc acc = Acc{0, 0, 0, 0};
    for (int ci = 0; ci < nch; ++ci) {
        // chunk ci has landed once at most the chunks issued after it are pending
        wait_stages<NB - 2, WL>(min(nch - 1 - ci, NB - 2));
        barrier();  // every wave's share of chunk ci (and the codes) is in LDS; slot (ci - 1) % NB is free
        const int kc = chunk_k(ci);
        const uint8_t* wrow = wbuf[ci % NB] + r16 * CH;
#pragma unroll
        for (int sv = 0; sv < SW; ++sv) {
            const int u = 4 * sv + wave;
            const int k = kc + u * kBK + 32 * g;  // this lane's 32 K bytes of the slice
            if (kc + u * kBK >= K) break;
            const int c0 = (8 * u + 2 * g) ^ r16, c1 = (8 * u + 2 * g + 1) ^ r16;
            const i32x8 wf = join(*reinterpret_cast<const u32x4*>(wrow + 16 * c0),
                                  *reinterpret_cast<const u32x4*>(wrow + 16 * c1));
            // only MFMA row 0 carries the token; the other rows multiply zeros
            const bool lo = r16 == 0 && k < K, hi = lo && k + 16 < K;
            const i32x8 af = join(lo ? *reinterpret_cast<const u32x4*>(arow + k) : z,
                                  hi ? *reinterpret_cast<const u32x4*>(arow + k + 16) : z);
            mma<QT>(acc, af, wf);
        }
        if (ci + NB - 1 < nch) chunk(ci + NB - 1, (ci + NB - 1) % NB, false);
    }

    // Add the four waves' sums in a fixed order; row 0 of column l % 16 is
    // element 0 of lanes 0..15.
    __syncthreads();  // every wave is done with the ring
    Acc* red = reinterpret_cast<Acc*>(wbuf[0]);
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0 && lane < 16) {
        Acc t = red[lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) t += red[w * 64 + lane];
        const int n = n0 + lane;
        if (n < p.N) store_scaled<OT>(p, 0, n, t[0], s);
    }
    if (blockIdx.x == 0) {  // the codes and the scale, for the caller
        for (int k = 16 * threadIdx.x; k < K; k += 16 * 256)
            *reinterpret_cast<u32x4*>(q + k) = *reinterpret_cast<const u32x4*>(arow + k);
        if (threadIdx.x == 0) *x_scale = s;
    }
}

// Split-K epilogue: D = scales * (sum of the splits' partial sums, added in
// split order), 4 elements per thread. Every load (partial sums at clamped
// indices, scales, zero-point operands) is issued before the first is used.
constexpr int kMaxSplitsK = 4;  // plan_splitk splits K at most 4 ways

template <int QT, int OT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p) {
    typedef typename std::conditional<QT == Q_FP8, float, int32_t>::type Part;
    const Part* part = static_cast<const Part*>(p.part);
    const int64_t plane = static_cast<int64_t>(p.M) * p.N;
    const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (e0 >= plane) return;
    Part v[kMaxSplitsK][4];
    float sa[4], sb[4];
    int32_t z[4] = {0, 0, 0, 0}, cs[4] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t e = min(e0 + r, plane - 1);
        const int m = static_cast<int>(e / p.N), n = static_cast<int>(e % p.N);
#pragma unroll
        for (int q = 0; q < kMaxSplitsK; ++q) v[q][r] = part[min(q, p.splits - 1) * plane + e];
        sa[r] = p.sa ? p.sa[p.sa_per_row ? m : 0] : 1.0f;
        sb[r] = p.sb ? p.sb[p.sb_per_col ? n : 0] : 1.0f;
        if constexpr (QT == Q_INT8) {
            if (p.azp) {
                z[r] = p.azp[p.azp_per_row ? m : 0];
                cs[r] = p.colsum[n];
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t e = e0 + r;
        if (e >= plane) break;
        Part sum = v[0][r];
#pragma unroll
        for (int q = 1; q < kMaxSplitsK; ++q)
            if (q < p.splits) sum += v[q][r];
        if constexpr (QT == Q_INT8)
            if (p.azp) sum -= z[r] * cs[r];
        const int64_t o = (e / p.N) * p.ldo + e % p.N;
        if constexpr (OT == D_I32) {
            static_cast<int32_t*>(p.out)[o] = static_cast<int32_t>(sum);
        } else {
            const float d = static_cast<float>(sum) * sa[r] * sb[r];
            if constexpr (OT == D_BF16) static_cast<uint16_t*>(p.out)[o] = to_bf16_bits(d);
            else if constexpr (OT == D_FP16) static_cast<uint16_t*>(p.out)[o] = to_fp16_bits(d);
            else static_cast<float*>(p.out)[o] = d;
        }
    }
}

template <int QT, int OT, int BM, int BN, int WGM, int WGN, int ST>
hipError_t run_tile(GemmArgs a, hipStream_t st) {
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    const int total = a.tiles_m * a.tiles_n;
    const int grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((gemm_tile_kernel<QT, OT, BM, BN, WGM, WGN, ST>), dim3(grid),
                       dim3(WGM * WGN * 64), 0, st, a);
    return hipGetLastError();
}

template <int QT, int OT, int CB, int MT, int CH, int ST>
hipError_t run_decode(const GemmArgs& a, hipStream_t st) {
    const int S = a.splits > 1 ? a.splits : 1;
    const int grid = (a.N + CB - 1) / CB * S;
    hipLaunchKernelGGL((gemm_decode_kernel<QT, OT, CB, MT, CH, ST>), dim3(grid), dim3(256), 0, st, a);
    if (S > 1) {
        const int64_t elems = static_cast<int64_t>(a.M) * a.N;
        hipLaunchKernelGGL((splitk_reduce_kernel<QT, OT>), dim3(static_cast<int>((elems + 1023) / 1024)),
                           dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

// The kernel configuration a problem runs with (shared by the launch and by
// scaled_mm_kernel_name, so that profiles can be matched to launches).
enum Config {
    kDecode64x16,    // gemm_decode_kernel, 64 columns, M <= 16 (stage 512 B, 2 stages)
    kDecode64x16R,   // the same, 4 stages of 256 B
    kDecode64x64,    // gemm_decode_kernel, 64 columns, M <= 64 (stage 256 B, 2 stages)
    kDecode16x16,    // gemm_decode_kernel, 16 columns, M <= 16 (stage 1 KB, 2 stages)
    kDecode16x16R,   // the same, 4 stages of 512 B
    kDecode16x64,    // gemm_decode_kernel, 16 columns, M <= 64 (stage 512 B, 2 stages)
    kDecode16x64R,   // the same, 3 stages
    kDecode16x16L,   // gemm_decode_kernel, 16 columns, M <= 16, long K (4 stages of 1 KB)
    kDecode16x64L,   // gemm_decode_kernel, 16 columns, M <= 64, long K (stage 1 KB, 2 stages)
    kTile256x256,    // gemm_tile_kernel 256 x 256, 8 waves, 2 stages
    kTile256x128,    // gemm_tile_kernel 256 x 128, 8 waves, 3 stages
    kTile128x128,    // gemm_tile_kernel 128 x 128, 4 waves, 2 stages
    kTile128x128R,   // gemm_tile_kernel 128 x 128, 8 waves, 3 stages (4 waves: 5% slower)
    kTile128x64,     // gemm_tile_kernel 128 x 64, 8 waves, 4 stages
    kTile64x64,      // gemm_tile_kernel 64 x 64, 4 waves, 4 stages
};

// 16-column workgroups on a long K that fill at most one per CU: a stage
// twice as long (the ring then fills a CU's LDS) keeps twice the bytes in
// flight. Measured on MI355X at 4096 x 14336: 16 -> 14.8 us (16 rows) and
// 28.8 -> 23.6 us (64 rows); with more workgroups than CUs the lost second
// workgroup per CU costs more than it gains. At up to 16 rows it pays on
// narrower weights too (A/B in one process: 1 x 1280 x 8192 7.4 -> 6.7 us,
// 1 x 2048 x 8192 8.9 -> 7.3, 1 x 1024 x 14336 10.3 -> 9.0, 16 x 2048 x
// 8192 9.3 -> 8.8); above 16 rows, 128 groups or fewer keep the 3-slot
// ring of 512-byte stages (or split K, given a workspace).
bool long_k_16(int64_t M, int64_t N, int64_t K) {
    const int64_t groups = (N + 15) / 16;
    return K >= 8192 && groups <= 256 && (M <= 16 || groups > 128);
}

// Ring depth: the direct loads of later stages stay in flight across the
// stage barriers, so a deeper ring keeps more bytes in flight per
// workgroup, at the cost of LDS and so of resident workgroups. Measured on
// MI355X (A/B, same process): deeper pays where the grid still fits one
// round of the deeper ring's resident workgroups, and loses where it then
// needs two (decode: 1 x 4096 x 4096 7.1 -> 6.0 us, 16 x 4096 x 14336 16.1
// -> 13.3, 64 x 4096 x 4096 11.6 -> 9.7, 1 x 28672 x 4096 21.3 -> 20.1, but
// 64 x 6144 x 4096 14.0 -> 17.0 and 1 x 57344 x 8192 72 -> 97; tiles:
// 512 x 4096 x 4096 26.3 -> 20.3, 512 x 4096 x 14336 81.9 -> 63.6,
// 1024 x 4096 x 4096 33.1 -> 25.5, 2048 x 4096 x 4096 43.7 -> 37.7, but
// 512 x 10240 x 8192 int8 on 128 x 128 tiles 73 -> 84).
Config select_config(int64_t M, int64_t N, int64_t K) {
    if (M <= 64) {
        // Measured on MI355X at the Llama-3 decode shapes: 64-column blocks
        // stream fastest once they still give every CU a block (N >= 16384);
        // narrower weights need 16-column blocks to reach every CU.
        const int64_t blocks64 = (N + 63) / 64, groups16 = (N + 15) / 16;
        if (blocks64 >= 256) {
            if (M > 16) return kDecode64x64;
            return blocks64 <= 512 ? kDecode64x16R : kDecode64x16;
        }
        if (long_k_16(M, N, K)) return M <= 16 ? kDecode16x16L : kDecode16x64L;
        if (M <= 16) return groups16 <= 384 ? kDecode16x16R : kDecode16x16;
        return groups16 <= 256 ? kDecode16x64R : kDecode16x64;
    }
    // The largest tile that still gives most CUs a block (measured on
    // MI355X, A/B in one process):
    //  - 256 x 256, else 256 x 128, from 160 tiles (five eighths of the
    //    CUs): one round of them beats more rounds of the next smaller tile,
    //    their longer main loops outweighing the idle CUs. 256 x 256: 2048 x
    //    5120 x 4096 51 us against 63 on 256 x 128, 3072 x 3584 x 4096 52
    //    against 61, 8192 x 1280 x 8192 101 against 115. 256 x 128: 4096 x
    //    1280 x 4096 31 against 37 on 128 x 128, 2048 x 3072 x 4096 31
    //    against 36, 4096 x 1280 x 14336 100 against 123, 512 x 10240 x 8192
    //    int8 59 against 73; at 120 to 128 tiles it loses (3072 x 1280 x
    //    8192 56 against 41).
    //  - Past 256 tiles of 128 x 128 (more than one round of its 3-slot
    //    ring), 256 x 128 from 144 tiles (640 x 6656 x 4096 30.3 us against
    //    33.3, 1152 x 3840 x 4096 30.1 against 32.4 on the 2-slot 128 x 128),
    //    else the 2-slot 128 x 128.
    //  - 128 x 64 tiles (eight 32 x 32 waves, a 96 KB ring: one workgroup per
    //    CU) where 192 to 256 of them fill one round: 512 x 4096 x 4096 20.2
    //    -> 17.1 us, 512 x 4096 x 14336 63.0 -> 51.1, 300 x 4096 x 4096 18.5
    //    -> 15.4, 128 x 16384 x 4096 27.2 -> 21.4 against 64 x 64, and 17.4
    //    against 20.9 on 128 x 128 at 512 x 4096 x 4096; past one round they
    //    lose (512 x 5120 x 4096, 320 tiles: 27.1 -> 30.5), and so they do
    //    below 192 (400 x 2048 x 8192, 128 tiles: 23.4 -> 27.7).
    //  - Else 128 x 128 (eight waves, 3 slots) from 128 tiles: against 64 x
    //    64, 512 x 5120 x 4096 21.4 us against 27.8, 640 x 4096 x 14336 66.7
    //    against 86.1, 512 x 4352 x 4096 (136 tiles) 21.1 against 24.6, 256 x
    //    8704 x 4096 22.7 against 29.0.
    //  - Else 64 x 64: below 128 tiles of 128 x 128 there are at most 508,
    //    one round of the 4-slot ring's resident workgroups.
    auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (tiles(256, 256) >= 160) return kTile256x256;
    if (tiles(256, 128) >= 160) return kTile256x128;
    if (tiles(128, 128) > 256) return tiles(256, 128) >= 144 ? kTile256x128 : kTile128x128;
    if (tiles(128, 64) >= 192 && tiles(128, 64) <= 256) return kTile128x64;
    if (tiles(128, 128) >= 128) return kTile128x128R;
    return kTile64x64;
}

template <int QT, int OT>
hipError_t dispatch(const GemmArgs& a, hipStream_t st) {
    switch (a.splits > 1 ? static_cast<Config>(a.split_config) : select_config(a.M, a.N, a.K)) {
        case kDecode64x16: return run_decode<QT, OT, 64, 1, 512, 2>(a, st);
        case kDecode64x16R: return run_decode<QT, OT, 64, 1, 256, 4>(a, st);
        case kDecode64x64: return run_decode<QT, OT, 64, 4, 256, 2>(a, st);
        case kDecode16x16: return run_decode<QT, OT, 16, 1, 1024, 2>(a, st);
        case kDecode16x16R: return run_decode<QT, OT, 16, 1, 512, 4>(a, st);
        case kDecode16x64: return run_decode<QT, OT, 16, 4, 512, 2>(a, st);
        case kDecode16x64R: return run_decode<QT, OT, 16, 4, 512, 3>(a, st);
        case kDecode16x16L: return run_decode<QT, OT, 16, 1, 1024, 4>(a, st);
        case kDecode16x64L: return run_decode<QT, OT, 16, 4, 1024, 2>(a, st);
        case kTile256x256: return run_tile<QT, OT, 256, 256, 2, 4, 2>(a, st);
        case kTile256x128: return run_tile<QT, OT, 256, 128, 4, 2, 3>(a, st);
        case kTile128x128: return run_tile<QT, OT, 128, 128, 2, 2, 2>(a, st);
        case kTile128x128R: return run_tile<QT, OT, 128, 128, 2, 4, 3>(a, st);
        case kTile128x64: return run_tile<QT, OT, 128, 64, 4, 2, 4>(a, st);
        case kTile64x64: return run_tile<QT, OT, 64, 64, 2, 2, 4>(a, st);
    }
    return hipErrorInvalidValue;  // not reached: select_config returns one of the above
}

template <int QT>
hipError_t dispatch_ot(int ot, const GemmArgs& a, hipStream_t st) {
    switch (ot) {
        case D_BF16: return dispatch<QT, D_BF16>(a, st);
        case D_FP16: return dispatch<QT, D_FP16>(a, st);
        case D_F32: return dispatch<QT, D_F32>(a, st);
        default:
            if constexpr (QT == Q_INT8) return dispatch<QT, D_I32>(a, st);
            return hipErrorInvalidValue;
    }
}

}  // namespace

// Split K for decode problems above 16 rows whose weights are too narrow to
// occupy the GPU, given a workspace:
//  - Narrow weights (at most 2048 rows, 128 sixteen-column groups) with
//    K >= 8192, or at most 1024 rows with K >= 4096: the 16-column kernel,
//    K split 4 ways (the 3-slot ring where each split walks at least 6 of
//    its 512-byte stages, or at K < 8192). Measured on MI355X (one process,
//    rotating weights), against the previous plans: 64 x 1280 x 8192 14.1
//    -> 11.4 us, 32 x 1280 x 8192 13.1 -> 10.2, 64 x 1024 x 14336 19.4 ->
//    11.6, 64 x 2048 x 8192 14.7 -> 12.2, 64 x 768 x 4096 8.8 -> 7.7; at K
//    = 4096 on 1280 to 3072 rows, and at 16 rows or fewer, no split was
//    faster.
//  - Wider weights with K >= 8192 that still give fewer than 256 64-column
//    blocks: the 64-column kernel, K split so that each activation tile is
//    read once per 64 columns instead of once per 16. The split count fills
//    one round of the kernel's workgroup slots (two 64 KB workgroups per CU
//    on 256 CUs), at most 4: Llama-3-70B QKV at 64 rows (160 column blocks)
//    33.6 us with 4 splits (640 workgroups, a second partial round) against
//    27.0 us with 3, and Llama-3-8B down 26.4 us on the long-stage 16-column
//    kernel against 24.0 us with 4 splits (24.4 us with 8). Shorter K does
//    not repay the extra pass there (Llama-3-8B QKV and O at 64 rows: 14.2
//    -> 17.3 us, 11.6 -> 14.7 us).
SplitPlan plan_splitk(int64_t M, int64_t N, int64_t K) {
    SplitPlan d{1, 0, 0, kDecode64x64};
    if (M <= 16 || M > 64) return d;
    const int64_t groups = (N + 15) / 16, blocks = (N + 63) / 64;
    if ((groups <= 128 && K >= 8192) || (groups <= 64 && K >= 4096)) {
        constexpr int kStageBytes = 512;  // the 16-column kernels' K stage at up to 64 rows
        const int64_t stages = (K + kStageBytes - 1) / kStageBytes;
        d.splits = 4;
        d.stages_per_split = static_cast<int>((stages + d.splits - 1) / d.splits);
        d.config = (d.stages_per_split >= 6 || K < 8192) ? kDecode16x64R : kDecode16x64;
    } else if (K >= 8192 && blocks < 256) {
        constexpr int64_t kSlots = 512;   // resident 64-column workgroups
        constexpr int kStageBytes = 256;  // the 64-column kernel's K stage
        const int64_t stages = (K + kStageBytes - 1) / kStageBytes;
        d.splits = static_cast<int>(std::min<int64_t>(kMaxSplitsK, std::max<int64_t>(2, kSlots / blocks)));
        d.stages_per_split = static_cast<int>((stages + d.splits - 1) / d.splits);
    } else {
        return d;
    }
    d.workspace_bytes = static_cast<int64_t>(d.splits) * M * N * 4;
    return d;
}

hipError_t launch_scaled_mm(const GemmProblem& p, hipStream_t st) {
    if (p.M == 0 || p.N == 0) return hipSuccess;
    GemmArgs a;
    a.out = p.out;
    a.ldo = p.ldo;
    a.a = p.a;
    a.lda = p.lda;
    a.b = p.b;
    a.ldb = p.ldb;
    a.M = static_cast<int>(p.M);
    a.N = static_cast<int>(p.N);
    a.K = static_cast<int>(p.K);
    a.sa = p.sa;
    a.sa_per_row = p.sa_per_row ? 1 : 0;
    a.sb = p.sb;
    a.sb_per_col = p.sb_per_col ? 1 : 0;
    a.tiles_m = a.tiles_n = 0;
    const int esz = (p.ot == D_BF16 || p.ot == D_FP16) ? 2 : 4;
    a.vec_out = (reinterpret_cast<uintptr_t>(p.out) % (4 * esz) == 0) && (p.ldo % 4 == 0);
    a.vec_row = (reinterpret_cast<uintptr_t>(p.out) % 16 == 0) && ((p.ldo * esz) % 16 == 0);
    a.part = nullptr;
    a.splits = 1;
    a.stages_per_split = 0;
    a.split_config = 0;
    a.azp = p.azp;
    a.azp_per_row = p.azp_per_row ? 1 : 0;
    a.colsum = p.colsum;
    if (p.workspace) {
        const SplitPlan d = plan_splitk(p.M, p.N, p.K);
        if (d.splits > 1 && p.workspace_bytes >= d.workspace_bytes) {
            a.part = p.workspace;
            a.splits = d.splits;
            a.stages_per_split = d.stages_per_split;
            a.split_config = d.config;
        }
    }
    if (p.qt == Q_FP8) return dispatch_ot<Q_FP8>(p.ot, a, st);
    return dispatch_ot<Q_INT8>(p.ot, a, st);
}

namespace {

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate (code under HIP graph capture,
// serving loops, harnesses that forbid allocation): the split-K partial sums
// of w8a8_scaled_mm_noalloc live in this file-scope device array instead of a
// caller workspace. Each GPU the library runs on holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, not the
// device address: the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that pointer is
// handed to kernels. Every call on one GPU shares that GPU's array; the split
// kernels overwrite every partial sum they later read, so nothing has to be
// cleared between calls, but calls that overlap on one GPU (concurrent
// streams, threads) race on it.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = int64_t(16) << 20;
// The largest split plan (M = 64, N = 16320, 4 splits of 4-byte sums) fits.
static_assert(int64_t(4) * 64 * 16320 * 4 <= kScratchBytes, "scratch holds every split plan");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device (looked up once).
hipError_t scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace

int64_t scaled_mm_noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t launch_scaled_mm_noalloc(const GemmProblem& p, hipStream_t st, int64_t* needed) {
    *needed = 0;
    if (p.M == 0 || p.N == 0) return hipSuccess;
    GemmProblem q = p;
    q.workspace = nullptr;
    q.workspace_bytes = 0;
    const SplitPlan d = plan_splitk(p.M, p.N, p.K);
    if (d.splits > 1) {
        if (d.workspace_bytes > kScratchBytes) {
            *needed = d.workspace_bytes;
            return hipErrorInvalidValue;
        }
        if (st) {  // the scratch used is the current device's: the stream must be on it
            int cur = -1;
            hipDevice_t sd = -1;
            hipError_t e = hipGetDevice(&cur);
            if (e == hipSuccess) e = hipStreamGetDevice(st, &sd);
            if (e != hipSuccess) return e;
            if (sd != cur) return hipErrorInvalidDevice;
        }
        hipError_t e = scratch_on_current_device(&q.workspace);
        if (e != hipSuccess) return e;
        q.workspace_bytes = kScratchBytes;
    }
    return launch_scaled_mm(q, st);
}

// Measured on MI355X (Llama-3-8B decode shapes): the fused kernel saves the
// quantizer launch on weights up to 16384 rows; on wider ones (gate_up,
// 28672) the per-workgroup quantisation over N / 16 workgroups costs more
// than the launch, and the 64-column decode kernel is faster.
// (K == 0 takes the two-call path: the fused kernel reads x[0 .. 7] whatever
// the row's length.)
bool quant_scaled_mm_fused(int64_t M, int64_t N, int64_t K) {
    return M == 1 && K > 0 && K <= kDynqMaxK && (N + 63) / 64 < 256;
}

hipError_t launch_quant_scaled_mm(const GemmProblem& p, int xt, const void* x, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* a_scales, hipStream_t st) {
    if (p.M == 0) return hipSuccess;
    if (!quant_scaled_mm_fused(p.M, p.N, p.K) || p.N == 0) {
        hipError_t e = launch_quant_per_token(xt, x, p.M, p.K, ldx, q, p.qt, ldq, a_scales, st);
        if (e != hipSuccess) return e;
        GemmProblem g = p;
        g.a = q;
        g.lda = ldq;
        g.sa = a_scales;
        g.sa_per_row = p.M != 1;
        return launch_scaled_mm(g, st);
    }
    GemmArgs a;
    a.out = p.out;
    a.ldo = p.ldo;
    a.a = q;
    a.lda = ldq;
    a.b = p.b;
    a.ldb = p.ldb;
    a.M = 1;
    a.N = static_cast<int>(p.N);
    a.K = static_cast<int>(p.K);
    a.sa = a_scales;
    a.sa_per_row = 0;
    a.sb = p.sb;
    a.sb_per_col = p.sb_per_col ? 1 : 0;
    a.tiles_m = a.tiles_n = 0;
    a.vec_out = 0;
    a.vec_row = 0;
    a.azp = nullptr;
    a.azp_per_row = 0;
    a.colsum = nullptr;
    a.part = nullptr;
    a.splits = 1;
    a.stages_per_split = 0;
    a.split_config = 0;
    const dim3 grid((p.N + 15) / 16), block(256);
#define W8A8_DYNQ(XT_, QT_, OT_) \
    hipLaunchKernelGGL((gemm_dynq_kernel<XT_, QT_, OT_>), grid, block, 0, st, a, x, q, a_scales)
#define W8A8_DYNQ_OT(XT_, QT_)                             \
    switch (p.ot) {                                         \
        case D_BF16: W8A8_DYNQ(XT_, QT_, D_BF16); break;    \
        case D_FP16: W8A8_DYNQ(XT_, QT_, D_FP16); break;    \
        default: W8A8_DYNQ(XT_, QT_, D_F32); break;         \
    }
#define W8A8_DYNQ_QT(XT_)                                                    \
    if (p.qt == Q_FP8) { W8A8_DYNQ_OT(XT_, Q_FP8) } else { W8A8_DYNQ_OT(XT_, Q_INT8) }
    switch (xt) {
        case D_BF16: W8A8_DYNQ_QT(D_BF16) break;
        case D_FP16: W8A8_DYNQ_QT(D_FP16) break;
        default: W8A8_DYNQ_QT(D_F32) break;
    }
#undef W8A8_DYNQ_QT
#undef W8A8_DYNQ_OT
#undef W8A8_DYNQ
    return hipGetLastError();
}

const char* scaled_mm_kernel_name(int64_t M, int64_t N, int64_t K, bool workspace) {
    if (workspace) {
        const SplitPlan d = plan_splitk(M, N, K);
        if (d.splits > 1) {
            switch (d.config) {
                case kDecode16x64: return "gemm_decode_kernel<16x64>+splitk_reduce_kernel";
                case kDecode16x64R: return "gemm_decode_kernel<16x64,3x512>+splitk_reduce_kernel";
                default: return "gemm_decode_kernel<64x64>+splitk_reduce_kernel";
            }
        }
    }
    switch (select_config(M, N, K)) {
        case kDecode64x16: return "gemm_decode_kernel<64x16>";
        case kDecode64x16R: return "gemm_decode_kernel<64x16,4x256>";
        case kDecode64x64: return "gemm_decode_kernel<64x64>";
        case kDecode16x16: return "gemm_decode_kernel<16x16>";
        case kDecode16x16R: return "gemm_decode_kernel<16x16,4x512>";
        case kDecode16x64: return "gemm_decode_kernel<16x64>";
        case kDecode16x64R: return "gemm_decode_kernel<16x64,3x512>";
        case kDecode16x16L: return "gemm_decode_kernel<16x16,4x1K>";
        case kDecode16x64L: return "gemm_decode_kernel<16x64,1K>";
        case kTile256x256: return "gemm_tile_kernel<256x256>";
        case kTile256x128: return "gemm_tile_kernel<256x128>";
        case kTile128x128: return "gemm_tile_kernel<128x128>";
        case kTile128x128R: return "gemm_tile_kernel<128x128,3x128>";
        case kTile128x64: return "gemm_tile_kernel<128x64,4x128>";
        case kTile64x64: return "gemm_tile_kernel<64x64,4x128>";
    }
    return "";  // not reached
}

}  // namespace w8a8

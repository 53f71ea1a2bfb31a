// gemm.hip -- the w8a8 scaled matrix multiply on gfx950 MFMA.
//
//   D[m, n] = a_scale[m|0] * b_scale[n|0] * sum_k A[m, k] * B[n, k]
//
// ("[Kernel] Add w8a8 CUTLASS kernels": the PR description's bullet list
// fixes the operation and its scale granularities; the misaligned-address
// report fixes B as K x N column-major, i.e. rows of an [N, K] weight.)
//
// The contraction runs on the CDNA4 matrix cores:
//   fp8 e4m3:  v_mfma_f32_16x16x128_f8f6f4 (format 0 = e4m3), fp32 accumulate
//   int8:      v_mfma_i32_16x16x64_i8, exact int32 accumulate
// Both consume, per lane, 32 bytes of an A row and 32 bytes of a B row
// (lane l: row l%16, bytes 32*(l/16) .. +32 of a 128-byte K slice), and
// leave lane l holding D rows 4*(l/16)+i (i < 4) of column l%16. The int8
// path issues two 64-deep MFMAs on the two 16-byte halves of the same
// fragment: both operands see the same K permutation, so the integer sum is
// unchanged.
//
// Two kernels:
//  - gemm_tile_kernel: a BM x BN block tile per workgroup (4 waves, 2 x 2),
//    K walked in 128-byte slices staged through LDS with double buffering
//    (global -> registers for slice k+1 while MFMAs consume slice k), rows
//    padded by 16 bytes so the 16-lane fragment reads spread over the banks.
//    Tiles are numbered so that consecutive tiles land on one XCD (blocks
//    are dealt round-robin over the 8 XCDs) and walk groups of 8 row-tiles,
//    keeping shared A and B slices in that XCD's L2.
//  - gemm_decode_kernel: M <= 64 rows. The weight stream dominates (HBM
//    bound), so each workgroup owns 16 output columns and its waves split K,
//    every lane keeping several 16-byte weight loads in flight; fragments go
//    straight from global memory to the MFMA, and the waves' partial sums are
//    added through LDS before the epilogue.
// The epilogue is fused: scales applied in fp32 and the result rounded to
// nearest even into bf16/fp16 in registers, then stored once.
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
template <int OT, typename T>
__device__ __forceinline__ void store_out(const GemmArgs& p, int m, int n, T acc) {
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

constexpr int kBK = 128;            // K bytes per slice (one MFMA depth for fp8)
constexpr int kLdsRow = kBK + 16;   // padded LDS row

template <int QT, int OT, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmArgs p) {
    typedef typename AccOf<QT>::type Acc;
    constexpr int WM = BM / 2, WN = BN / 2;  // 2 x 2 waves
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int AV = BM * kBK / 16 / 256;  // 16-byte vectors per lane per slice
    constexpr int BV = BN * kBK / 16 / 256;
    constexpr int kStage = (BM + BN) * kLdsRow;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

    int tm, tn;
    if (!tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn)) return;
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    u32x4 ra[AV], rb[BV];
    auto gload = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int v = tid + 256 * j, r = v >> 3, k = k0 + (v & 7) * 16;
            const int gm = m0 + r;
            ra[j] = (gm < p.M && k < p.K) ? load16(p.a + static_cast<int64_t>(gm) * p.lda + k)
                                          : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < BV; ++j) {
            const int v = tid + 256 * j, r = v >> 3, k = k0 + (v & 7) * 16;
            const int gn = n0 + r;
            rb[j] = (gn < p.N && k < p.K) ? load16(p.b + static_cast<int64_t>(gn) * p.ldb + k)
                                          : u32x4{0, 0, 0, 0};
        }
    };
    auto swrite = [&](int buf) {
        uint8_t* s = smem + buf * kStage;
#pragma unroll
        for (int j = 0; j < AV; ++j) {
            const int v = tid + 256 * j;
            *reinterpret_cast<u32x4*>(s + (v >> 3) * kLdsRow + (v & 7) * 16) = ra[j];
        }
#pragma unroll
        for (int j = 0; j < BV; ++j) {
            const int v = tid + 256 * j;
            *reinterpret_cast<u32x4*>(s + (BM + (v >> 3)) * kLdsRow + (v & 7) * 16) = rb[j];
        }
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    const int KT = (p.K + kBK - 1) / kBK;
    if (KT > 0) {
        gload(0);
        swrite(0);
    }
    __syncthreads();
    const int frag_row = lane & 15, frag_k = (lane >> 4) * 32;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const uint8_t* s = smem + cur * kStage;
        i32x8 af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint8_t* q = s + (wm * WM + i * 16 + frag_row) * kLdsRow + frag_k;
            af[i] = join(load16(q), load16(q + 16));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint8_t* q = s + (BM + wn * WN + j * 16 + frag_row) * kLdsRow + frag_k;
            bf[j] = join(load16(q), load16(q + 16));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) mma<QT>(acc[i][j], af[i], bf[j]);
        if (kt + 1 < KT) swrite(cur ^ 1);
        __syncthreads();
    }

    // Fused epilogue.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * WN + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + r;
                if (m < p.M && n < p.N) store_out<OT>(p, m, n, acc[i][j][r]);
            }
        }
}

// M <= 64 rows in up to 4 row-tiles of 16 (p.tiles_m of them, a runtime
// value so that one kernel serves every decode batch size); one workgroup
// per 16 columns; WAVES waves split the 128-byte K slices round-robin
// (neighbouring waves read neighbouring slices of the same weight rows);
// U slices per wave per step in flight.
template <int QT, int OT, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void gemm_decode_kernel(GemmArgs p) {
    typedef typename AccOf<QT>::type Acc;
    constexpr int TM = 4;
    const int mt = p.tiles_m;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int nrow = n0 + (lane & 15);
    const uint8_t* bp = p.b + static_cast<int64_t>(nrow < p.N ? nrow : p.N - 1) * p.ldb;
    const int koff = (lane >> 4) * 32;
    const int KS = (p.K + kBK - 1) / kBK;

    Acc acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = Acc{0, 0, 0, 0};

    const u32x4 z = {0, 0, 0, 0};
    for (int ks = wave; ks < KS; ks += WAVES * U) {
        i32x8 bf[U];
        i32x8 af[U][TM];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (ks + u * WAVES) * kBK + koff;
            const bool lo = k < p.K, hi = k + 16 < p.K;
            bf[u] = join(lo ? load16(bp + k) : z, hi ? load16(bp + k + 16) : z);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if (i >= mt) break;
                const int m = i * 16 + (lane & 15);
                const uint8_t* ap = p.a + static_cast<int64_t>(m) * p.lda + k;
                const bool mv = m < p.M;
                af[u][i] = join((mv && lo) ? load16(ap) : z, (mv && hi) ? load16(ap + 16) : z);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if (i >= mt) break;
                mma<QT>(acc[i], af[u][i], bf[u]);
            }
    }

    // Add the waves' partial sums (fixed order), then the fused epilogue.
    __shared__ Acc red[WAVES][TM][64];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        if (i < mt) red[wave][i][lane] = acc[i];
    __syncthreads();
    for (int i = wave; i < mt; i += WAVES) {
        Acc s = red[0][i][lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) s += red[w][i][lane];
        const int n = n0 + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = i * 16 + 4 * (lane >> 4) + r;
            if (m < p.M && n < p.N) store_out<OT>(p, m, n, s[r]);
        }
    }
}

template <int QT, int OT, int BM, int BN>
hipError_t run_tile(GemmArgs a, hipStream_t st) {
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    const int total = a.tiles_m * a.tiles_n;
    const int grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((gemm_tile_kernel<QT, OT, BM, BN>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int QT, int OT>
hipError_t run_decode(GemmArgs a, hipStream_t st) {
    constexpr int kWaves = 4, kU = 4;
    a.tiles_m = (a.M + 15) / 16;
    const int grid = (a.N + 15) / 16;
    hipLaunchKernelGGL((gemm_decode_kernel<QT, OT, kWaves, kU>), dim3(grid), dim3(kWaves * 64), 0, st, a);
    return hipGetLastError();
}

template <int QT, int OT>
hipError_t dispatch(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 64) return run_decode<QT, OT>(a, st);
    // Enough 128 x 128 tiles to cover the 256 CUs, else halve the row tile.
    const int64_t big = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (big >= 256) return run_tile<QT, OT, 128, 128>(a, st);
    return run_tile<QT, OT, 64, 128>(a, st);
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
    if (p.qt == Q_FP8) return dispatch_ot<Q_FP8>(p.ot, a, st);
    return dispatch_ot<Q_INT8>(p.ot, a, st);
}

}  // namespace w8a8

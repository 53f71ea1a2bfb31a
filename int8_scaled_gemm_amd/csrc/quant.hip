// quant.hip -- the quantizers that feed the scaled matrix multiply, and the
// scaled fp8 KV-cache quant/dequant, for gfx950.
//
// Definitions: "Enable scaled FP8 (e4m3fn) KV cache on ROCm", "Scaling
// semantics" (scale = absmax / 448, q = fp8(x / scale), x' = dequant(q) *
// scale); "[Kernel] Add w8a8 CUTLASS kernels", per_tensor_quantize snippet
// (divide, clamp to the e4m3 range, cast) and the PR's list of scale
// granularities (per token, per tensor); "[Kernel] Support Fp8 Checkpoints
// (Dynamic + Static)" (static calibrated vs dynamic activation scales).
//
// All of these are HBM-bound streams: 2 bytes in and 1 byte out per element
// (bf16 -> code), plus a 2-byte read pass for a dynamic per-tensor scale.
// Loads and stores are 16-byte vectors per lane; a row's absmax is reduced
// across the wavefront with lane shuffles, and across waves through LDS.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace w8a8 {

namespace {

constexpr int kBlock = 256;

// ------------------------------------------------------------------------
// Per-token (per-row) dynamic quantisation, row held in registers.
// TPR threads share one row (64: one wavefront, 256: the whole block); each
// thread holds VPT vectors of 8 elements. One HBM read, one HBM write.
// ------------------------------------------------------------------------
template <int XT, int QT, int TPR, int VPT, int BS = kBlock>
__global__ __launch_bounds__(BS) void quant_rows_kernel(const void* __restrict__ x, int64_t ldx,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            float* __restrict__ scales, int64_t M,
                                                            int64_t K) {
    constexpr int RPB = BS / TPR;
    const int t = threadIdx.x % TPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
    const bool active = row < M;

    // Every load is issued before the first is used (a conditional load
    // that is widened at once would be waited for before the next is
    // issued); lanes past the row load the tensor's first element group
    // instead and count zeros. K == 0 (a call that only writes scales of 1)
    // reads nothing.
    u32x4 raw[VPT][2] = {};
    if (K > 0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int64_t k = static_cast<int64_t>(t + i * TPR) * 8;
            load8_raw<XT>(x, active && k < K ? row * ldx + k : 0, raw[i]);
        }
    }
    float v[VPT][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t k = static_cast<int64_t>(t + i * TPR) * 8;
        widen8<XT>(raw[i], v[i]);
        if (!(active && k < K)) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
    }
    amax = wave_max(amax);
    if constexpr (TPR > 64) {
        __shared__ float part[BS / 64];
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < BS / 64; ++w) amax = fmaxf(amax, part[w]);
    }
    if (!active) return;

    const float s = scale_from_absmax<QT>(amax);
    const double r = 1.0 / static_cast<double>(s);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int64_t k = static_cast<int64_t>(t + i * TPR) * 8;
        if (k < K) *reinterpret_cast<u32x2*>(q + row * ldq + k) = quant8<QT>(v[i], r);
    }
    if (t == 0) scales[row] = s;
}

// Rows too long for registers: one block per row, absmax pass then a
// quantise pass that re-reads the row (from L2).
template <int XT, int QT>
__global__ __launch_bounds__(kBlock) void quant_rows_2pass_kernel(const void* __restrict__ x,
                                                                  int64_t ldx,
                                                                  uint8_t* __restrict__ q,
                                                                  int64_t ldq,
                                                                  float* __restrict__ scales,
                                                                  int64_t M, int64_t K) {
    const int64_t row = blockIdx.x;
    float amax = 0.0f;
    for (int64_t k = static_cast<int64_t>(threadIdx.x) * 8; k < K; k += kBlock * 8) {
        float v[8];
        load8<XT>(x, row * ldx + k, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
    amax = wave_max(amax);
    __shared__ float part[kBlock / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) amax = fmaxf(amax, part[w]);

    const float s = scale_from_absmax<QT>(amax);
    const double r = 1.0 / static_cast<double>(s);
    for (int64_t k = static_cast<int64_t>(threadIdx.x) * 8; k < K; k += kBlock * 8) {
        float v[8];
        load8<XT>(x, row * ldx + k, v);
        *reinterpret_cast<u32x2*>(q + row * ldq + k) = quant8<QT>(v, r);
    }
    if (threadIdx.x == 0) scales[row] = s;
}

// ------------------------------------------------------------------------
// Per-tensor passes over an [M, K] tensor with a row stride. Work is cut in
// units of one row x 2048 elements (256 lanes x 8); each block takes kUnroll
// units per step so that every lane keeps kUnroll 16-byte loads in flight
// (2 rather than 4: twice the workgroups, measured 8192 x 4096 27.7 -> 24.0
// us, 512 x 14336 7.5 -> 6.7 us on MI355X).
// ------------------------------------------------------------------------
constexpr int kUnroll = 2;
// The quantising pass of a dynamic per-tensor scale keeps 4 (fewer
// workgroups, each reducing the partial maxima once: KV quant call 40.6 us
// against 41.2 us with 2).
constexpr int kUnrollDynamic = 4;
constexpr int kUnitElems = kBlock * 8;

struct Units {
    uint32_t per_row;  // units per row
    uint32_t total;
};

__device__ __forceinline__ bool unit_coords(const Units& u, uint32_t id, int64_t K, int64_t& row,
                                            int64_t& k) {
    if (id >= u.total) return false;
    const uint32_t r = id / u.per_row;
    row = r;
    k = static_cast<int64_t>(id - r * u.per_row) * kUnitElems + threadIdx.x * 8;
    return k < K;
}

// Writes v into *p (a float), as a kernel so that a captured graph holds no
// memset node.
__global__ void fill_f32_kernel(float* p, float v) { *p = v; }

// Dynamic per-tensor scale without atomics or a workspace: every absmax
// workgroup stores its partial maximum (a float) in the tail of the code
// buffer q, the last `tail` elements of the tensor in row order. The quantise
// pass reduces the partials in every workgroup (a few KB, L2-resident) and
// leaves the tail alone; a last one-workgroup kernel reduces them once more,
// writes the scale and quantises the tail over them. The maximum does not
// depend on the order of the partials, so the scale is deterministic.
constexpr int kAbsUnroll = 8;  // loads in flight per lane in the read-only absmax pass

struct Tail {
    int64_t start;  // first tail element (row-major index over M x K)
    int parts;      // partial maxima stored at the start of the tail, 4 bytes each
};

// Address of byte e of the row-major M x K code tensor with row stride ldq.
__device__ __forceinline__ uint8_t* code_at(uint8_t* q, int64_t ldq, int64_t K, int64_t e) {
    return q + (e / K) * ldq + (e % K);
}

// The 8 elements at x + off[j] for each of U units, every load issued before
// the first is widened (a conditional load widened at once is waited for
// before the next one is issued). A unit that is not ok loads the tensor's
// first 8 elements instead, and its values are not to be used.
template <int XT, bool NT, int U>
__device__ __forceinline__ void load_units(const void* x, const int64_t (&off)[U], const bool (&ok)[U],
                                           float (&v)[U][8]) {
    u32x4 raw[U][2];
#pragma unroll
    for (int j = 0; j < U; ++j) load8_raw<XT, NT>(x, ok[j] ? off[j] : 0, raw[j]);
#pragma unroll
    for (int j = 0; j < U; ++j) widen8<XT>(raw[j], v[j]);
}

template <int XT>
__global__ __launch_bounds__(kBlock) void absmax_kernel(const void* __restrict__ x, int64_t ldx,
                                                        Units u, int64_t K, uint8_t* q,
                                                        int64_t ldq, Tail tail) {
    float amax = 0.0f;
    for (uint32_t base = blockIdx.x * kAbsUnroll; base < u.total; base += gridDim.x * kAbsUnroll) {
        float v[kAbsUnroll][8];
        bool ok[kAbsUnroll];
        int64_t off[kAbsUnroll];
#pragma unroll
        for (int j = 0; j < kAbsUnroll; ++j) {
            int64_t row, k;
            ok[j] = unit_coords(u, base + j, K, row, k);
            off[j] = row * ldx + k;
        }
        load_units<XT, false>(x, off, ok, v);  // cached: read again next
#pragma unroll
        for (int j = 0; j < kAbsUnroll; ++j)
            if (ok[j])
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
    amax = wave_max(amax);
    __shared__ float part[kBlock / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) amax = fmaxf(amax, part[w]);
        *reinterpret_cast<float*>(code_at(q, ldq, K, tail.start + 4 * blockIdx.x)) = amax;
    }
}

// Maximum of the stored partials (at most 1024, at least 1), in every
// thread of the workgroup; a thread's loads are all issued before the first
// is used (past the count they re-read partial 0).
__device__ float reduce_partials(uint8_t* q, int64_t ldq, int64_t K, const Tail& tail) {
    constexpr int kPer = 1024 / kBlock;
    float pv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = threadIdx.x + j * kBlock;
        pv[j] = *reinterpret_cast<const float*>(code_at(q, ldq, K, tail.start + 4 * (i < tail.parts ? i : 0)));
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (static_cast<int>(threadIdx.x) + j * kBlock < tail.parts) amax = fmaxf(amax, pv[j]);
    amax = wave_max(amax);
    __shared__ float part[kBlock / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) amax = fmaxf(amax, part[w]);
    return amax;
}

// Quantise with one scale for the whole tensor. DYNAMIC: the scale comes
// from the partial maxima in the tail, and the tail is left to
// finish_tail_kernel; otherwise *scale is the scale (NULL: 1.0).
template <int XT, int QT, bool DYNAMIC, int U = DYNAMIC ? kUnrollDynamic : kUnroll>
__global__ __launch_bounds__(kBlock) void quant_tensor_kernel(const void* __restrict__ x,
                                                              int64_t ldx, uint8_t* q, int64_t ldq,
                                                              const float* __restrict__ scale,
                                                              Units u, int64_t K, Tail tail) {
    float s;
    if constexpr (DYNAMIC) s = scale_from_absmax<QT>(reduce_partials(q, ldq, K, tail));
    else s = scale ? *scale : 1.0f;
    const double r = 1.0 / static_cast<double>(s);
    for (uint32_t base = blockIdx.x * U; base < u.total; base += gridDim.x * U) {
        float v[U][8];
        bool ok[U];
        int64_t row[U], k[U], off[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            ok[j] = unit_coords(u, base + j, K, row[j], k[j]);
            if (DYNAMIC && ok[j] && row[j] * K + k[j] >= tail.start) ok[j] = false;
            off[j] = row[j] * ldx + k[j];
        }
        load_units<XT, true>(x, off, ok, v);
#pragma unroll
        for (int j = 0; j < U; ++j)
            if (ok[j]) *reinterpret_cast<u32x2*>(q + row[j] * ldq + k[j]) = quant8<QT>(v[j], r);
    }
}

// One workgroup: the scale from the partials, written to *scale, then the
// tail's codes, over the partials once every thread has read them.
template <int XT, int QT>
__global__ __launch_bounds__(kBlock) void finish_tail_kernel(const void* __restrict__ x,
                                                             int64_t ldx, uint8_t* q, int64_t ldq,
                                                             float* scale, int64_t M, int64_t K,
                                                             Tail tail) {
    // The thread's first two 8-element groups of the tail are requested
    // together with the partial maxima (a tail past a large tensor has at
    // most 4096 elements: two groups per thread); groups past the tensor
    // load its first group and are not used.
    const int64_t total = M * K;
    const int64_t e0 = tail.start + 8 * static_cast<int64_t>(threadIdx.x), e1 = e0 + 8 * kBlock;
    auto xoff = [&](int64_t e) { return e < total ? (e / K) * ldx + e % K : 0; };  // never across a row (K % 16 == 0)
    u32x4 ra[2][2];
    load8_raw<XT>(x, xoff(e0), ra[0]);
    load8_raw<XT>(x, xoff(e1), ra[1]);
    const float s = scale_from_absmax<QT>(reduce_partials(q, ldq, K, tail));
    __syncthreads();  // every partial has been read
    if (threadIdx.x == 0) *scale = s;
    const double r = 1.0 / static_cast<double>(s);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t e = j ? e1 : e0;
        float v[8];
        widen8<XT>(ra[j], v);
        if (e < total) *reinterpret_cast<u32x2*>(q + (e / K) * ldq + e % K) = quant8<QT>(v, r);
    }
    for (int64_t e = e1 + 8 * kBlock; e < total; e += 8 * kBlock) {  // small tensors: the whole tensor is the tail
        const int64_t row = e / K, k = e % K;
        float v[8];
        load8<XT>(x, row * ldx + k, v);
        *reinterpret_cast<u32x2*>(q + row * ldq + k) = quant8<QT>(v, r);
    }
}

// ------------------------------------------------------------------------
// KV dequant: 8 codes per lane (one 8-byte load), product in float32,
// rounded once into the output type. A 2-byte output is one 16-byte
// non-temporal store per lane, so that each store instruction of a wave
// writes 1 KB of whole cache lines (16 codes per lane wrote two 16-byte
// pieces 32 bytes apart, each instruction leaving every other piece to the
// next); float32 output is two 16-byte stores per lane, cached.
// ------------------------------------------------------------------------
constexpr int kDequantUnroll = 8;

template <int XT>
__global__ __launch_bounds__(kBlock) void kv_dequant_kernel(const uint8_t* __restrict__ q,
                                                            int64_t n,
                                                            const float* __restrict__ scale,
                                                            void* __restrict__ x) {
    constexpr int U = kDequantUnroll;  // 8-byte loads in flight per lane
    const float s = scale ? *scale : 1.0f;
    const int64_t nvec = n / 8;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kBlock * U + threadIdx.x;
         base < nvec; base += static_cast<int64_t>(gridDim.x) * kBlock * U) {
        // Every load is issued before the first is used, and every store
        // after the last conversion: a load under its bounds check was
        // waited for before the next was issued, and a load after a store
        // made the compiler wait for the store as well. Pieces past the
        // tensor load its first 8 codes and are not stored.
        u32x2 c[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t i = base + j * kBlock;
            c[j] = reinterpret_cast<const u32x2*>(q)[i < nvec ? i : 0];
        }
        typedef typename std::conditional<XT == D_F32, f32x4, u32x4>::type Out;
        Out o[U][XT == D_F32 ? 2 : 1];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float f[8];
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                f[4 * w + 0] = __builtin_amdgcn_cvt_f32_fp8(c[j][w], 0) * s;
                f[4 * w + 1] = __builtin_amdgcn_cvt_f32_fp8(c[j][w], 1) * s;
                f[4 * w + 2] = __builtin_amdgcn_cvt_f32_fp8(c[j][w], 2) * s;
                f[4 * w + 3] = __builtin_amdgcn_cvt_f32_fp8(c[j][w], 3) * s;
            }
            if constexpr (XT == D_F32) {
                o[j][0] = f32x4{f[0], f[1], f[2], f[3]};
                o[j][1] = f32x4{f[4], f[5], f[6], f[7]};
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t lo, hi;
                    if constexpr (XT == D_BF16) {
                        lo = to_bf16_bits(f[2 * w]);
                        hi = to_bf16_bits(f[2 * w + 1]);
                    } else {
                        lo = to_fp16_bits(f[2 * w]);
                        hi = to_fp16_bits(f[2 * w + 1]);
                    }
                    o[j][0][w] = lo | (hi << 16);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int64_t i = base + j * kBlock;
            if (i >= nvec) continue;
            if constexpr (XT == D_F32) {
                f32x4* out = reinterpret_cast<f32x4*>(static_cast<float*>(x) + i * 8);
                out[0] = o[j][0];
                out[1] = o[j][1];
            } else {
                __builtin_nontemporal_store(o[j][0], reinterpret_cast<u32x4*>(static_cast<uint16_t*>(x) + i * 8));
            }
        }
    }
}

int grid_for(uint64_t work_items, uint64_t per_block) {
    uint64_t g = (work_items + per_block - 1) / per_block;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return static_cast<int>(g);
}

Units make_units(int64_t M, int64_t K) {
    Units u;
    u.per_row = static_cast<uint32_t>((K + kUnitElems - 1) / kUnitElems);
    u.total = static_cast<uint32_t>(M) * u.per_row;
    return u;
}

template <int XT, int QT>
hipError_t per_token_typed(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                           int64_t ldq, float* scales, hipStream_t st) {
    // The row in registers, a whole workgroup per row (256 lanes up to 8192
    // elements, 1024 up to 32768), else two passes. Each lane's share of its
    // row, and with it the serial load -> divide -> store chain, is short:
    // measured on MI355X against one wave per row, 8192 x 4096 28.4 -> 24.0
    // us, 4096 x 8192 34.8 -> 28.0 us, 4096 x 28672 117 -> 81 us, and 4.5-5.4
    // -> 3.1-4.1 us for decode batches.
    if (K <= 32768) {
        const int g = static_cast<int>(M);
        if (K <= 2048)
            hipLaunchKernelGGL((quant_rows_kernel<XT, QT, 256, 1>), dim3(g), dim3(kBlock), 0, st, x, ldx, q, ldq, scales, M, K);
        else if (K <= 4096)
            hipLaunchKernelGGL((quant_rows_kernel<XT, QT, 256, 2>), dim3(g), dim3(kBlock), 0, st, x, ldx, q, ldq, scales, M, K);
        else if (K <= 8192)
            hipLaunchKernelGGL((quant_rows_kernel<XT, QT, 256, 4>), dim3(g), dim3(kBlock), 0, st, x, ldx, q, ldq, scales, M, K);
        else if (K <= 16384)  // 1024 lanes per row: two 8-element groups each
            hipLaunchKernelGGL((quant_rows_kernel<XT, QT, 1024, 2, 1024>), dim3(g), dim3(1024), 0, st, x, ldx, q, ldq, scales, M, K);
        else
            hipLaunchKernelGGL((quant_rows_kernel<XT, QT, 1024, 4, 1024>), dim3(g), dim3(1024), 0, st, x, ldx, q, ldq, scales, M, K);
    } else {
        hipLaunchKernelGGL((quant_rows_2pass_kernel<XT, QT>), dim3(static_cast<int>(M)), dim3(kBlock), 0, st, x, ldx, q, ldq, scales, M, K);
    }
    return hipGetLastError();
}

template <int XT, int QT>
hipError_t per_tensor_typed(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, float* scale, bool dynamic, hipStream_t st) {
    const Units u = make_units(M, K);
    const int g = grid_for(u.total, kUnroll);
    if (dynamic) {
        const int64_t total = M * K;
        if (total == 0) {  // an empty tensor has absmax 0: scale 1.0
            hipLaunchKernelGGL(fill_f32_kernel, dim3(1), dim3(1), 0, st, scale, scale_of_zero<QT>());
            return hipGetLastError();
        }
        Tail tail;
        tail.parts = std::min(grid_for(u.total, kAbsUnroll), 1024);
        // the tail holds the partials; small tensors are finished by the last kernel alone
        const int64_t tail_len = (4 * static_cast<int64_t>(tail.parts) + 15) / 16 * 16;
        tail.start = total <= 65536 ? 0 : total - tail_len;
        hipLaunchKernelGGL((absmax_kernel<XT>), dim3(tail.parts), dim3(kBlock), 0, st, x, ldx, u, K, q, ldq, tail);
        // at most 8 workgroups per CU: each reduces the partials once, then
        // strides over the units
        if (tail.start > 0)
            hipLaunchKernelGGL((quant_tensor_kernel<XT, QT, true>), dim3(std::min(grid_for(u.total, kUnrollDynamic), 2048)), dim3(kBlock), 0, st, x, ldx, q, ldq, static_cast<const float*>(scale), u, K, tail);
        hipLaunchKernelGGL((finish_tail_kernel<XT, QT>), dim3(1), dim3(kBlock), 0, st, x, ldx, q, ldq, scale, M, K, tail);
    } else {
        hipLaunchKernelGGL((quant_tensor_kernel<XT, QT, false>), dim3(g), dim3(kBlock), 0, st, x, ldx, q, ldq, static_cast<const float*>(scale), u, K, Tail{0, 0});
    }
    return hipGetLastError();
}

template <int QT>
hipError_t per_token_q(int xt, const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                       int64_t ldq, float* scales, hipStream_t st) {
    switch (xt) {
        case D_BF16: return per_token_typed<D_BF16, QT>(x, M, K, ldx, q, ldq, scales, st);
        case D_FP16: return per_token_typed<D_FP16, QT>(x, M, K, ldx, q, ldq, scales, st);
        default: return per_token_typed<D_F32, QT>(x, M, K, ldx, q, ldq, scales, st);
    }
}

template <int QT>
hipError_t per_tensor_q(int xt, const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                        int64_t ldq, float* scale, bool dynamic, hipStream_t st) {
    switch (xt) {
        case D_BF16: return per_tensor_typed<D_BF16, QT>(x, M, K, ldx, q, ldq, scale, dynamic, st);
        case D_FP16: return per_tensor_typed<D_FP16, QT>(x, M, K, ldx, q, ldq, scale, dynamic, st);
        default: return per_tensor_typed<D_F32, QT>(x, M, K, ldx, q, ldq, scale, dynamic, st);
    }
}

}  // namespace

hipError_t launch_quant_per_token(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int qt, int64_t ldq, float* scales, hipStream_t st) {
    if (M == 0) return hipSuccess;
    if (qt == Q_FP8) return per_token_q<Q_FP8>(xt, x, M, K, ldx, q, ldq, scales, st);
    return per_token_q<Q_INT8>(xt, x, M, K, ldx, q, ldq, scales, st);
}

hipError_t launch_quant_per_tensor(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* q, int qt, int64_t ldq, float* scale, bool dynamic,
                                   hipStream_t st) {
    if (qt == Q_FP8) return per_tensor_q<Q_FP8>(xt, x, M, K, ldx, q, ldq, scale, dynamic, st);
    return per_tensor_q<Q_INT8>(xt, x, M, K, ldx, q, ldq, scale, dynamic, st);
}

// ------------------------------------------------------------------------
// Asymmetric int8 activations [P1: the asymmetric int8 case and its small
// fused operations; the scheme itself is the textbook one]. One workgroup
// per row: a read pass for the row's range with 0 included, then a
// quantising pass over the row again (from L2).
//   s = (hi - lo) / 255 (1.0 for an all-zero row), z = rint(-128 - lo / s)
//   clamped to [-128, 127], q = clamp(rint(x / s) + z, -128, 127),
// every division correctly rounded in binary32 and every rint half-to-even.
// ------------------------------------------------------------------------
template <int XT>
__global__ __launch_bounds__(kBlock) void quant_rows_azp_kernel(const void* __restrict__ x, int64_t ldx,
                                                               uint8_t* __restrict__ q, int64_t ldq,
                                                               float* __restrict__ scales,
                                                               int32_t* __restrict__ azp, int64_t K) {
    __shared__ float part[2][kBlock / 64];
    const int64_t row = blockIdx.x;
    float hi = 0.0f, nlo = 0.0f;  // max(x, 0) and max(-x, 0)
    for (int64_t k = static_cast<int64_t>(threadIdx.x) * 8; k < K; k += kBlock * 8) {
        float v[8];
        load8<XT>(x, row * ldx + k, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            hi = fmaxf(hi, v[j]);
            nlo = fmaxf(nlo, -v[j]);
        }
    }
    hi = wave_max(hi);
    nlo = wave_max(nlo);
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = hi;
        part[1][threadIdx.x >> 6] = nlo;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) {
        hi = fmaxf(hi, part[0][w]);
        nlo = fmaxf(nlo, part[1][w]);
    }
    const float lo = -nlo;
    const float d = hi - lo;
    const float s = d == 0.0f ? 1.0f : d / 255.0f;
    const double r = 1.0 / static_cast<double>(s);
    const float zf = fminf(fmaxf(__builtin_rintf(-128.0f - div_rn(lo, r)), -128.0f), 127.0f);
    if (threadIdx.x == 0) {
        scales[row] = s;
        azp[row] = static_cast<int32_t>(zf);
    }
    for (int64_t k = static_cast<int64_t>(threadIdx.x) * 8; k < K; k += kBlock * 8) {
        float v[8];
        load8<XT>(x, row * ldx + k, v);
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float c = fminf(fmaxf(__builtin_rintf(div_rn(v[j], r)) + zf, -128.0f), 127.0f);
            w[j >> 2] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xFFu) << (8 * (j & 3));
        }
        *reinterpret_cast<u32x2*>(q + row * ldq + k) = u32x2{w[0], w[1]};
    }
}

// The asymmetric scheme's scale, its reciprocal and the zero point from the
// range: lo = -nlo <= 0 <= hi.
struct AzpParams {
    float s, zf;
    double r;
};

__device__ __forceinline__ AzpParams azp_params(float hi, float nlo) {
    AzpParams a;
    const float lo = -nlo;
    const float d = hi - lo;
    a.s = d == 0.0f ? 1.0f : d / 255.0f;
    a.r = 1.0 / static_cast<double>(a.s);
    a.zf = fminf(fmaxf(__builtin_rintf(-128.0f - div_rn(lo, a.r)), -128.0f), 127.0f);
    return a;
}

__device__ __forceinline__ u32x2 quant8_azp(const float v[8], double r, float zf) {
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float c = fminf(fmaxf(__builtin_rintf(div_rn(v[j], r)) + zf, -128.0f), 127.0f);
        w[j >> 2] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xFFu) << (8 * (j & 3));
    }
    return u32x2{w[0], w[1]};
}

// Asymmetric per tensor: the range pass, as absmax_kernel, with two partial
// maxima per workgroup, max(x, 0) and max(-x, 0), stored as 8 bytes in the
// tail of the code buffer.
template <int XT>
__global__ __launch_bounds__(kBlock) void range_kernel(const void* __restrict__ x, int64_t ldx,
                                                       Units u, int64_t K, uint8_t* q, int64_t ldq,
                                                       Tail tail) {
    float hi = 0.0f, nlo = 0.0f;
    for (uint32_t base = blockIdx.x * kAbsUnroll; base < u.total; base += gridDim.x * kAbsUnroll) {
        float v[kAbsUnroll][8];
        bool ok[kAbsUnroll];
        int64_t off[kAbsUnroll];
#pragma unroll
        for (int j = 0; j < kAbsUnroll; ++j) {
            int64_t row, k;
            ok[j] = unit_coords(u, base + j, K, row, k);
            off[j] = row * ldx + k;
        }
        load_units<XT, false>(x, off, ok, v);  // cached: read again next
#pragma unroll
        for (int j = 0; j < kAbsUnroll; ++j)
            if (ok[j])
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    hi = fmaxf(hi, v[j][e]);
                    nlo = fmaxf(nlo, -v[j][e]);
                }
    }
    hi = wave_max(hi);
    nlo = wave_max(nlo);
    __shared__ float part[2][kBlock / 64];
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = hi;
        part[1][threadIdx.x >> 6] = nlo;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) {
            hi = fmaxf(hi, part[0][w]);
            nlo = fmaxf(nlo, part[1][w]);
        }
        *reinterpret_cast<f32x2*>(code_at(q, ldq, K, tail.start + 8 * blockIdx.x)) = f32x2{hi, nlo};
    }
}

// The range from the stored partials, in every thread of the workgroup.
__device__ void reduce_range(uint8_t* q, int64_t ldq, int64_t K, const Tail& tail, float& hi,
                             float& nlo) {
    hi = nlo = 0.0f;
    for (int i = threadIdx.x; i < tail.parts; i += kBlock) {
        const f32x2 p = *reinterpret_cast<const f32x2*>(code_at(q, ldq, K, tail.start + 8 * i));
        hi = fmaxf(hi, p[0]);
        nlo = fmaxf(nlo, p[1]);
    }
    hi = wave_max(hi);
    nlo = wave_max(nlo);
    __shared__ float part[2][kBlock / 64];
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = hi;
        part[1][threadIdx.x >> 6] = nlo;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) {
        hi = fmaxf(hi, part[0][w]);
        nlo = fmaxf(nlo, part[1][w]);
    }
}

// Quantise with one scale and zero point. DYNAMIC: from the partials in the
// tail, which is left to finish_tail_azp_kernel; otherwise *scale and *azp
// (NULL: 1.0 and 0).
template <int XT, bool DYNAMIC>
__global__ __launch_bounds__(kBlock) void quant_tensor_azp_kernel(const void* __restrict__ x,
                                                                  int64_t ldx, uint8_t* q,
                                                                  int64_t ldq,
                                                                  const float* __restrict__ scale,
                                                                  const int32_t* __restrict__ azp,
                                                                  Units u, int64_t K, Tail tail) {
    AzpParams a;
    if constexpr (DYNAMIC) {
        float hi, nlo;
        reduce_range(q, ldq, K, tail, hi, nlo);
        a = azp_params(hi, nlo);
    } else {
        a.s = scale ? *scale : 1.0f;
        a.r = 1.0 / static_cast<double>(a.s);
        a.zf = azp ? static_cast<float>(*azp) : 0.0f;
    }
    for (uint32_t base = blockIdx.x * kUnroll; base < u.total; base += gridDim.x * kUnroll) {
        float v[kUnroll][8];
        bool ok[kUnroll];
        int64_t row[kUnroll], k[kUnroll], off[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            ok[j] = unit_coords(u, base + j, K, row[j], k[j]);
            if (DYNAMIC && ok[j] && row[j] * K + k[j] >= tail.start) ok[j] = false;
            off[j] = row[j] * ldx + k[j];
        }
        load_units<XT, true>(x, off, ok, v);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j)
            if (ok[j]) *reinterpret_cast<u32x2*>(q + row[j] * ldq + k[j]) = quant8_azp(v[j], a.r, a.zf);
    }
}

// One workgroup: scale and zero point from the partials, written out, then
// the tail's codes over the partials once every thread has read them.
template <int XT>
__global__ __launch_bounds__(kBlock) void finish_tail_azp_kernel(const void* __restrict__ x,
                                                                 int64_t ldx, uint8_t* q,
                                                                 int64_t ldq, float* scale,
                                                                 int32_t* azp, int64_t M,
                                                                 int64_t K, Tail tail) {
    float hi, nlo;
    reduce_range(q, ldq, K, tail, hi, nlo);
    const AzpParams a = azp_params(hi, nlo);
    __syncthreads();  // every partial has been read
    if (threadIdx.x == 0) {
        *scale = a.s;
        *azp = static_cast<int32_t>(a.zf);
    }
    for (int64_t e = tail.start + 8 * static_cast<int64_t>(threadIdx.x); e < M * K; e += 8 * kBlock) {
        const int64_t row = e / K, k = e % K;  // 8 elements, never across a row (K % 16 == 0)
        float v[8];
        load8<XT>(x, row * ldx + k, v);
        *reinterpret_cast<u32x2*>(q + row * ldq + k) = quant8_azp(v, a.r, a.zf);
    }
}

// scale 1.0, zero point -128: the range [0, 0] of an empty tensor
__global__ void fill_azp_empty_kernel(float* s, int32_t* z) {
    *s = 1.0f;
    *z = -128;
}

template <int XT>
hipError_t per_tensor_azp_typed(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                int64_t ldq, float* scale, int32_t* azp, bool dynamic,
                                hipStream_t st) {
    const Units u = make_units(M, K);
    const int g = grid_for(u.total, kUnroll);
    if (!dynamic) {
        if (M * K == 0) return hipSuccess;
        hipLaunchKernelGGL((quant_tensor_azp_kernel<XT, false>), dim3(g), dim3(kBlock), 0, st, x, ldx, q, ldq,
                           static_cast<const float*>(scale), static_cast<const int32_t*>(azp), u, K, Tail{0, 0});
        return hipGetLastError();
    }
    const int64_t total = M * K;
    if (total == 0) {
        hipLaunchKernelGGL(fill_azp_empty_kernel, dim3(1), dim3(1), 0, st, scale, azp);
        return hipGetLastError();
    }
    Tail tail;
    tail.parts = std::min(grid_for(u.total, kAbsUnroll), 1024);
    const int64_t tail_len = (8 * static_cast<int64_t>(tail.parts) + 15) / 16 * 16;
    tail.start = total <= 65536 ? 0 : total - tail_len;
    hipLaunchKernelGGL((range_kernel<XT>), dim3(tail.parts), dim3(kBlock), 0, st, x, ldx, u, K, q, ldq, tail);
    if (tail.start > 0)
        hipLaunchKernelGGL((quant_tensor_azp_kernel<XT, true>), dim3(std::min(g, 2048)), dim3(kBlock), 0, st, x, ldx,
                           q, ldq, static_cast<const float*>(scale), static_cast<const int32_t*>(azp), u, K, tail);
    hipLaunchKernelGGL((finish_tail_azp_kernel<XT>), dim3(1), dim3(kBlock), 0, st, x, ldx, q, ldq, scale, azp, M, K, tail);
    return hipGetLastError();
}

// Per-row sums of int8 weight codes: one wave per row.
__global__ __launch_bounds__(kBlock) void colsum_kernel(const uint8_t* __restrict__ b, int64_t ldb,
                                                       int64_t N, int64_t K, int32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + (threadIdx.x >> 6);
    if (row >= N) return;
    int sum = 0;
    for (int64_t k = 16 * lane; k < K; k += 1024) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(b + row * ldb + k);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum += static_cast<int8_t>(c[j] >> (8 * e));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
    if (lane == 0) out[row] = sum;
}

hipError_t launch_quant_per_token_azp(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* scales, int32_t* azp,
                                      hipStream_t st) {
    if (M == 0) return hipSuccess;
    const dim3 g(static_cast<unsigned>(M)), blk(kBlock);
    switch (xt) {
        case D_BF16: hipLaunchKernelGGL((quant_rows_azp_kernel<D_BF16>), g, blk, 0, st, x, ldx, q, ldq, scales, azp, K); break;
        case D_FP16: hipLaunchKernelGGL((quant_rows_azp_kernel<D_FP16>), g, blk, 0, st, x, ldx, q, ldq, scales, azp, K); break;
        default: hipLaunchKernelGGL((quant_rows_azp_kernel<D_F32>), g, blk, 0, st, x, ldx, q, ldq, scales, azp, K); break;
    }
    return hipGetLastError();
}

hipError_t launch_quant_per_tensor_azp(int xt, const void* x, int64_t M, int64_t K, int64_t ldx,
                                       uint8_t* q, int64_t ldq, float* scale, int32_t* azp,
                                       bool dynamic, hipStream_t st) {
    switch (xt) {
        case D_BF16: return per_tensor_azp_typed<D_BF16>(x, M, K, ldx, q, ldq, scale, azp, dynamic, st);
        case D_FP16: return per_tensor_azp_typed<D_FP16>(x, M, K, ldx, q, ldq, scale, azp, dynamic, st);
        default: return per_tensor_azp_typed<D_F32>(x, M, K, ldx, q, ldq, scale, azp, dynamic, st);
    }
}

hipError_t launch_colsum(const uint8_t* b, int64_t ldb, int64_t N, int64_t K, int32_t* colsum,
                         hipStream_t st) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(colsum_kernel, dim3(static_cast<unsigned>((N + kBlock / 64 - 1) / (kBlock / 64))),
                       dim3(kBlock), 0, st, b, ldb, N, K, colsum);
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Merged layers [P2]: S shards stacked along N (QKV, gate_up), shard i on
// rows [end[i-1], end[i]) with its own per-tensor weight scale s_i.
// ------------------------------------------------------------------------
struct ShardTable {
    int S;
    int64_t end[kMaxShards];  // running row counts; end[S-1] = N
};

// The shard of row n: the number of shard ends at or below n (unrolled over
// the table so that it is indexed statically, from the kernel arguments).
__device__ __forceinline__ int shard_of(const ShardTable& t, int64_t n) {
    int i = 0;
#pragma unroll
    for (int j = 0; j < kMaxShards - 1; ++j)
        if (j < t.S - 1) i += n >= t.end[j] ? 1 : 0;
    return i;
}

__global__ __launch_bounds__(kBlock) void expand_shard_scales_kernel(const float* __restrict__ s,
                                                                    ShardTable t,
                                                                    float* __restrict__ out) {
    const int64_t n = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (n < t.end[t.S - 1]) out[n] = s[shard_of(t, n)];
}

// One wave per row at a time (the row's shard, and so its ratio, is uniform
// across the wave), 2 KB of the row in flight per wave: the int8 encode keeps
// many registers live, and the smaller unroll leaves room for more waves per
// CU, which streams faster than more bytes per wave. The codes are written
// with non-temporal stores (nothing reads them back soon). The shared scale is
// the largest shard scale; the row's ratio t = s_i / s is rounded once to
// binary32 (the double quotient of two binary32 values rounds to the same
// binary32 value as the exact one: 53 >= 2 * 24 + 2 bits), and every code
// becomes enc(fl32(dec(c) * t)).
constexpr int kRequantUnroll = 2;  // 16-byte chunks per lane in flight

template <int QT>
__device__ __forceinline__ uint32_t requant4(uint32_t c, float ratio) {
    float d0, d1, d2, d3;
    if constexpr (QT == Q_FP8) {
        d0 = __builtin_amdgcn_cvt_f32_fp8(c, 0);
        d1 = __builtin_amdgcn_cvt_f32_fp8(c, 1);
        d2 = __builtin_amdgcn_cvt_f32_fp8(c, 2);
        d3 = __builtin_amdgcn_cvt_f32_fp8(c, 3);
    } else {
        d0 = static_cast<float>(static_cast<int8_t>(c));
        d1 = static_cast<float>(static_cast<int8_t>(c >> 8));
        d2 = static_cast<float>(static_cast<int8_t>(c >> 16));
        d3 = static_cast<float>(static_cast<int8_t>(c >> 24));
    }
    const float v0 = d0 * ratio, v1 = d1 * ratio, v2 = d2 * ratio, v3 = d3 * ratio;
    return QT == Q_FP8 ? enc4_fp8(v0, v1, v2, v3) : enc4_i8(v0, v1, v2, v3);
}

template <int QT>
__global__ __launch_bounds__(kBlock) void requant_shared_kernel(const uint8_t* __restrict__ w, int64_t ldw,
                                                               int64_t K, const float* __restrict__ s,
                                                               ShardTable t, uint8_t* out, int64_t ldo,
                                                               float* __restrict__ shared) {
    __shared__ float smax_lds;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (wave == 0) {
        // scales are positive: 0 is neutral for the lanes past S
        float v = lane < t.S ? s[lane] : 0.0f;
        v = wave_max(v);
        if (lane == 0) smax_lds = v;
    }
    __syncthreads();
    const float smax = smax_lds;
    if (blockIdx.x == 0 && threadIdx.x == 0) *shared = smax;
    const int64_t N = t.end[t.S - 1];
    constexpr int kWaves = kBlock / 64;
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + wave; row < N;
         row += static_cast<int64_t>(gridDim.x) * kWaves) {
        const int64_t r = __builtin_amdgcn_readfirstlane(static_cast<int>(row));
        const float ratio =
            static_cast<float>(static_cast<double>(s[shard_of(t, r)]) / static_cast<double>(smax));
        const uint8_t* src = w + r * ldw;
        uint8_t* dst = out + r * ldo;
        for (int64_t k0 = 16 * lane; k0 < K; k0 += 1024 * kRequantUnroll) {
            u32x4 c[kRequantUnroll];
#pragma unroll
            for (int u = 0; u < kRequantUnroll; ++u)
                if (k0 + 1024 * u < K) c[u] = *reinterpret_cast<const u32x4*>(src + k0 + 1024 * u);
#pragma unroll
            for (int u = 0; u < kRequantUnroll; ++u) {
                if (k0 + 1024 * u >= K) continue;
                u32x4 q;
#pragma unroll
                for (int j = 0; j < 4; ++j) q[j] = requant4<QT>(c[u][j], ratio);
                __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(dst + k0 + 1024 * u));
            }
        }
    }
}

static ShardTable shard_table(const int64_t* rows, int64_t S) {
    ShardTable t{};
    t.S = static_cast<int>(S);
    int64_t n = 0;
    for (int64_t i = 0; i < S; ++i) t.end[i] = (n += rows[i]);
    return t;
}

hipError_t launch_expand_shard_scales(const float* s, const int64_t* rows, int64_t S, float* out,
                                      hipStream_t st) {
    const ShardTable t = shard_table(rows, S);
    const int64_t N = t.end[S - 1];
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(expand_shard_scales_kernel, dim3(static_cast<unsigned>((N + kBlock - 1) / kBlock)),
                       dim3(kBlock), 0, st, s, t, out);
    return hipGetLastError();
}

hipError_t launch_requant_shared_scale(const uint8_t* w, int64_t ldw, int qt, int64_t K,
                                       const int64_t* rows, int64_t S, const float* s, uint8_t* out,
                                       int64_t ldo, float* shared, hipStream_t st) {
    const ShardTable t = shard_table(rows, S);
    // a wave per row, at most 8 workgroups per CU's worth of grid (a grid-stride over rows)
    const int64_t wg = (t.end[S - 1] + kBlock / 64 - 1) / (kBlock / 64);
    const unsigned g = static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>(wg, 1), 2048));
    if (qt == Q_FP8)
        hipLaunchKernelGGL((requant_shared_kernel<Q_FP8>), dim3(g), dim3(kBlock), 0, st, w, ldw, K, s, t, out, ldo, shared);
    else
        hipLaunchKernelGGL((requant_shared_kernel<Q_INT8>), dim3(g), dim3(kBlock), 0, st, w, ldw, K, s, t, out, ldo, shared);
    return hipGetLastError();
}

hipError_t launch_kv_dequant(const uint8_t* q, int64_t n, const float* scale, void* x, int xt,
                             hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int g = grid_for(static_cast<uint64_t>(n / 8), static_cast<uint64_t>(kBlock) * kDequantUnroll);
    switch (xt) {
        case D_BF16: hipLaunchKernelGGL((kv_dequant_kernel<D_BF16>), dim3(g), dim3(kBlock), 0, st, q, n, scale, x); break;
        case D_FP16: hipLaunchKernelGGL((kv_dequant_kernel<D_FP16>), dim3(g), dim3(kBlock), 0, st, q, n, scale, x); break;
        default: hipLaunchKernelGGL((kv_dequant_kernel<D_F32>), dim3(g), dim3(kBlock), 0, st, q, n, scale, x); break;
    }
    return hipGetLastError();
}

}  // namespace w8a8

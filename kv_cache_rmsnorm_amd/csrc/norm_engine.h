// norm_engine.h -- the row-norm kernels and their launch-shape dispatch.
//
// RMSNorm as defined in the koas-w.github.io 2026-03-31 post, section 3
// (pow, mean, add eps, rsqrt, mul x, mul weight; fp32 inside, one cast back
// on write) and m.lsln.cn/news/61269 section 2.3; the residual-add variant
// from section 4 of the koas-w post (x updated in place to the sum, the
// normalised sum returned).
//
// gfx950 design
//  * A row group of LANES = 64 * WPR lanes owns one row at a time. Vector
//    slot j of lane l holds the 16-byte vector number j * LANES + l of the
//    row, so each load instruction of a wave reads 1 KiB of consecutive
//    bytes, and the row is read from HBM exactly once into registers (the
//    one-pass form of the csdn "Qwen3 from scratch (4-2)" page).
//  * WPR waves share a row (1..8, chosen per width, see norm_shape), with a
//    two-slot LDS exchange of the wave partial sums when WPR > 1.
//  * The sum of squares is reduced in-wave with DPP and v_readlane (no LDS,
//    no barrier when WPR = 1).
//  * Ragged widths (1536, 2176, primes) need no power-of-two padding: only
//    the vector that straddles the end of a row is read element by element.
//    A row whose base is not 16-byte aligned (odd widths packed densely) is
//    accessed element by element; the choice is uniform per row.
//  * One-pass grid (a workgroup per GROUPS rows) with nontemporal loads and
//    stores: on MI355X this streams HBM 10-20% faster than a persistent
//    grid-stride loop; the weight is read once per workgroup (from L2).
//  * Rows wider than the register-resident engine (4096 vectors) take the
//    two-pass form of the Zhihu "RMSNorm in Triton" page (loop 1: sum of
//    squares; loop 2: reload, scale, write), one 1024-lane workgroup per
//    row. While the row fits in the 160 KB of LDS, loop 1 parks every
//    vector there and loop 2 reads it back, so HBM still sees the row once;
//    wider rows are read twice (the second time mostly from L2/MALL).
#pragma once

#include "norm.h"

namespace kcr {

template <typename T>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t stride) {
    return static_cast<const typename T::storage*>(base) + row * stride;
}
template <typename T>
__device__ __forceinline__ void* row_ptr(void* base, int64_t row, int64_t stride) {
    return static_cast<typename T::storage*>(base) + row * stride;
}

// Launch shape of the row engine: VPT 16-byte vectors per lane, WPR waves
// per row, GROUPS rows per workgroup, nontemporal loads (NTL) and stores
// (NTS) for the streamed rows.
template <int VPT_, int WPR_, int GROUPS_, bool NTL_, bool NTS_>
struct NormCfg {
    static constexpr int VPT = VPT_, WPR = WPR_, GROUPS = GROUPS_;
    static constexpr bool NTL = NTL_, NTS = NTS_;
    static constexpr int BLOCK = 64 * WPR * GROUPS;
};

template <typename T, typename C, bool ADD>
__global__ __launch_bounds__(C::BLOCK) void row_norm_kernel(const NormArgs a) {
    constexpr int kVec = T::kVec, VPT = C::VPT, WPR = C::WPR, GROUPS = C::GROUPS;
    constexpr int LANES = 64 * WPR;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int grp = wave / WPR;                    // row group within the workgroup
    const int rl = (wave % WPR) * 64 + lane;       // lane within the row group
    const int64_t d = a.d;

    // The weight, once per workgroup, in registers.
    const bool vw = aligned16(a.w);
    u32x4 wr[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) wr[j] = load_raw<T, false>(a.w, (int64_t)(j * LANES + rl) * kVec, d, vw);

    __shared__ float part[2][GROUPS][WPR];
    int it = 0;
    // The loop bound depends only on the workgroup, so every wave reaches
    // every barrier; `live` is uniform per row group.
    for (int64_t base = (int64_t)blockIdx.x * GROUPS; base < a.rows;
         base += (int64_t)gridDim.x * GROUPS, ++it) {
        const int64_t row = base + grp;
        const bool live = row < a.rows;
        u32x4 xr[VPT];
        float ss = 0.0f;
        bool vx = false;
        if (live) {
            const void* xrow = row_ptr<T>(a.x, row, a.x_stride);
            vx = aligned16(xrow);  // row-uniform: vector or element access
#pragma unroll
            for (int j = 0; j < VPT; ++j)
                xr[j] = load_raw<T, C::NTL>(xrow, (int64_t)(j * LANES + rl) * kVec, d, vx);
            if constexpr (ADD) {
                const void* drow = row_ptr<T>(a.delta, row, a.delta_stride);
                const bool vd = aligned16(drow);
                u32x4 dr[VPT];
#pragma unroll
                for (int j = 0; j < VPT; ++j)
                    dr[j] = load_raw<T, C::NTL>(drow, (int64_t)(j * LANES + rl) * kVec, d, vd);
                void* orow = row_ptr<T>(a.x_out, row, a.x_stride);
#pragma unroll
                for (int j = 0; j < VPT; ++j) {
                    float xf[kVec], df[kVec];
                    unpack<T>(xr[j], xf);
                    unpack<T>(dr[j], df);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) xf[e] += df[e];
                    xr[j] = pack<T>(xf);  // the rounded sum: stored, and normalised below
                    store_raw<T, C::NTS>(orow, (int64_t)(j * LANES + rl) * kVec, d, xr[j], vx);
                }
            }
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                float xf[kVec];
                unpack<T>(xr[j], xf);
#pragma unroll
                for (int e = 0; e < kVec; ++e) ss += xf[e] * xf[e];
            }
        }
        ss = wave_sum(ss);
        if constexpr (WPR > 1) {
            float* slot = part[it & 1][grp];
            if (lane == 0) slot[wave % WPR] = ss;
            __syncthreads();
            ss = 0.0f;
#pragma unroll
            for (int i = 0; i < WPR; ++i) ss += slot[i];
        }
        if (live) {
            const float r = __builtin_amdgcn_rsqf(ss / (float)a.d + a.eps);
            void* yrow = row_ptr<T>(a.y, row, a.y_stride);
            const bool vy = aligned16(yrow);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                float xf[kVec], wf[kVec], yf[kVec];
                unpack<T>(xr[j], xf);
                unpack<T>(wr[j], wf);
#pragma unroll
                for (int e = 0; e < kVec; ++e) yf[e] = xf[e] * r * wf[e];
                store_raw<T, C::NTS>(yrow, (int64_t)(j * LANES + rl) * kVec, d, pack<T>(yf), vy);
            }
        }
    }
}

// Launches with a grid of ceil(rows / GROUPS) workgroups, capped at
// `wgs_per_cu` resident rounds per CU (a large cap gives a one-pass grid).
template <typename T, typename C, bool ADD>
static int launch_norm(const NormArgs& a, void* stream, int wgs_per_cu) {
    const dim3 grid(grid_for(a.rows, C::GROUPS, device_cus(), wgs_per_cu));
    return launch(row_norm_kernel<T, C, ADD>, grid, dim3(C::BLOCK), stream, a);
}

// ------------------------------------------------------------ wide rows
constexpr int kWideThreads = 1024;
constexpr int kWideWaves = kWideThreads / 64;
constexpr int kWideUnroll = 8;        // vectors in flight per lane in loop 1

// Two-pass row norm, one row per workgroup at a time. Lane t owns vectors
// t, t + 1024, t + 2048, ... of the row in both loops; with STAGED, loop 1
// keeps them in `stage` (private to the lane, so no barrier guards it) and
// loop 2 reads them back. The add variant stores the rounded sum in loop 1
// and normalises that stored value, as the register engine does.
template <typename T, bool ADD, bool STAGED>
__global__ __launch_bounds__(kWideThreads) void wide_norm_kernel(const NormArgs a) {
    extern __shared__ u32x4 stage[];
    __shared__ float part[2][kWideWaves];
    constexpr int kVec = T::kVec;
    constexpr bool kNtLoad = STAGED;  // a row read twice keeps its lines in L2
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int64_t d = a.d;
    const int nvec = (a.d + kVec - 1) / kVec;
    const bool vw = aligned16(a.w);
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const void* xrow = row_ptr<T>(a.x, row, a.x_stride);
        const bool vx = aligned16(xrow);
        const void* drow = ADD ? row_ptr<T>(a.delta, row, a.delta_stride) : nullptr;
        const bool vd = ADD && aligned16(drow);
        void* orow = ADD ? row_ptr<T>(a.x_out, row, a.x_stride) : nullptr;
        float ss = 0.0f;
        for (int v0 = tid; v0 < nvec; v0 += kWideThreads * kWideUnroll) {
            u32x4 xr[kWideUnroll];
#pragma unroll
            for (int u = 0; u < kWideUnroll; ++u) {
                const int v = v0 + u * kWideThreads;
                xr[u] = u32x4{0u, 0u, 0u, 0u};
                if (v < nvec) xr[u] = load_raw<T, kNtLoad>(xrow, (int64_t)v * kVec, d, vx);
            }
            if constexpr (ADD) {
                u32x4 dr[kWideUnroll];
#pragma unroll
                for (int u = 0; u < kWideUnroll; ++u) {
                    const int v = v0 + u * kWideThreads;
                    dr[u] = u32x4{0u, 0u, 0u, 0u};
                    if (v < nvec) dr[u] = load_raw<T, kNtLoad>(drow, (int64_t)v * kVec, d, vd);
                }
#pragma unroll
                for (int u = 0; u < kWideUnroll; ++u) {
                    const int v = v0 + u * kWideThreads;
                    if (v >= nvec) continue;
                    float xf[kVec], df[kVec];
                    unpack<T>(xr[u], xf);
                    unpack<T>(dr[u], df);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) xf[e] += df[e];
                    xr[u] = pack<T>(xf);
                    store_raw<T, STAGED>(orow, (int64_t)v * kVec, d, xr[u], vx);
                }
            }
#pragma unroll
            for (int u = 0; u < kWideUnroll; ++u) {
                const int v = v0 + u * kWideThreads;
                if (v >= nvec) continue;
                if constexpr (STAGED) stage[v] = xr[u];
                float xf[kVec];
                unpack<T>(xr[u], xf);
#pragma unroll
                for (int e = 0; e < kVec; ++e) ss += xf[e] * xf[e];
            }
        }
        ss = wave_sum(ss);
        if (lane == 0) part[it & 1][wave] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int i = 0; i < kWideWaves; ++i) tot += part[it & 1][i];
        const float r = __builtin_amdgcn_rsqf(tot / (float)a.d + a.eps);

        const void* src = ADD ? static_cast<const void*>(orow) : xrow;
        void* yrow = row_ptr<T>(a.y, row, a.y_stride);
        const bool vy = aligned16(yrow);
        for (int v = tid; v < nvec; v += kWideThreads) {
            const u32x4 xv = STAGED ? stage[v] : load_raw<T, false>(src, (int64_t)v * kVec, d, vx);
            const u32x4 wv = load_raw<T, false>(a.w, (int64_t)v * kVec, d, vw);
            float xf[kVec], wf[kVec], yf[kVec];
            unpack<T>(xv, xf);
            unpack<T>(wv, wf);
#pragma unroll
            for (int e = 0; e < kVec; ++e) yf[e] = xf[e] * r * wf[e];
            store_raw<T, true>(yrow, (int64_t)v * kVec, d, pack<T>(yf), vy);
        }
    }
}


constexpr size_t kWideStaticLds = 2 * kWideWaves * sizeof(float);
constexpr int64_t kWideGridCap = 1 << 16;

template <typename T, bool ADD>
static int launch_wide(const NormArgs& a, void* stream) {
    const int64_t nvec = (a.d + T::kVec - 1) / T::kVec;
    const dim3 grid((uint32_t)(a.rows < kWideGridCap ? a.rows : kWideGridCap));
    const size_t stage = (size_t)nvec * 16;
    if (stage + kWideStaticLds <= lds_per_block()) {
        auto kern = wide_norm_kernel<T, ADD, true>;
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)stage) != hipSuccess)
            return KCR_ERR_LAUNCH;
        return launch(kern, grid, dim3(kWideThreads), stream, a, stage);
    }
    return launch(wide_norm_kernel<T, ADD, false>, grid, dim3(kWideThreads), stream, a);
}

// ------------------------------------------------------------ dispatch
template <typename T, bool ADD, int VPT, int WPR>
static int launch_g(const NormArgs& a, void* stream, int groups) {
    constexpr int kOnePass = 1 << 20;  // grid cap per CU: effectively one pass
    if (groups == 4) return launch_norm<T, NormCfg<VPT, WPR, 4, true, true>, ADD>(a, stream, kOnePass);
    if (groups == 2) return launch_norm<T, NormCfg<VPT, WPR, 2, true, true>, ADD>(a, stream, kOnePass);
    return launch_norm<T, NormCfg<VPT, WPR, 1, true, true>, ADD>(a, stream, kOnePass);
}

template <typename T, bool ADD, int WPR>
static int launch_w(const NormArgs& a, void* stream, int vpt, int groups) {
    switch (vpt) {
        case 1: return launch_g<T, ADD, 1, WPR>(a, stream, groups);
        case 2: return launch_g<T, ADD, 2, WPR>(a, stream, groups);
        case 3: return launch_g<T, ADD, 3, WPR>(a, stream, groups);
        case 4: return launch_g<T, ADD, 4, WPR>(a, stream, groups);
        case 5: return launch_g<T, ADD, 5, WPR>(a, stream, groups);
        case 6: return WPR == 8 ? launch_g<T, ADD, 6, WPR>(a, stream, groups) : KCR_ERR_SHAPE;
        case 7: return WPR == 8 ? launch_g<T, ADD, 7, WPR>(a, stream, groups) : KCR_ERR_SHAPE;
        case 8: return WPR == 8 ? launch_g<T, ADD, 8, WPR>(a, stream, groups) : KCR_ERR_SHAPE;
    }
    return KCR_ERR_SHAPE;
}

template <typename T, bool ADD>
int run_norm(const NormArgs& a, void* stream) {
    if ((a.d + T::kVec - 1) / T::kVec > kRegMaxVec) return launch_wide<T, ADD>(a, stream);
    const NormShape s = norm_shape((a.d + T::kVec - 1) / T::kVec, ADD);
    switch (s.wpr) {
        case 1: return launch_w<T, ADD, 1>(a, stream, s.vpt, s.groups);
        case 2: return launch_w<T, ADD, 2>(a, stream, s.vpt, s.groups);
        case 3: return launch_w<T, ADD, 3>(a, stream, s.vpt, s.groups);
        case 4: return launch_w<T, ADD, 4>(a, stream, s.vpt, s.groups);
        case 5: return launch_w<T, ADD, 5>(a, stream, s.vpt, s.groups);
        case 6: return launch_w<T, ADD, 6>(a, stream, s.vpt, s.groups);
        case 7: return launch_w<T, ADD, 7>(a, stream, s.vpt, s.groups);
        case 8: return launch_w<T, ADD, 8>(a, stream, s.vpt, s.groups);
    }
    return KCR_ERR_SHAPE;
}

}  // namespace kcr

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
//  * WPR waves share a row (1..8, chosen per width, see norm_shape), with an
//    LDS exchange of the wave partial sums when WPR > 1. A row group may
//    take RPG rows, all read before any is written: longer read-only then
//    write-only phases per wave stream HBM better on MI355X.
//  * The sum of squares is reduced in-wave with DPP, ending in lane 63 (no
//    LDS, no barrier when WPR = 1), and the mean square is that sum times
//    the width's reciprocal.
//  * Ragged widths (1536, 2176, primes) need no power-of-two padding: only
//    the vector that straddles the end of a row is read element by element.
//    Vectors need only dword alignment, so rows of e.g. 8196 bf16 still move
//    as 16-byte vectors; a row at an odd 2-byte offset (odd widths packed
//    densely) is accessed element by element; the choice is uniform per row.
//  * One-pass grid (a workgroup per GROUPS * RPG rows, no loop) with
//    nontemporal loads and stores: on MI355X this streams HBM 10-20% faster
//    than a persistent grid-stride loop; the weight is read once per
//    workgroup (from L2).
//  * Rows wider than the register-resident engine (4096 vectors) take the
//    two-pass form of the csdn page "Qwen3 from scratch (4-2): RMSNorm with
//    Triton", section "basic Triton implementation" (loop 1: sum of
//    squares; loop 2: reload, scale, write), one 1024-lane workgroup per
//    row. While the row fits in the 160 KB of LDS, loop 1 parks every
//    vector there and loop 2 reads it back, so HBM still sees the row once;
//    of wider rows, the part beyond LDS is read twice (the second time
//    mostly from L2/MALL).
#pragma once

#include <atomic>

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
// per row, GROUPS row groups per workgroup, RPG rows per row group (all RPG
// rows are read before any is written), nontemporal loads (NTL) and stores
// (NTS) for the streamed rows.
template <int VPT_, int WPR_, int GROUPS_, bool NTL_, bool NTS_, int RPG_ = 1, bool EAGER_ = false>
struct NormCfg {
    static constexpr int VPT = VPT_, WPR = WPR_, GROUPS = GROUPS_, RPG = RPG_;
    static constexpr bool NTL = NTL_, NTS = NTS_, EAGER = EAGER_;  // EAGER: see load_whole
    static constexpr int BLOCK = 64 * WPR * GROUPS;
};

// VEC: the host has checked that every row base (x, delta, y, w) is dword
// aligned, so the kernel carries no per-row alignment test (measured 3-4%
// faster than testing each row at run time).
template <typename T, typename C, bool ADD, bool VEC>
__global__ __launch_bounds__(C::BLOCK) void row_norm_kernel(const NormArgs a) {
    constexpr int kVec = T::kVec, VPT = C::VPT, WPR = C::WPR, GROUPS = C::GROUPS, RPG = C::RPG;
    constexpr int LANES = 64 * WPR;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int grp = wave / WPR;                    // row group within the workgroup
    const int rl = (wave % WPR) * 64 + lane;       // lane within the row group
    const int64_t d = a.d;
    const float inv_d = inv_width(a.d);
    // One pass: workgroup b owns rows [b * GROUPS * RPG, (b + 1) * GROUPS * RPG).
    // (A loop over several row blocks per workgroup measured 2-5% slower: the
    // compiler then waits for the weight before the first row load.)
    const int64_t row0 = ((int64_t)blockIdx.x * GROUPS + grp) * RPG;

    // The weight, once per workgroup (an L2 hit), in registers.
    const bool vw = VEC || vec_ok(a.w);
    // EAGER (small calls whose shape leaves lanes past the row's end; the
    // host sends only dword-aligned rows there): whole vectors first, and
    // the one vector that straddles the end once every load is in flight.
    constexpr bool kTail = C::EAGER && VEC;
    const bool ragged = kTail && d % kVec != 0;
    u32x4 wr[VPT];
    if constexpr (kTail) {
#pragma unroll
        for (int j = 0; j < VPT; ++j) wr[j] = load_whole<T, false>(a.w, (int64_t)(j * LANES + rl) * kVec, d);
    } else {
#pragma unroll
        for (int j = 0; j < VPT; ++j) wr[j] = load_raw<T, false>(a.w, (int64_t)(j * LANES + rl) * kVec, d, vw);
    }

    // All RPG rows are read before any is written. `live[r]` is uniform per
    // row group; every wave reaches the barrier.
    u32x4 xr[RPG][VPT];
    float ss[RPG];
    bool live[RPG], vx[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        live[r] = row0 + r < a.rows;
        ss[r] = 0.0f;
        vx[r] = false;
        if (live[r]) {
            const void* xrow = row_ptr<T>(a.x, row0 + r, a.x_stride);
            vx[r] = VEC || vec_ok(xrow);  // row-uniform: vector or element access
            if constexpr (kTail) {
#pragma unroll
                for (int j = 0; j < VPT; ++j)
                    xr[r][j] = load_whole<T, C::NTL>(xrow, (int64_t)(j * LANES + rl) * kVec, d);
            } else {
#pragma unroll
                for (int j = 0; j < VPT; ++j)
                    xr[r][j] = load_raw<T, C::NTL>(xrow, (int64_t)(j * LANES + rl) * kVec, d, vx[r]);
            }
        }
    }
    // The straddling vectors of the weight and of x (for the add variant,
    // after its delta loads below are issued too).
    auto tails = [&]() {
        if (!ragged) return;
#pragma unroll
        for (int j = 0; j < VPT; ++j) load_tail<T>(a.w, (int64_t)(j * LANES + rl) * kVec, d, wr[j]);
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            if (!live[r]) continue;
            const void* xrow = row_ptr<T>(a.x, row0 + r, a.x_stride);
#pragma unroll
            for (int j = 0; j < VPT; ++j) load_tail<T>(xrow, (int64_t)(j * LANES + rl) * kVec, d, xr[r][j]);
        }
    };
    if constexpr (kTail && !ADD) tails();
    if constexpr (ADD) {
        u32x4 dr[RPG][VPT];
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            if (!live[r]) continue;
            const void* drow = row_ptr<T>(a.delta, row0 + r, a.delta_stride);
            const bool vd = VEC || vec_ok(drow);
            if constexpr (kTail) {
#pragma unroll
                for (int j = 0; j < VPT; ++j)
                    dr[r][j] = load_whole<T, C::NTL>(drow, (int64_t)(j * LANES + rl) * kVec, d);
            } else {
#pragma unroll
                for (int j = 0; j < VPT; ++j)
                    dr[r][j] = load_raw<T, C::NTL>(drow, (int64_t)(j * LANES + rl) * kVec, d, vd);
            }
        }
        if constexpr (kTail) {
            tails();
            if (ragged) {
#pragma unroll
                for (int r = 0; r < RPG; ++r) {
                    if (!live[r]) continue;
                    const void* drow = row_ptr<T>(a.delta, row0 + r, a.delta_stride);
#pragma unroll
                    for (int j = 0; j < VPT; ++j)
                        load_tail<T>(drow, (int64_t)(j * LANES + rl) * kVec, d, dr[r][j]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            if (!live[r]) continue;
            void* orow = row_ptr<T>(a.x_out, row0 + r, a.x_stride);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                float xf[kVec], df[kVec];
                unpack<T>(xr[r][j], xf);
                unpack<T>(dr[r][j], df);
#pragma unroll
                for (int e = 0; e < kVec; ++e) xf[e] += df[e];
                xr[r][j] = pack<T>(xf);  // the rounded sum: stored, and normalised below
                store_raw<T, C::NTS>(orow, (int64_t)(j * LANES + rl) * kVec, d, xr[r][j], vx[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        if (live[r]) {
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                float xf[kVec];
                unpack<T>(xr[r][j], xf);
#pragma unroll
                for (int e = 0; e < kVec; ++e) ss[r] += xf[e] * xf[e];
            }
        }
        // (with several waves per row only lane 63 publishes the wave's sum)
        ss[r] = WPR > 1 ? wave_total_lane63(ss[r]) : wave_sum(ss[r]);
    }
    if constexpr (WPR > 1) {
        __shared__ float part[RPG][GROUPS][WPR];
        if (lane == 63) {
#pragma unroll
            for (int r = 0; r < RPG; ++r) part[r][grp][wave % WPR] = ss[r];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            ss[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < WPR; ++i) ss[r] += part[r][grp][i];
        }
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        if (!live[r]) continue;
        const float rs = __builtin_amdgcn_rsqf(ss[r] * inv_d + a.eps);
        void* yrow = row_ptr<T>(a.y, row0 + r, a.y_stride);
        const bool vy = VEC || vec_ok(yrow);
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            float xf[kVec], wf[kVec], yf[kVec];
            unpack<T>(xr[r][j], xf);
            unpack<T>(wr[j], wf);
#pragma unroll
            for (int e = 0; e < kVec; ++e) yf[e] = xf[e] * rs * wf[e];
            store_raw<T, C::NTS>(yrow, (int64_t)(j * LANES + rl) * kVec, d, pack<T>(yf), vy);
        }
    }
}

// Launches ceil(rows / (GROUPS * RPG)) workgroups. A grid holds at most
// 2^32 - 1 work-items, so a call with more rows than that covers is split
// into several launches over consecutive row ranges.
template <typename T, typename C, bool ADD, bool VEC = true>
static int launch_norm(const NormArgs& a, void* stream) {
    constexpr int64_t kRowsPerWg = (int64_t)C::GROUPS * C::RPG;
    constexpr int64_t kMaxWgs = (int64_t)0xFFFFFFFFu / C::BLOCK;
    constexpr int64_t es = sizeof(typename T::storage);
    const int64_t per_launch = kMaxWgs * kRowsPerWg;
    for (int64_t off = 0; off < a.rows; off += per_launch) {
        NormArgs c = a;
        c.rows = a.rows - off < per_launch ? a.rows - off : per_launch;
        c.x = static_cast<const char*>(a.x) + off * a.x_stride * es;
        c.y = static_cast<char*>(a.y) + off * a.y_stride * es;
        if (ADD) {
            c.x_out = static_cast<char*>(a.x_out) + off * a.x_stride * es;
            c.delta = static_cast<const char*>(a.delta) + off * a.delta_stride * es;
        }
        const dim3 grid((uint32_t)((c.rows + kRowsPerWg - 1) / kRowsPerWg));
        const int rc = launch(row_norm_kernel<T, C, ADD, VEC>, grid, dim3(C::BLOCK), stream, c);
        if (rc != KCR_OK) return rc;
    }
    return KCR_OK;
}

template <typename T, bool ADD>
static bool rows_dword_aligned(const NormArgs& a);

// ------------------------------------------------------- decode-size rows
// Small calls whose rows are whole 16-byte vectors (every row base dword
// aligned), at most VPT * 64 of them: one wave per row, lane l holding
// vectors l, l + 64, ..., so the row needs no LDS exchange. The code is kept
// to the straight line the decode chain rewards: every load of the row is
// issued before the first wait, offsets within the row are 32-bit, and there
// is no element path. In the 28-layer, batch-256 decode chain on MI355X (a
// graph of 112 launches) this took the step from 331 to 314 us against the
// row engine at the same sizes; the next launches' loads waited less (RoPE's
// median load latency 373 -> 224 ns) when the add kernel's stores followed
// this pattern.
// RAGGED: the row has fewer than VPT * 64 vectors. Lanes past its end load
// the row's last vector (in bounds, on lines the wave reads anyway), select
// zero in place of it and store nothing, so the loads stay unconditional:
// at [512, 2176] bf16, 2.92 against 3.20 us per launch in a graph for the
// row engine's one-wave shape with predicated loads.
template <typename T, int VPT, bool ADD, bool RAGGED = false>
__global__ __launch_bounds__(64) void row_norm_wave_kernel(const NormArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec;
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float inv_d = inv_width(a.d);
    const S* xr = static_cast<const S*>(a.x) + row * a.x_stride;
    const S* dr = ADD ? static_cast<const S*>(a.delta) + row * a.delta_stride : nullptr;
    u32x4 x[VPT], dv[VPT], w[VPT];
    bool in[VPT];  // RAGGED: the lane's vector j lies in the row
    if constexpr (RAGGED) {
        const int nvec = a.d / kVec;  // whole vectors (checked on the host)
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = j * 64 + lane;
            in[j] = v < nvec;
            const int e = (in[j] ? v : nvec - 1) * kVec;
            x[j] = ld16_nt<T>(xr, e);
            if constexpr (ADD) dv[j] = ld16_nt<T>(dr, e);
            w[j] = ld16<T>(a.w, e);
        }
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            x[j] = in[j] ? x[j] : z;
            if constexpr (ADD) dv[j] = in[j] ? dv[j] : z;
        }
    } else {
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int e = (j * 64 + lane) * kVec;
            x[j] = ld16_nt<T>(xr, e);
            if constexpr (ADD) dv[j] = ld16_nt<T>(dr, e);
            w[j] = ld16<T>(a.w, e);
        }
    }
    float ss = 0.0f;
    S* const xo = ADD ? static_cast<S*>(a.x_out) + row * a.x_stride : nullptr;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float xf[kVec];
        unpack<T>(x[j], xf);
        if constexpr (ADD) {
            float df[kVec];
            unpack<T>(dv[j], df);
#pragma unroll
            for (int e = 0; e < kVec; ++e) xf[e] += df[e];
            x[j] = pack<T>(xf);  // the rounded sum: stored, and normalised below
            if (!RAGGED || in[j]) st16_nt<T>(xo, (j * 64 + lane) * kVec, x[j]);
            unpack<T>(x[j], xf);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) ss += xf[e] * xf[e];
    }
    ss = wave_sum(ss);
    const float rs = __builtin_amdgcn_rsqf(ss * inv_d + a.eps);
    S* const yr = static_cast<S*>(a.y) + row * a.y_stride;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float xf[kVec], wf[kVec], yf[kVec];
        unpack<T>(x[j], xf);
        unpack<T>(w[j], wf);
#pragma unroll
        for (int e = 0; e < kVec; ++e) yf[e] = xf[e] * rs * wf[e];
        if (!RAGGED || in[j]) st16_nt<T>(yr, (j * 64 + lane) * kVec, pack<T>(yf));
    }
}

// Rows of whole vectors short of a multiple of 64 take one wave while they
// need at most this many vectors per lane: 5 plain (where the rule gives one
// wave too), 4 for the add variant. Measured in graphs of [512, D] launches
// on MI355X against the rule's shapes: plain D = 1000 and 2176 bf16, 1000
// fp32 5-9% faster; add D = 1000 bf16 and fp32 7-8% faster, D = 2176 bf16
// 1% slower; one wave of 6-8 vectors 3-10% slower.
template <bool ADD>
constexpr int kRaggedWaveMaxVpt = ADD ? 4 : 5;

// Launches row_norm_wave_kernel when the call qualifies (dword-aligned rows
// of whole vectors: exactly 64, 128, ..., 512 of them, or a ragged count up
// to kRaggedWaveMaxVpt * 64); returns 1 when it does not.
template <typename T, bool ADD>
static int launch_wave_rows(const NormArgs& a, void* stream) {
    constexpr int64_t kRow = 64 * T::kVec;
    if (a.d % T::kVec != 0 || !rows_dword_aligned<T, ADD>(a)) return 1;
    // one 64-lane workgroup per row; small calls stay far below 2^26 rows
    if (a.rows >= (int64_t(1) << 26)) return 1;
    const int64_t vpt = (a.d + kRow - 1) / kRow;
    const bool exact = a.d % kRow == 0;
    if (vpt > (exact ? 8 : kRaggedWaveMaxVpt<ADD>)) return 1;
    const dim3 grid((uint32_t)a.rows), block(64);
    if (!exact) {
        switch (vpt) {
            case 1: return launch(row_norm_wave_kernel<T, 1, ADD, true>, grid, block, stream, a);
            case 2: return launch(row_norm_wave_kernel<T, 2, ADD, true>, grid, block, stream, a);
            case 3: return launch(row_norm_wave_kernel<T, 3, ADD, true>, grid, block, stream, a);
            case 4: return launch(row_norm_wave_kernel<T, 4, ADD, true>, grid, block, stream, a);
            default:
                if constexpr (kRaggedWaveMaxVpt<ADD> >= 5)
                    return launch(row_norm_wave_kernel<T, 5, ADD, true>, grid, block, stream, a);
                return 1;
        }
    }
    switch (vpt) {
        case 1: return launch(row_norm_wave_kernel<T, 1, ADD>, grid, block, stream, a);
        case 2: return launch(row_norm_wave_kernel<T, 2, ADD>, grid, block, stream, a);
        case 3: return launch(row_norm_wave_kernel<T, 3, ADD>, grid, block, stream, a);
        case 4: return launch(row_norm_wave_kernel<T, 4, ADD>, grid, block, stream, a);
        case 5: return launch(row_norm_wave_kernel<T, 5, ADD>, grid, block, stream, a);
        case 6: return launch(row_norm_wave_kernel<T, 6, ADD>, grid, block, stream, a);
        case 7: return launch(row_norm_wave_kernel<T, 7, ADD>, grid, block, stream, a);
        default: return launch(row_norm_wave_kernel<T, 8, ADD>, grid, block, stream, a);
    }
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
    const float inv_d = inv_width(a.d);
    const int nvec = (a.d + kVec - 1) / kVec;
    const bool vw = vec_ok(a.w);
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const void* xrow = row_ptr<T>(a.x, row, a.x_stride);
        const bool vx = vec_ok(xrow);
        const void* drow = ADD ? row_ptr<T>(a.delta, row, a.delta_stride) : nullptr;
        const bool vd = ADD && vec_ok(drow);
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
        ss = wave_total_lane63(ss);
        if (lane == 63) part[it & 1][wave] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int i = 0; i < kWideWaves; ++i) tot += part[it & 1][i];
        const float r = __builtin_amdgcn_rsqf(tot * inv_d + a.eps);

        const void* src = ADD ? static_cast<const void*>(orow) : xrow;
        void* yrow = row_ptr<T>(a.y, row, a.y_stride);
        const bool vy = vec_ok(yrow);
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


// Two-pass row norm for rows wider than LDS: lane t owns vectors
// t + k * 1024 of the row; the first `lds_vecs` vectors of the row stay in
// LDS after loop 1, and only those beyond are read again in loop 2 (from L2
// or the Infinity Cache when they are still there), so the extra traffic is
// the part that fits nowhere. U vectors per lane are in flight per step of
// loop 1. Measured on MI355X at [512, 262144] bf16: 128.4 us with the LDS
// full, against 139.7 us re-reading the whole row; also keeping 2 or 4
// vectors per lane in registers measured 140-164 us (the register tier
// lengthens loop 1 without adding bytes in flight), so there is none.
struct TierArgs {
    NormArgs n;
    int32_t lds_vecs;  // vectors of each row kept in LDS
};

template <typename T, bool ADD, int U>
__global__ __launch_bounds__(kWideThreads) void wide_tier_kernel(const TierArgs ta) {
    extern __shared__ u32x4 stage[];
    __shared__ float part[2][kWideWaves];
    const NormArgs& a = ta.n;
    const int lds_vecs = ta.lds_vecs;
    constexpr int kVec = T::kVec, W = kWideThreads;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int64_t d = a.d;
    const float inv_d = inv_width(a.d);
    const int nvec = (int)((d + kVec - 1) / kVec);
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const void* xrow = row_ptr<T>(a.x, row, a.x_stride);
        const bool vx = vec_ok(xrow);
        const void* drow = ADD ? row_ptr<T>(a.delta, row, a.delta_stride) : nullptr;
        const bool vd = ADD && vec_ok(drow);
        void* orow = ADD ? row_ptr<T>(a.x_out, row, a.x_stride) : nullptr;
        float ss = 0.0f;
        // Loop 1: the part kept in LDS with nontemporal loads, the part read
        // again with cached ones; the add variant stores the rounded sum,
        // which is what the norm sees (and what loop 2 reads again).
        for (int v0 = tid; v0 < nvec; v0 += W * U) {
            u32x4 xv[U], dv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * W;
                xv[u] = u32x4{0u, 0u, 0u, 0u};
                dv[u] = xv[u];
                if (v < nvec) {
                    xv[u] = v < lds_vecs ? load_raw<T, true>(xrow, (int64_t)v * kVec, d, vx)
                                         : load_raw<T, false>(xrow, (int64_t)v * kVec, d, vx);
                    if constexpr (ADD) dv[u] = load_raw<T, true>(drow, (int64_t)v * kVec, d, vd);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * W;
                if (v >= nvec) continue;
                float xf[kVec];
                unpack<T>(xv[u], xf);
                if constexpr (ADD) {
                    float df[kVec];
                    unpack<T>(dv[u], df);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) xf[e] += df[e];
                    xv[u] = pack<T>(xf);
                    store_raw<T, true>(orow, (int64_t)v * kVec, d, xv[u], vx);
                    unpack<T>(xv[u], xf);
                }
#pragma unroll
                for (int e = 0; e < kVec; ++e) ss += xf[e] * xf[e];
                if (v < lds_vecs) stage[v] = xv[u];
            }
        }
        ss = wave_total_lane63(ss);
        if (lane == 63) part[it & 1][wave] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int i = 0; i < kWideWaves; ++i) tot += part[it & 1][i];
        const float r = __builtin_amdgcn_rsqf(tot * inv_d + a.eps);

        // Loop 2: the same lane owns the same vectors as in loop 1.
        void* yrow = row_ptr<T>(a.y, row, a.y_stride);
        const bool vy = vec_ok(yrow);
        const bool vw = vec_ok(a.w);
        const void* src = ADD ? static_cast<const void*>(orow) : xrow;
        for (int v = tid; v < nvec; v += W) {
            const u32x4 xv = v < lds_vecs ? stage[v] : load_raw<T, false>(src, (int64_t)v * kVec, d, vx);
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

// A kernel's dynamic-LDS limit is raised once per device to all the device
// allows beyond the kernel's static LDS, so every launch fits under it and
// concurrent calls with different widths never race on the attribute.
template <typename T, bool ADD, bool TIER>
static bool wide_lds_ready(size_t limit) {
    static std::atomic<int> done[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
    if (done[dev].load(std::memory_order_acquire)) return true;
    const void* kern = TIER ? reinterpret_cast<const void*>(wide_tier_kernel<T, ADD, kWideUnroll>)
                            : reinterpret_cast<const void*>(wide_norm_kernel<T, ADD, true>);
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)limit) != hipSuccess)
        return false;
    done[dev].store(1, std::memory_order_release);
    return true;
}

// Rows that fit in LDS: the staged kernel (read once). Wider rows: the
// tiered kernel with as much of the row in LDS as fits and the rest read
// again.
template <typename T, bool ADD>
static int launch_wide(const NormArgs& a, void* stream) {
    const int64_t nvec = (a.d + T::kVec - 1) / T::kVec;
    const dim3 grid((uint32_t)(a.rows < kWideGridCap ? a.rows : kWideGridCap));
    const size_t stage = (size_t)nvec * 16;
    const size_t lds = lds_per_block();
    const size_t cap = lds > kWideStaticLds ? lds - kWideStaticLds : 0;
    if (cap > 0 && stage <= cap) {
        if (!wide_lds_ready<T, ADD, false>(cap)) return KCR_ERR_LAUNCH;
        return launch(wide_norm_kernel<T, ADD, true>, grid, dim3(kWideThreads), stream, a, stage);
    }
    const int lds_vecs = (int)(cap / 16);
    if (lds_vecs > 0 && !wide_lds_ready<T, ADD, true>(cap)) return KCR_ERR_LAUNCH;
    return launch(wide_tier_kernel<T, ADD, kWideUnroll>, grid, dim3(kWideThreads), stream,
                  TierArgs{a, lds_vecs}, (size_t)lds_vecs * 16);
}

// ------------------------------------------------------------ dispatch
// Large calls: the rule's shape with the rule's row groups per workgroup.
// Only the shapes the rule can return are instantiated (kRuleShapes).
template <typename T, bool ADD, int VPT, int WPR>
static int launch_rule(const NormArgs& a, void* stream) {
    constexpr int G = kRuleShapes<ADD>.groups[VPT][WPR];
    if constexpr (G == 0) return KCR_ERR_SHAPE;
    else return launch_norm<T, NormCfg<VPT, WPR, G, true, true>, ADD>(a, stream);
}

// Small calls (decode batches): the rule's shape with one row group per
// workgroup. In the 28-layer, batch-256 decode chain on MI355X (a captured
// graph of 112 launches) this takes the step from 341 to 335 us against the
// two-group shapes that win at large shapes. Loads and stores stay nontemporal: cached
// ones measured 20-34 us slower per step there, since every kernel must
// write its dirty L2 lines back before the next one starts. Small calls are
// latency-bound: where the shape leaves lanes past the row's end, they issue
// every load before waiting (EAGER, load_whole); where every lane holds a whole
// vector, the plain form saves the zeroing moves.
template <typename T, bool ADD, int VPT, int WPR, bool EAGER>
static int launch_rule_small(const NormArgs& a, void* stream) {
    if constexpr (kRuleShapes<ADD>.groups[VPT][WPR] == 0) return KCR_ERR_SHAPE;
    else return launch_norm<T, NormCfg<VPT, WPR, 1, true, true, 1, EAGER>, ADD>(a, stream);
}

template <typename T, bool ADD, int VPT>
static int launch_rule_v(const NormArgs& a, void* stream, int wpr, bool small, bool eager) {
    switch (wpr) {
#define KCR_RULE_CASE(W)                                                                    \
    case W:                                                                                 \
        if (!small) return launch_rule<T, ADD, VPT, W>(a, stream);                          \
        return eager ? launch_rule_small<T, ADD, VPT, W, true>(a, stream)                   \
                     : launch_rule_small<T, ADD, VPT, W, false>(a, stream);
        KCR_RULE_CASE(1) KCR_RULE_CASE(2) KCR_RULE_CASE(3) KCR_RULE_CASE(4)
        KCR_RULE_CASE(5) KCR_RULE_CASE(6) KCR_RULE_CASE(7) KCR_RULE_CASE(8)
#undef KCR_RULE_CASE
    }
    return KCR_ERR_SHAPE;
}

template <typename T, bool ADD>
static int launch_by_rule(const NormArgs& a, void* stream, const NormShape& s, bool small) {
    const int64_t nvec = (a.d + T::kVec - 1) / T::kVec;
    if (!small && kRuleShapes<ADD>.groups[s.vpt][s.wpr] != s.groups) return KCR_ERR_SHAPE;
    const bool eager = (int64_t)s.vpt * 64 * s.wpr > nvec;
    switch (s.vpt) {
        case 1: return launch_rule_v<T, ADD, 1>(a, stream, s.wpr, small, eager);
        case 2: return launch_rule_v<T, ADD, 2>(a, stream, s.wpr, small, eager);
        case 3: return launch_rule_v<T, ADD, 3>(a, stream, s.wpr, small, eager);
        case 4: return launch_rule_v<T, ADD, 4>(a, stream, s.wpr, small, eager);
        case 5: return launch_rule_v<T, ADD, 5>(a, stream, s.wpr, small, eager);
        case 6: return launch_rule_v<T, ADD, 6>(a, stream, s.wpr, small, eager);
        case 7: return launch_rule_v<T, ADD, 7>(a, stream, s.wpr, small, eager);
        case 8: return launch_rule_v<T, ADD, 8>(a, stream, s.wpr, small, eager);
    }
    return KCR_ERR_SHAPE;
}

// Shapes measured best for plain rows at common model widths on MI355X
// (about 570 MB per call, four repeats each), 2.5-5% above the rule's shape
// there; other widths, small calls and the add variant take the rule.
template <typename T>
static int launch_tuned(const NormArgs& a, void* stream) {
    if constexpr (T::kVec == 8) {
        switch (a.d) {
            case 1536: return launch_norm<T, NormCfg<1, 3, 2, true, true, 2>, false>(a, stream);
            case 2048: return launch_norm<T, NormCfg<3, 2, 1, true, true, 1>, false>(a, stream);
            case 2176: return launch_norm<T, NormCfg<3, 2, 2, true, true, 2>, false>(a, stream);
            case 4096: return launch_norm<T, NormCfg<1, 8, 1, true, true, 2>, false>(a, stream);
            case 5120: return launch_norm<T, NormCfg<4, 3, 2, true, true, 1>, false>(a, stream);
        }
    } else {
        if (a.d == 1024) return launch_norm<T, NormCfg<1, 4, 1, true, true, 1>, false>(a, stream);
        // 2 waves x 5 vectors, 4 rows per workgroup: 6.25-6.28 TB/s at
        // [131072, 2176] against 6.17-6.20 for the rule's 3 x 3 shape.
        if (a.d == 2176) return launch_norm<T, NormCfg<5, 2, 4, true, true, 1>, false>(a, stream);
    }
    return 1;  // not in the table
}

// Whether every row of the call starts on a dword boundary (base pointers
// and strides in bytes); always true for fp32.
template <typename T, bool ADD>
static bool rows_dword_aligned(const NormArgs& a) {
    constexpr int64_t es = sizeof(typename T::storage);
    auto ok = [](const void* p, int64_t stride) { return vec_ok(p) && (stride * es) % 4 == 0; };
    return ok(a.x, a.x_stride) && ok(a.y, a.y_stride) && vec_ok(a.w) &&
           (!ADD || ok(a.delta, a.delta_stride));
}

// Calls with rows at odd 2-byte offsets (element access for those rows): a
// small fixed family of shapes that test each row's alignment at run time.
template <typename T, bool ADD>
static int launch_unaligned(const NormArgs& a, void* stream) {
    const int64_t nvec = (a.d + T::kVec - 1) / T::kVec;
    if (nvec <= 8 * 64) {
        switch ((nvec + 63) / 64) {
            case 1: return launch_norm<T, NormCfg<1, 1, 2, true, true>, ADD, false>(a, stream);
            case 2: return launch_norm<T, NormCfg<2, 1, 2, true, true>, ADD, false>(a, stream);
            case 3: return launch_norm<T, NormCfg<3, 1, 2, true, true>, ADD, false>(a, stream);
            case 4: return launch_norm<T, NormCfg<4, 1, 2, true, true>, ADD, false>(a, stream);
            case 5: return launch_norm<T, NormCfg<5, 1, 2, true, true>, ADD, false>(a, stream);
            case 6: return launch_norm<T, NormCfg<6, 1, 2, true, true>, ADD, false>(a, stream);
            case 7: return launch_norm<T, NormCfg<7, 1, 2, true, true>, ADD, false>(a, stream);
            case 8: return launch_norm<T, NormCfg<8, 1, 2, true, true>, ADD, false>(a, stream);
        }
    }
    switch ((nvec + 511) / 512) {  // 2..8 here: up to 512 vectors took the one-wave shapes
        case 2: return launch_norm<T, NormCfg<2, 8, 1, true, true>, ADD, false>(a, stream);
        case 3: return launch_norm<T, NormCfg<3, 8, 1, true, true>, ADD, false>(a, stream);
        case 4: return launch_norm<T, NormCfg<4, 8, 1, true, true>, ADD, false>(a, stream);
        case 5: return launch_norm<T, NormCfg<5, 8, 1, true, true>, ADD, false>(a, stream);
        case 6: return launch_norm<T, NormCfg<6, 8, 1, true, true>, ADD, false>(a, stream);
        case 7: return launch_norm<T, NormCfg<7, 8, 1, true, true>, ADD, false>(a, stream);
        case 8: return launch_norm<T, NormCfg<8, 8, 1, true, true>, ADD, false>(a, stream);
    }
    return KCR_ERR_SHAPE;
}

// Bytes a call streams (rows read and written; the add variant also reads
// delta and writes x back).
template <typename T, bool ADD>
static int64_t norm_call_bytes(const NormArgs& a) {
    return (ADD ? 4 : 2) * a.rows * (int64_t)a.d * (int64_t)sizeof(typename T::storage);
}

template <typename T, bool ADD>
int run_norm(const NormArgs& a, void* stream) {
    if ((a.d + T::kVec - 1) / T::kVec > kRegMaxVec) return launch_wide<T, ADD>(a, stream);
    if constexpr (sizeof(typename T::storage) < 4) {
        if (!rows_dword_aligned<T, ADD>(a)) return launch_unaligned<T, ADD>(a, stream);
    }
    if (!ADD && a.rows >= kTunedMinRows) {
        const int rc = launch_tuned<T>(a, stream);
        if (rc <= 0) return rc;
    }
    const NormShape s = norm_shape((a.d + T::kVec - 1) / T::kVec, ADD);
    if (norm_call_bytes<T, ADD>(a) <= kNormSmallCallBytes) {
        const int rc = launch_wave_rows<T, ADD>(a, stream);
        if (rc <= 0) return rc;
        return launch_by_rule<T, ADD>(a, stream, s, true);
    }
    return launch_by_rule<T, ADD>(a, stream, s, false);
}

}  // namespace kcr

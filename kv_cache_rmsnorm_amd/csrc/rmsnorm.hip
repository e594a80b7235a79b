// rmsnorm.hip -- the row-norm engine behind kcr_rmsnorm and kcr_add_rmsnorm.
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
//  * WPR = 1 (one wave per row, four rows per 256-lane workgroup) up to
//    16 vectors per lane: 8192 bf16 or 4096 fp32 columns. Wider rows use a
//    256-lane workgroup per row (WPR = 4) and a two-slot LDS exchange of the
//    four wave partial sums.
//  * The sum of squares is reduced in-wave with DPP and v_readlane (no LDS,
//    no barrier when WPR = 1).
//  * Ragged widths (1536, 2176, primes) need no power-of-two padding: only
//    the vector that straddles the end of a row is read element by element.
//    A row whose base is not 16-byte aligned (odd widths packed densely) is
//    accessed element by element; the choice is uniform per row.
//  * Grid-stride over rows with the weight held in registers for every row
//    a group processes; the grid is capped at a few resident workgroups per
//    CU, so large batches run as a persistent grid and batch-1 decode as a
//    single workgroup.
#include "kcr_device.h"
#include "kcr_host.h"

namespace kcr {

struct NormArgs {
    const void* x;      // input rows
    void* x_out;        // add variant: where round(x + delta) goes (== x)
    const void* delta;  // add variant: the residual branch
    const void* w;      // [d] weight
    void* y;            // output rows
    int64_t x_stride, delta_stride, y_stride;  // elements
    int64_t rows;
    int32_t d;
    float eps;
};

template <typename T>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t stride) {
    return static_cast<const typename T::storage*>(base) + row * stride;
}
template <typename T>
__device__ __forceinline__ void* row_ptr(void* base, int64_t row, int64_t stride) {
    return static_cast<typename T::storage*>(base) + row * stride;
}

template <typename T, int VPT, int WPR, bool ADD>
__global__ __launch_bounds__(WPR == 1 ? 256 : 64 * WPR) void row_norm_kernel(const NormArgs a) {
    constexpr int kVec = T::kVec;
    constexpr int LANES = 64 * WPR;
    constexpr int GROUPS = WPR == 1 ? 4 : 1;  // row groups per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int grp = WPR == 1 ? wave : 0;
    const int rl = (WPR == 1 ? 0 : wave) * 64 + lane;  // lane within the row group
    const int64_t d = a.d;

    // The weight, once per row group, in registers.
    const bool vw = aligned16(a.w);
    u32x4 wr[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) wr[j] = load_raw<T, false>(a.w, (int64_t)(j * LANES + rl) * kVec, d, vw);

    __shared__ float part[2][WPR];
    int it = 0;
    for (int64_t row = (int64_t)blockIdx.x * GROUPS + grp; row < a.rows;
         row += (int64_t)gridDim.x * GROUPS, ++it) {
        u32x4 xr[VPT];
        const void* xrow = row_ptr<T>(a.x, row, a.x_stride);
        const bool vx = aligned16(xrow);  // row-uniform: vector or element access
#pragma unroll
        for (int j = 0; j < VPT; ++j) xr[j] = load_raw<T, false>(xrow, (int64_t)(j * LANES + rl) * kVec, d, vx);

        if constexpr (ADD) {
            const void* drow = row_ptr<T>(a.delta, row, a.delta_stride);
            const bool vd = aligned16(drow);
            u32x4 dr[VPT];
#pragma unroll
            for (int j = 0; j < VPT; ++j)
                dr[j] = load_raw<T, false>(drow, (int64_t)(j * LANES + rl) * kVec, d, vd);
            void* orow = row_ptr<T>(a.x_out, row, a.x_stride);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                float xf[kVec], df[kVec];
                unpack<T>(xr[j], xf);
                unpack<T>(dr[j], df);
#pragma unroll
                for (int e = 0; e < kVec; ++e) xf[e] += df[e];
                xr[j] = pack<T>(xf);  // the rounded sum: stored, and normalised below
                store_raw<T, false>(orow, (int64_t)(j * LANES + rl) * kVec, d, xr[j], vx);
            }
        }

        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            float xf[kVec];
            unpack<T>(xr[j], xf);
#pragma unroll
            for (int e = 0; e < kVec; ++e) ss += xf[e] * xf[e];
        }
        ss = wave_sum(ss);
        if constexpr (WPR > 1) {
            float* slot = part[it & 1];
            if (lane == 0) slot[wave] = ss;
            __syncthreads();
            ss = 0.0f;
#pragma unroll
            for (int i = 0; i < WPR; ++i) ss += slot[i];
        }
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
            store_raw<T, false>(yrow, (int64_t)(j * LANES + rl) * kVec, d, pack<T>(yf), vy);
        }
    }
}

// Resident workgroups per CU that the grid-stride launch aims for.
constexpr int kNormWgsPerCu = 8;

template <typename T, int VPT, int WPR, bool ADD>
static int launch_norm(const NormArgs& a, void* stream) {
    constexpr int GROUPS = WPR == 1 ? 4 : 1;
    const dim3 block(WPR == 1 ? 256 : 64 * WPR);
    const dim3 grid(grid_for(a.rows, GROUPS, device_cus(), kNormWgsPerCu));
    return launch(row_norm_kernel<T, VPT, WPR, ADD>, grid, block, stream, a);
}

// Vectors per lane for one wave per row (WPR = 1) and for a 4-wave row
// group (WPR = 4); the 4-wave buckets are coarser.
constexpr int kWaveMaxVpt = 16;
constexpr int kWgBuckets[] = {6, 8, 10, 12, 16};

// (VPT, WPR) for a row of `nvec` 16-byte vectors; VPT = 0 if too wide.
struct NormShape {
    int vpt, wpr;
};
inline NormShape norm_shape(int64_t nvec) {
    if (nvec <= (int64_t)kWaveMaxVpt * 64) return {(int)((nvec + 63) / 64), 1};
    for (int b : kWgBuckets)
        if (nvec <= (int64_t)b * 256) return {b, 4};
    return {0, 0};
}

template <typename T, bool ADD>
static int dispatch_norm(const NormArgs& a, void* stream) {
    const NormShape s = norm_shape((a.d + T::kVec - 1) / T::kVec);
    if (s.wpr == 1) {
        switch (s.vpt) {
            case 1: return launch_norm<T, 1, 1, ADD>(a, stream);
            case 2: return launch_norm<T, 2, 1, ADD>(a, stream);
            case 3: return launch_norm<T, 3, 1, ADD>(a, stream);
            case 4: return launch_norm<T, 4, 1, ADD>(a, stream);
            case 5: return launch_norm<T, 5, 1, ADD>(a, stream);
            case 6: return launch_norm<T, 6, 1, ADD>(a, stream);
            case 7: return launch_norm<T, 7, 1, ADD>(a, stream);
            case 8: return launch_norm<T, 8, 1, ADD>(a, stream);
            case 9: return launch_norm<T, 9, 1, ADD>(a, stream);
            case 10: return launch_norm<T, 10, 1, ADD>(a, stream);
            case 11: return launch_norm<T, 11, 1, ADD>(a, stream);
            case 12: return launch_norm<T, 12, 1, ADD>(a, stream);
            case 13: return launch_norm<T, 13, 1, ADD>(a, stream);
            case 14: return launch_norm<T, 14, 1, ADD>(a, stream);
            case 15: return launch_norm<T, 15, 1, ADD>(a, stream);
            case 16: return launch_norm<T, 16, 1, ADD>(a, stream);
        }
    } else if (s.wpr == 4) {
        switch (s.vpt) {
            case 6: return launch_norm<T, 6, 4, ADD>(a, stream);
            case 8: return launch_norm<T, 8, 4, ADD>(a, stream);
            case 10: return launch_norm<T, 10, 4, ADD>(a, stream);
            case 12: return launch_norm<T, 12, 4, ADD>(a, stream);
            case 16: return launch_norm<T, 16, 4, ADD>(a, stream);
        }
    }
    return KCR_ERR_SHAPE;
}

static int check_norm_common(int64_t rows, int64_t d, int dtype, const void* w, const void* y,
                             int64_t y_stride) {
    if (!dtype_ok(dtype)) return KCR_ERR_DTYPE;
    if (rows < 0 || d < 1) return KCR_ERR_SHAPE;
    if (d > (dtype == KCR_BF16 ? KCR_NORM_MAX_D_BF16 : KCR_NORM_MAX_D_F32)) return KCR_ERR_SHAPE;
    if (rows == 0) return KCR_OK;
    if (!w || !y) return KCR_ERR_NULL;
    if (y_stride < d) return KCR_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    if (!aligned_elem(w, es) || !aligned_elem(y, es)) return KCR_ERR_ALIGN;
    return KCR_OK;
}

}  // namespace kcr

using namespace kcr;

extern "C" int kcr_rmsnorm(const void* x, int64_t x_stride, const void* w, void* y,
                           int64_t y_stride, int64_t rows, int64_t d, float eps, int dtype,
                           void* stream) {
    int rc = check_norm_common(rows, d, dtype, w, y, y_stride);
    if (rc != KCR_OK || rows == 0) return rc;
    if (!x) return KCR_ERR_NULL;
    if (x_stride < d) return KCR_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    if (!aligned_elem(x, es)) return KCR_ERR_ALIGN;
    const Span sx = span2d(x, rows, x_stride, d, es), sy = span2d(y, rows, y_stride, d, es);
    const Span sw = span2d(w, 1, d, d, es);
    const bool in_place = (x == y && x_stride == y_stride);
    if ((!in_place && overlap(sx, sy)) || overlap(sy, sw)) return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;
    NormArgs a{x, nullptr, nullptr, w, y, x_stride, 0, y_stride, rows, (int32_t)d, eps};
    return dtype == KCR_BF16 ? dispatch_norm<Bf16, false>(a, stream)
                             : dispatch_norm<F32, false>(a, stream);
}

extern "C" int kcr_add_rmsnorm(void* x, int64_t x_stride, const void* delta, int64_t delta_stride,
                               const void* w, void* y, int64_t y_stride, int64_t rows, int64_t d,
                               float eps, int dtype, void* stream) {
    int rc = check_norm_common(rows, d, dtype, w, y, y_stride);
    if (rc != KCR_OK || rows == 0) return rc;
    if (!x || !delta) return KCR_ERR_NULL;
    if (x_stride < d || delta_stride < d) return KCR_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    if (!aligned_elem(x, es) || !aligned_elem(delta, es)) return KCR_ERR_ALIGN;
    const Span sx = span2d(x, rows, x_stride, d, es), sy = span2d(y, rows, y_stride, d, es);
    const Span sd = span2d(delta, rows, delta_stride, d, es), sw = span2d(w, 1, d, d, es);
    if (overlap(sy, sx) || overlap(sy, sd) || overlap(sy, sw) || overlap(sd, sx) || overlap(sx, sw))
        return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;
    NormArgs a{x, x, delta, w, y, x_stride, delta_stride, y_stride, rows, (int32_t)d, eps};
    return dtype == KCR_BF16 ? dispatch_norm<Bf16, true>(a, stream)
                             : dispatch_norm<F32, true>(a, stream);
}

// Host self-test hook: every width up to the limit maps to a shape that
// covers it. Returns 0 when all widths pass.
int kcr_norm_shape_selftest() {
    for (int dt = 0; dt < 2; ++dt) {
        const int vec = dt == 0 ? Bf16::kVec : F32::kVec;
        const int64_t maxd = dt == 0 ? KCR_NORM_MAX_D_BF16 : KCR_NORM_MAX_D_F32;
        for (int64_t d = 1; d <= maxd; ++d) {
            const int64_t nvec = (d + vec - 1) / vec;
            const NormShape s = norm_shape(nvec);
            if (s.vpt < 1 || s.vpt > 16) return 1;
            if ((int64_t)s.vpt * 64 * s.wpr < nvec) return 2;
        }
    }
    return 0;
}

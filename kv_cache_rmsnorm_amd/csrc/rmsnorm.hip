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

// ------------------------------------------------------------ dispatch
// The launch shape for a row of `nvec` 16-byte vectors, chosen from sweeps
// of every (VPT, WPR, GROUPS) on MI355X at widths 512..8192 in bf16 and
// fp32 (one-pass grids, nontemporal loads and stores):
//  * HBM streams best when each lane holds only a few vectors of each
//    stream: one wave per row while a plain row needs at most 5 vectors per
//    lane, otherwise 2 or 3 vectors per lane over up to 8 waves, whichever
//    leaves fewer lanes idle; the add variant reads two streams and takes 1
//    or 2 vectors per lane;
//  * rows of up to 3 waves go two to a workgroup (four for single-wave rows
//    of 3 or more vectors per lane).
struct NormShape {
    int vpt, wpr, groups;
};

inline NormShape norm_shape(int64_t nvec, bool add) {
    if (nvec <= 0) return {0, 0, 0};
    if (!add && nvec <= 5 * 64) {
        const int vpt = (int)((nvec + 63) / 64);
        return {vpt, 1, vpt >= 3 ? 4 : 2};
    }
    if (add && nvec <= 64) return {1, 1, 2};
    const int lo = add ? 1 : 2, hi = add ? 2 : 3;
    int best_v = 0, best_w = 0;
    double best_util = -1.0;
    for (int v = lo; v <= hi; ++v) {
        const int64_t w = (nvec + 64 * v - 1) / (64 * v);
        if (w > 8) continue;
        const double util = (double)nvec / (double)(64 * v * w);
        if (util > best_util + 1e-9) {
            best_util = util;
            best_v = v;
            best_w = (int)w;
        }
    }
    if (best_v == 0) {  // wider than 8 waves at hi vectors per lane
        best_w = 8;
        best_v = (int)((nvec + 511) / 512);
        if (best_v > 8) return {0, 0, 0};
    }
    return {best_v, best_w, best_w <= 3 ? 2 : 1};
}

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
static int dispatch_norm(const NormArgs& a, void* stream) {
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
// covers it, within the instantiated range. Returns 0 when all widths pass.
int kcr_norm_shape_selftest() {
    for (int dt = 0; dt < 2; ++dt) {
        const int vec = dt == 0 ? Bf16::kVec : F32::kVec;
        const int64_t maxd = dt == 0 ? KCR_NORM_MAX_D_BF16 : KCR_NORM_MAX_D_F32;
        for (int add = 0; add < 2; ++add)
            for (int64_t d = 1; d <= maxd; ++d) {
                const int64_t nvec = (d + vec - 1) / vec;
                const NormShape s = norm_shape(nvec, add != 0);
                if (s.vpt < 1 || s.wpr < 1 || s.wpr > 8 || s.vpt > 8) return 1;
                if (s.vpt > 5 && s.wpr != 8) return 1;
                if ((int64_t)s.vpt * 64 * s.wpr < nvec) return 2;
                if (64 * s.wpr * s.groups > 1024) return 3;
            }
    }
    return 0;
}

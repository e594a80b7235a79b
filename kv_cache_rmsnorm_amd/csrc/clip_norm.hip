// clip_norm.hip -- the DyHT clip norm, y = clamp(alpha * x, lo, hi) * gamma,
// over strided [n_tok, n_head, d] views (kcr_clip_norm).
//
// DyHT(x) = y * clamp(a x, -1, 1) replaces every RMSNorm of the AsyncT model
// (mer.dev "AsyncT vLLM notes (1)", section 0), and the page's clip-norm
// kernel (section 3.3) computes clamp(a x, clip_min, clip_max) * g with a
// and g per channel or scalar. That section also names the pitfall this
// interface avoids: Q/K are narrow views of the fused QKV projection, and a
// kernel with a single row stride gets [N, H, D] views wrong, so the view's
// token and head strides are both taken.
//
// gfx950 design: one 16-byte vector per lane over the flat space (token,
// head, vector), split by multiply-shift division; 64-lane workgroups, a
// one-pass grid, nontemporal loads and stores. Per-channel parameters are
// read as vectors (L1-resident), scalars as one element. A head row whose
// base is not dword aligned is accessed element by element.
#include "kcr_device.h"
#include "kcr_host.h"

namespace kcr {

struct ClipArgs {
    const void* x;
    void* y;
    const void* alpha;
    const void* gamma;
    int64_t x_ts, x_hs, y_ts, y_hs;  // elements
    int64_t d;
    float lo, hi;
    uint32_t total;  // n_tok * n_head * vectors per head row
    FastDiv vpr;     // vectors per head row
    FastDiv heads;   // n_head
    int32_t alpha_pc, gamma_pc;
};

// APC / GPC: alpha / gamma per channel (else one scalar). VEC: every head
// row of x and y starts on a dword boundary (checked on the host), so no
// per-row alignment test is compiled in.
template <typename T, bool APC, bool GPC, bool VEC>
__global__ __launch_bounds__(64) void clip_norm_kernel(const ClipArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec;
    const uint32_t idx = blockIdx.x * 64u + threadIdx.x;
    if (idx >= a.total) return;
    const uint32_t hr = fastdiv(idx, a.vpr);
    const int64_t col = (int64_t)(idx - hr * a.vpr.d) * kVec;
    const uint32_t t = fastdiv(hr, a.heads);
    const uint32_t h = hr - t * a.heads.d;
    const S* xp = static_cast<const S*>(a.x) + (int64_t)t * a.x_ts + (int64_t)h * a.x_hs;
    S* yp = static_cast<S*>(a.y) + (int64_t)t * a.y_ts + (int64_t)h * a.y_hs;
    float xf[kVec], af[kVec], gf[kVec], yf[kVec];
    unpack<T>(load_raw<T, true>(xp, col, a.d, VEC || vec_ok(xp)), xf);
    if constexpr (APC) {
        unpack<T>(load_raw<T, false>(a.alpha, col, a.d, VEC || vec_ok(a.alpha)), af);
    } else {
        const float s = load_one<T>(a.alpha, 0);
#pragma unroll
        for (int e = 0; e < kVec; ++e) af[e] = s;
    }
    if constexpr (GPC) {
        unpack<T>(load_raw<T, false>(a.gamma, col, a.d, VEC || vec_ok(a.gamma)), gf);
    } else {
        const float s = load_one<T>(a.gamma, 0);
#pragma unroll
        for (int e = 0; e < kVec; ++e) gf[e] = s;
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) yf[e] = fminf(fmaxf(af[e] * xf[e], a.lo), a.hi) * gf[e];
    store_raw<T, true>(yp, col, a.d, pack<T>(yf), VEC || vec_ok(yp));
}

template <typename T, bool APC, bool GPC>
static int launch_clip(const ClipArgs& a, dim3 grid, void* stream, bool vec) {
    // fp32 rows are always dword aligned: only 2-byte types need element access.
    if constexpr (sizeof(typename T::storage) == 4)
        return launch(clip_norm_kernel<T, APC, GPC, true>, grid, dim3(64), stream, a);
    else
        return vec ? launch(clip_norm_kernel<T, APC, GPC, true>, grid, dim3(64), stream, a)
                   : launch(clip_norm_kernel<T, APC, GPC, false>, grid, dim3(64), stream, a);
}

}  // namespace kcr

using namespace kcr;

extern "C" int kcr_clip_norm(const void* x, int64_t x_tok_stride, int64_t x_head_stride, void* y,
                             int64_t y_tok_stride, int64_t y_head_stride, int64_t n_tok, int n_head,
                             int d, const void* alpha, int alpha_per_channel, const void* gamma,
                             int gamma_per_channel, float lo, float hi, int dtype, void* stream) {
    if (!dtype_ok(dtype)) return KCR_ERR_DTYPE;
    if (n_tok < 0 || n_head < 1 || d < 1 || !(lo <= hi)) return KCR_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const int64_t vpr = (d + (int64_t)(16 / es) - 1) / (int64_t)(16 / es);
    if (n_tok * n_head * vpr >= (int64_t(1) << 31)) return KCR_ERR_SHAPE;
    if (n_tok == 0) return KCR_OK;
    if (!x || !y || !alpha || !gamma) return KCR_ERR_NULL;
    if (x_head_stride < d || y_head_stride < d || x_tok_stride < 0 || y_tok_stride < 0)
        return KCR_ERR_SHAPE;
    if (!aligned_elem(x, es) || !aligned_elem(y, es) || !aligned_elem(alpha, es) ||
        !aligned_elem(gamma, es))
        return KCR_ERR_ALIGN;
    const Span sx = span3d(x, n_tok, x_tok_stride, n_head, x_head_stride, d, es);
    const Span sy = span3d(y, n_tok, y_tok_stride, n_head, y_head_stride, d, es);
    const Span sa = span2d(alpha, 1, 0, alpha_per_channel ? d : 1, es);
    const Span sg = span2d(gamma, 1, 0, gamma_per_channel ? d : 1, es);
    const bool in_place = x == y && x_tok_stride == y_tok_stride && x_head_stride == y_head_stride;
    if ((!in_place && overlap(sx, sy)) || overlap(sy, sa) || overlap(sy, sg)) return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;
    const uint32_t total = (uint32_t)(n_tok * n_head * vpr);
    ClipArgs a{x, y, alpha, gamma, x_tok_stride, x_head_stride, y_tok_stride, y_head_stride, d, lo, hi,
               total, make_fastdiv((uint32_t)vpr), make_fastdiv((uint32_t)n_head),
               alpha_per_channel ? 1 : 0, gamma_per_channel ? 1 : 0};
    const dim3 grid((total + 63) / 64);
    auto rows_ok = [es](const void* p, int64_t ts, int64_t hs) {
        return vec_ok(p) && (ts * (int64_t)es) % 4 == 0 && (hs * (int64_t)es) % 4 == 0;
    };
    const bool vec = rows_ok(x, x_tok_stride, x_head_stride) && rows_ok(y, y_tok_stride, y_head_stride) &&
                     (!alpha_per_channel || vec_ok(alpha)) && (!gamma_per_channel || vec_ok(gamma));
    return by_dtype(dtype, [&](auto t) {
        using T = decltype(t);
        if (alpha_per_channel)
            return gamma_per_channel ? launch_clip<T, true, true>(a, grid, stream, vec)
                                     : launch_clip<T, true, false>(a, grid, stream, vec);
        return gamma_per_channel ? launch_clip<T, false, true>(a, grid, stream, vec)
                                 : launch_clip<T, false, false>(a, grid, stream, vec);
    });
}

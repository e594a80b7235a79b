// rmsnorm.hip -- the C entry points kcr_rmsnorm and kcr_add_rmsnorm:
// argument checks, then the row-norm engine (norm_engine.h).
#include <atomic>

#include "norm.h"

namespace kcr {

// LDS bytes a workgroup may take on the current device (160 KB on gfx950),
// queried once per device (0 if there is no usable device).
size_t lds_per_block() {
    static std::atomic<size_t> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    size_t n = cache[dev].load(std::memory_order_relaxed);
    if (n) return n;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
        return 0;
    cache[dev].store((size_t)v, std::memory_order_relaxed);
    return (size_t)v;
}

static int check_norm_common(int64_t rows, int64_t d, int dtype, const void* w, const void* y,
                             int64_t y_stride) {
    if (!dtype_ok(dtype)) return KCR_ERR_DTYPE;
    if (rows < 0 || d < 1) return KCR_ERR_SHAPE;
    if (d > KCR_NORM_MAX_D) return KCR_ERR_SHAPE;
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
    return by_dtype(dtype, [&](auto t) { return run_norm<decltype(t), false>(a, stream); });
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
    return by_dtype(dtype, [&](auto t) { return run_norm<decltype(t), true>(a, stream); });
}

// Host self-test hook: every width up to the limit maps to a shape that
// covers it, within the instantiated range. Returns 0 when all widths pass.
int kcr_norm_shape_selftest() {
    for (int dt = 0; dt < 2; ++dt) {
        const int vec = dt == 0 ? Bf16::kVec : F32::kVec;
        const int64_t maxd = (int64_t)kRegMaxVec * vec;
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

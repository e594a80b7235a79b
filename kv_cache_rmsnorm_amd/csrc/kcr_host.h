// kcr_host.h -- host-side helpers of the C ABI: argument checks, the
// per-device compute-unit count, fast division constants and kernel launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kcr.h"
#include "kcr_device.h"

namespace kcr {

constexpr int kMaxDevices = 64;

// Compute units of the current device, cached per device (0 if no device).
int device_cus();

inline size_t dtype_size(int dtype) { return dtype == KCR_F32 ? 4 : 2; }
inline bool dtype_ok(int dtype) { return dtype == KCR_BF16 || dtype == KCR_F32 || dtype == KCR_F16; }

// Calls fn(Bf16{}), fn(F16{}) or fn(F32{}) for a dtype that passed dtype_ok.
template <typename Fn>
inline int by_dtype(int dtype, Fn&& fn) {
    switch (dtype) {
        case KCR_BF16: return fn(Bf16{});
        case KCR_F16: return fn(F16{});
        default: return fn(F32{});
    }
}

inline bool aligned_elem(const void* p, size_t esize) {
    return (reinterpret_cast<uintptr_t>(p) & (esize - 1)) == 0;
}
inline bool stride_ok(int64_t stride_elems, size_t esize) {
    return stride_elems >= 0 && ((uint64_t)stride_elems * esize) % 16u == 0;
}

// Byte range [lo, hi) touched by a strided 2-D tensor.
struct Span {
    uintptr_t lo, hi;
};
inline Span span2d(const void* p, int64_t rows, int64_t stride, int64_t cols, size_t esize) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (rows <= 0 || cols <= 0) return {lo, lo};
    return {lo, lo + (uintptr_t)(((rows - 1) * stride + cols) * (int64_t)esize)};
}
inline Span span3d(const void* p, int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2,
                   size_t esize) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (n0 <= 0 || n1 <= 0 || n2 <= 0) return {lo, lo};
    return {lo, lo + (uintptr_t)(((n0 - 1) * s0 + (n1 - 1) * s1 + n2) * (int64_t)esize)};
}
inline bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// True when no element of the row set A (rows x cols at row stride sa) is an
// element of B. Besides disjoint byte ranges this accepts two row sets with
// the same stride whose rows interleave, such as the gate and up halves of
// one fused [rows, 2*cols] buffer.
inline bool rows_disjoint(const void* a, int64_t sa, const void* b, int64_t sb, int64_t rows,
                          int64_t cols, size_t esize) {
    if (!overlap(span2d(a, rows, sa, cols, esize), span2d(b, rows, sb, cols, esize))) return true;
    if (sa != sb || sa <= 0) return false;
    const int64_t diff = (int64_t)(reinterpret_cast<uintptr_t>(b) - reinterpret_cast<uintptr_t>(a));
    if (diff % (int64_t)esize != 0) return false;
    const int64_t m = ((diff / (int64_t)esize) % sa + sa) % sa;
    return m >= cols && m <= sa - cols;
}

// Unsigned division by a run-time constant d >= 1 for numerators n < 2^31:
//   q = (umulhi(n, magic) + n) >> shift
// with shift = ceil(log2 d) and magic = floor(2^32 (2^shift - d) / d) + 1
// (the round-up method of Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994).
struct FastDiv {
    uint32_t d, magic, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t shift = 0;
    while ((1ull << shift) < d) ++shift;
    uint64_t magic = ((1ull << 32) * ((1ull << shift) - d)) / d + 1;
    return {d, (uint32_t)magic, shift};
}
__host__ __device__ inline uint32_t fastdiv(uint32_t n, const FastDiv& f) {
#ifdef __HIP_DEVICE_COMPILE__
    uint32_t hi = __umulhi(n, f.magic);
#else
    uint32_t hi = (uint32_t)(((uint64_t)n * f.magic) >> 32);
#endif
    return (hi + n) >> f.shift;
}

// Events armed by kcr_time_next_launch for the calling thread's next launch.
struct TimingEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
TimingEvents& next_launch_events();

// Debug mode (environment KCR_DEBUG set to a non-zero integer when the
// library first launches): after every launch the stream is synchronized
// and a kernel failure is reported as KCR_ERR_LAUNCH by the call that
// launched it. A stream under graph capture is never synchronized.
bool debug_sync();
int debug_check(void* stream);

// Launches `kern` with a single by-value argument struct and reports the
// runtime's verdict for this launch. When the calling thread armed timing
// events, the launch goes through hipExtLaunchKernel, which stamps them at
// the kernel's own start and end.
// `lds` is the dynamic LDS size in bytes.
template <typename Args>
inline int launch(void (*kern)(Args), dim3 grid, dim3 block, void* stream, const Args& args,
                  size_t lds = 0) {
    Args copy = args;
    void* params[] = {&copy};
    TimingEvents& ev = next_launch_events();
    hipError_t e;
    if (ev.start || ev.stop) {
        const TimingEvents use = ev;
        ev = TimingEvents{};
        e = hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, params, lds,
                               static_cast<hipStream_t>(stream), use.start, use.stop, 0);
    } else {
        e = hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, params, lds,
                            static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return KCR_ERR_LAUNCH;
    return debug_sync() ? debug_check(stream) : KCR_OK;
}

// Grid size for a grid-stride kernel: enough workgroups to cover `work`
// items of `per_wg` each, capped at `waves_per_cu_cap` resident rounds of
// the device.
inline uint32_t grid_for(int64_t work, int64_t per_wg, int cus, int wgs_per_cu) {
    int64_t need = (work + per_wg - 1) / per_wg;
    int64_t cap = (int64_t)(cus > 0 ? cus : 256) * wgs_per_cu;
    if (need > cap) need = cap;
    return (uint32_t)(need < 1 ? 1 : need);
}

}  // namespace kcr

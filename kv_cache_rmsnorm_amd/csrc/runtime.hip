// runtime.hip -- library-wide pieces of the C ABI: device query, the plain
// copy kernel used as the bandwidth ceiling, status strings and the host
// self-test.
#include <stdlib.h>

#include <atomic>

#include "kcr_device.h"
#include "kcr_host.h"

int kcr_norm_shape_selftest();  // rmsnorm.hip

namespace kcr {

static std::atomic<int> g_cus[kMaxDevices];

TimingEvents& next_launch_events() {
    static thread_local TimingEvents ev;
    return ev;
}

bool debug_sync() {
    static const bool on = [] {
        const char* v = getenv("KCR_DEBUG");
        return v != nullptr && atoi(v) != 0;
    }();
    return on;
}

int debug_check(void* stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return KCR_ERR_LAUNCH;
    if (cap != hipStreamCaptureStatusNone) return KCR_OK;
    if (hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) return KCR_ERR_LAUNCH;
    return KCR_OK;
}

int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 0;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

struct CopyArgs {
    u32x4* dst;
    const u32x4* src;
    int64_t n;  // 16-byte vectors
};

// One 16-byte vector per lane, 64-lane workgroups, a one-pass grid and
// nontemporal loads and stores: the fastest copy shape measured on MI355X
// (sweeps over unroll, block size, grid-stride vs one-pass and cache
// hints), so it stands for the attainable read+write bandwidth.
__global__ __launch_bounds__(64) void copy_kernel(const CopyArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (i < a.n) __builtin_nontemporal_store(__builtin_nontemporal_load(a.src + i), a.dst + i);
}

}  // namespace kcr

using namespace kcr;

extern "C" int kcr_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return KCR_ERR_SHAPE;
    if (bytes == 0) return KCR_OK;
    if (!dst || !src) return KCR_ERR_NULL;
    if (!aligned16(dst) || !aligned16(src)) return KCR_ERR_ALIGN;
    if (overlap(span2d(dst, 1, 0, bytes, 1), span2d(src, 1, 0, bytes, 1))) return KCR_ERR_ALIAS;
    const int cus = device_cus();
    if (cus <= 0) return KCR_ERR_DEVICE;
    // A grid holds at most 2^32 - 1 work-items: a copy of more vectors than
    // that (64 GiB) is split into launches over consecutive ranges.
    constexpr int64_t kPerLaunch = (int64_t)(0xFFFFFFFFu / 64) * 64;
    const int64_t n = bytes / 16;
    for (int64_t off = 0; off < n; off += kPerLaunch) {
        const CopyArgs a{static_cast<u32x4*>(dst) + off, static_cast<const u32x4*>(src) + off,
                         n - off < kPerLaunch ? n - off : kPerLaunch};
        const int rc = launch(copy_kernel, dim3((uint32_t)((a.n + 63) / 64)), dim3(64), stream, a);
        if (rc != KCR_OK) return rc;
    }
    return KCR_OK;
}

extern "C" int kcr_device_cus(void) { return device_cus(); }

extern "C" int kcr_time_next_launch(void* start_event, void* stop_event) {
    TimingEvents& ev = next_launch_events();
    ev.start = static_cast<hipEvent_t>(start_event);
    ev.stop = static_cast<hipEvent_t>(stop_event);
    return KCR_OK;
}

extern "C" const char* kcr_strerror(int status) {
    switch (status) {
        case KCR_OK: return "ok";
        case KCR_ERR_NULL: return "a required pointer is NULL";
        case KCR_ERR_SHAPE: return "a size is out of range";
        case KCR_ERR_DTYPE: return "unknown dtype";
        case KCR_ERR_ALIGN: return "pointer or stride breaks 16-byte alignment";
        case KCR_ERR_HEADS: return "n_head is not a multiple of n_kv_head";
        case KCR_ERR_ALIAS: return "an output overlaps an input";
        case KCR_ERR_LAUNCH: return "kernel launch failed";
        case KCR_ERR_DEVICE: return "no usable HIP device";
        default: return "unknown status";
    }
}

extern "C" const char* kcr_version(void) { return "kcr 0.1.0 (gfx950)"; }

extern "C" int kcr_selftest_host(void) {
    // 1: fast division, exhaustive over small divisors and numerators.
    for (uint32_t d = 1; d <= 2048; ++d) {
        const FastDiv f = make_fastdiv(d);
        for (uint32_t n = 0; n < 8192; ++n)
            if (fastdiv(n, f) != n / d) return 1;
    }
    // 2: fast division, sampled over the whole range n < 2^31 (a 64-bit LCG).
    uint64_t s = 0x9E3779B97F4A7C15ull;
    for (int i = 0; i < 200000; ++i) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        const uint32_t d = (uint32_t)(s >> 40) % 0x7FFFFFFFu + 1u;
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        const uint32_t n = (uint32_t)(s >> 33);
        const FastDiv f = make_fastdiv(d);
        if (fastdiv(n, f) != n / d) return 2;
        const uint32_t near = (n / d) * d;  // a multiple of d and its neighbour
        if (fastdiv(near, f) != near / d || (near > 0 && fastdiv(near - 1, f) != (near - 1) / d)) return 2;
    }
    // 3: every RMSNorm width maps to a register shape that covers it.
    if (kcr_norm_shape_selftest() != 0) return 3;
    // 4: interleaved halves of a fused buffer are element-disjoint; a shifted
    //    copy of the same rows is not.
    alignas(16) static char buf[64];
    if (!rows_disjoint(buf, 8, buf + 8, 8, 4, 4, 2)) return 4;
    if (rows_disjoint(buf, 8, buf + 2, 8, 4, 4, 2)) return 4;
    return 0;
}

// swiglu.hip -- SwiGLU activation, out = silu(gate) * up (kcr_swiglu).
//
// The fused kernel of the koas-w.github.io 2026-03-31 post, section 2
// ("Fused SwiGLU"): gate and up are loaded together, sigmoid, the SiLU
// product and the multiply by up happen in registers, and the output is
// written once; the (batch x seq x hidden) input is flattened so that any
// row count works.
//
// gfx950 design
//  * The index space is rows x ceil(cols / kVec) 16-byte vectors, flattened;
//    consecutive lanes take consecutive vectors, so every wave instruction
//    moves 1 KiB of consecutive bytes. The (row, vector) split uses a
//    precomputed multiply-shift division, so strided gate/up halves of a
//    fused gate_up buffer need no copy. Rows whose base is not dword
//    aligned are accessed element by element (a kernel variant that the
//    host picks only when some row needs it).
//  * One vector of gate and of up per lane, 64-lane workgroups, a one-pass
//    grid and nontemporal loads and stores: on MI355X many small waves
//    stream HBM faster than fewer waves with more loads each.
//  * sigmoid(g) = 1 / (1 + 2^(-g log2 e)) on the hardware v_exp_f32 and
//    v_rcp_f32 (no IEEE divide): two quarter-rate transcendentals per
//    element, well under the VALU budget at HBM speed.
#include "kcr_device.h"
#include "kcr_host.h"

namespace kcr {

struct SwigluArgs {
    const void* g;
    const void* u;
    void* out;
    int64_t g_stride, u_stride, out_stride;  // elements
    int64_t cols;
    uint32_t total;  // rows * vectors per row
    FastDiv vpr;     // vectors per row
};

// Gate activations times up.
struct SiluMul {  // SwiGLU: silu(g) * u, silu(g) = g / (1 + exp(-g))
    static __device__ __forceinline__ float apply(float g, float u) {
        const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);  // exp(-g)
        return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
    }
};
struct ReluMul {  // ReGLU: relu(g) * u
    static __device__ __forceinline__ float apply(float g, float u) { return (g > 0.0f ? g : 0.0f) * u; }
};

// Launch shape: BLOCK threads, UNROLL vectors of each stream per lane before
// any math, nontemporal loads (NTL) and stores (NTS).
template <int BLOCK_, int UNROLL_, bool NTL_, bool NTS_>
struct SwigluCfg {
    static constexpr int BLOCK = BLOCK_, UNROLL = UNROLL_;
    static constexpr bool NTL = NTL_, NTS = NTS_;
};

// One pass, no loop: thread i of workgroup b takes vectors
// b * BLOCK * UNROLL + k * BLOCK + i. VEC: the host has checked that every
// row base of gate, up and out is dword aligned, so no per-row alignment
// test is compiled in.
template <typename T, typename C, typename Act, bool VEC>
__global__ __launch_bounds__(C::BLOCK) void swiglu_kernel(const SwigluArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec, B = C::BLOCK, U = C::UNROLL;
    const uint32_t base = blockIdx.x * (uint32_t)(B * U) + threadIdx.x;
    u32x4 gr[U], ur[U];
    int64_t row[U], col[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const uint32_t idx = base + k * (uint32_t)B;
        if (idx < a.total) {
            const uint32_t r = fastdiv(idx, a.vpr);
            row[k] = r;
            col[k] = (int64_t)(idx - r * a.vpr.d) * kVec;
            const S* gp = static_cast<const S*>(a.g) + row[k] * a.g_stride;
            const S* up = static_cast<const S*>(a.u) + row[k] * a.u_stride;
            gr[k] = load_raw<T, C::NTL>(gp, col[k], a.cols, VEC || vec_ok(gp));
            ur[k] = load_raw<T, C::NTL>(up, col[k], a.cols, VEC || vec_ok(up));
        }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if (base + k * (uint32_t)B < a.total) {
            float gf[kVec], uf[kVec], of[kVec];
            unpack<T>(gr[k], gf);
            unpack<T>(ur[k], uf);
#pragma unroll
            for (int e = 0; e < kVec; ++e) of[e] = Act::apply(gf[e], uf[e]);
            S* op = static_cast<S*>(a.out) + row[k] * a.out_stride;
            store_raw<T, C::NTS>(op, col[k], a.cols, pack<T>(of), VEC || vec_ok(op));
        }
    }
}

// Small calls of whole-vector rows (cols a multiple of kVec, every row base
// dword aligned): workgroup b takes vectors [k * BLOCK, (k + 1) * BLOCK) of
// row b / wpr (k = b % wpr, wpr = workgroups per row), so the split into
// (row, vector) is scalar work on the workgroup index rather than a
// per-lane division, and no access is predicated beyond the row's last
// vector. In the 28-layer, batch-256 decode chain on MI355X, with 256-lane
// workgroups, this measured 2-4 us per step below the flat form above.
struct SwigluRowArgs {
    const void* g;
    const void* u;
    void* out;
    int64_t g_stride, u_stride, out_stride;  // elements
    uint32_t vpr;                            // vectors per row
    FastDiv wpr;                             // workgroups per row
};
constexpr int kSwigluRowBlock = 256;

template <typename T, typename Act>
__global__ __launch_bounds__(kSwigluRowBlock) void swiglu_rows_kernel(const SwigluRowArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec;
    const uint32_t b = blockIdx.x;
    const uint32_t row = fastdiv(b, a.wpr);
    const uint32_t v = (b - row * a.wpr.d) * kSwigluRowBlock + threadIdx.x;
    if (v >= a.vpr) return;
    const int e = (int)v * kVec;
    const u32x4 gv = ld16_nt<T>(static_cast<const S*>(a.g) + (int64_t)row * a.g_stride, e);
    const u32x4 uv = ld16_nt<T>(static_cast<const S*>(a.u) + (int64_t)row * a.u_stride, e);
    float gf[kVec], uf[kVec], of[kVec];
    unpack<T>(gv, gf);
    unpack<T>(uv, uf);
#pragma unroll
    for (int i = 0; i < kVec; ++i) of[i] = Act::apply(gf[i], uf[i]);
    st16_nt<T>(static_cast<S*>(a.out) + (int64_t)row * a.out_stride, e, pack<T>(of));
}

template <typename T, typename C, typename Act>
static int launch_swiglu(const SwigluArgs& a, void* stream, bool vec) {
    const dim3 grid((uint32_t)(((int64_t)a.total + C::BLOCK * C::UNROLL - 1) / (C::BLOCK * C::UNROLL)));
    // fp32 rows are always dword aligned: only 2-byte types need element access.
    if constexpr (sizeof(typename T::storage) == 4)
        return launch(swiglu_kernel<T, C, Act, true>, grid, dim3(C::BLOCK), stream, a);
    else
        return vec ? launch(swiglu_kernel<T, C, Act, true>, grid, dim3(C::BLOCK), stream, a)
                   : launch(swiglu_kernel<T, C, Act, false>, grid, dim3(C::BLOCK), stream, a);
}

// Shared argument checks of the gated activations.
static int gated_prepare(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
                         void* out, int64_t out_stride, int64_t rows, int64_t cols, int dtype,
                         SwigluArgs* a, bool* work) {
    *work = false;
    if (!dtype_ok(dtype)) return KCR_ERR_DTYPE;
    if (rows < 0 || cols < 1) return KCR_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const int vec = (int)(16 / es);
    const int64_t vpr = (cols + vec - 1) / vec;
    if (rows * vpr >= (int64_t(1) << 31)) return KCR_ERR_SHAPE;
    if (rows == 0) return KCR_OK;
    if (!gate || !up || !out) return KCR_ERR_NULL;
    if (gate_stride < cols || up_stride < cols || out_stride < cols) return KCR_ERR_SHAPE;
    if (!aligned_elem(gate, es) || !aligned_elem(up, es) || !aligned_elem(out, es))
        return KCR_ERR_ALIGN;
    // The output may be one of the inputs itself (same pointer and stride);
    // otherwise it must share no element with either input.
    const bool on_gate = out == gate && out_stride == gate_stride;
    const bool on_up = out == up && out_stride == up_stride;
    if ((!on_gate && !rows_disjoint(out, out_stride, gate, gate_stride, rows, cols, es)) ||
        (!on_up && !rows_disjoint(out, out_stride, up, up_stride, rows, cols, es)))
        return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;
    *a = SwigluArgs{gate, up, out, gate_stride, up_stride, out_stride, cols,
                    (uint32_t)(rows * vpr), make_fastdiv((uint32_t)vpr)};
    *work = true;
    return KCR_OK;
}

// 64-lane workgroups, one vector of each stream per lane, one-pass grid,
// nontemporal loads and stores: the fastest shape in sweeps on MI355X.
// Calls that stream at most kGatedSmallBytes (decode batches) take 128-lane
// workgroups, which measured 2.5 us faster per step in the 28-layer,
// batch-256 decode chain (half as many workgroups to dispatch per launch).
using GatedCfg = SwigluCfg<64, 1, true, true>;
using GatedSmallCfg = SwigluCfg<128, 1, true, true>;
constexpr int64_t kGatedSmallBytes = 32ll << 20;

template <typename Act>
static int run_gated(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
                     void* out, int64_t out_stride, int64_t rows, int64_t cols, int dtype,
                     void* stream) {
    SwigluArgs a;
    bool work;
    const int rc = gated_prepare(gate, gate_stride, up, up_stride, out, out_stride, rows, cols, dtype,
                                 &a, &work);
    if (rc != KCR_OK || !work) return rc;
    const size_t es = dtype_size(dtype);
    auto rows_ok = [es](const void* p, int64_t stride) { return vec_ok(p) && (stride * (int64_t)es) % 4 == 0; };
    const bool vec = rows_ok(gate, gate_stride) && rows_ok(up, up_stride) && rows_ok(out, out_stride);
    const bool small = 3 * rows * cols * (int64_t)es <= kGatedSmallBytes;
    const int64_t vpr = a.vpr.d, wpr = (vpr + kSwigluRowBlock - 1) / kSwigluRowBlock;
    if (small && vec && cols % (int64_t)(16 / es) == 0 && rows * wpr < (int64_t(1) << 23)) {
        const SwigluRowArgs r{gate, up, out, gate_stride, up_stride, out_stride, (uint32_t)vpr,
                              make_fastdiv((uint32_t)wpr)};
        const dim3 grid((uint32_t)(rows * wpr)), block(kSwigluRowBlock);
        return by_dtype(dtype, [&](auto t) {
            return launch(swiglu_rows_kernel<decltype(t), Act>, grid, block, stream, r);
        });
    }
    return by_dtype(dtype, [&](auto t) {
        return small ? launch_swiglu<decltype(t), GatedSmallCfg, Act>(a, stream, vec)
                     : launch_swiglu<decltype(t), GatedCfg, Act>(a, stream, vec);
    });
}

}  // namespace kcr

using namespace kcr;

extern "C" int kcr_swiglu(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
                          void* out, int64_t out_stride, int64_t rows, int64_t cols, int dtype,
                          void* stream) {
    return run_gated<SiluMul>(gate, gate_stride, up, up_stride, out, out_stride, rows, cols, dtype,
                              stream);
}

extern "C" int kcr_reglu(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
                         void* out, int64_t out_stride, int64_t rows, int64_t cols, int dtype,
                         void* stream) {
    return run_gated<ReluMul>(gate, gate_stride, up, up_stride, out, out_stride, rows, cols, dtype,
                              stream);
}

// norm.h -- the interface between the RMSNorm entry points (rmsnorm.hip)
// and the row-norm engine (norm_engine.h), which is compiled once per
// storage type and variant in its own translation unit (norm_inst.hip).
#pragma once

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

// Runs the row-norm engine over `a` on `stream`: y = rmsnorm(x) (ADD =
// false) or x <- round(x + delta), y = rmsnorm(x) (ADD = true). Defined in
// norm_engine.h, instantiated in norm_inst.hip for T in {Bf16, F16, F32}.
template <typename T, bool ADD>
int run_norm(const NormArgs& a, void* stream);

// Widest row of the register-resident engine, in 16-byte vectors (8 waves
// of 64 lanes, 8 vectors per lane); wider rows take the two-pass kernel.
constexpr int kRegMaxVec = 8 * 64 * 8;

// Calls with at least this many rows may take a measured per-width shape
// (norm_engine.h, launch_tuned) instead of norm_shape's.
constexpr int64_t kTunedMinRows = 4096;

// Calls that stream at most this many bytes take one row group per
// workgroup (norm_engine.h, launch_small).
constexpr int64_t kNormSmallCallBytes = 32ll << 20;

// LDS bytes a workgroup may take on the current device.
size_t lds_per_block();

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

constexpr NormShape norm_shape(int64_t nvec, bool add) {
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

// The (vpt, wpr) pairs norm_shape returns for some width of up to kRegMaxVec
// vectors, with the groups it pairs them with (0: never returned). Evaluated
// at compile time, so the dispatch instantiates exactly these shapes.
struct RuleShapes {
    int8_t groups[9][9];
};

constexpr RuleShapes rule_shapes(bool add) {
    RuleShapes r{};
    for (int64_t n = 1; n <= kRegMaxVec; ++n) {
        const NormShape s = norm_shape(n, add);
        if (s.vpt >= 1 && s.vpt <= 8 && s.wpr >= 1 && s.wpr <= 8) r.groups[s.vpt][s.wpr] = (int8_t)s.groups;
    }
    return r;
}

template <bool ADD>
constexpr RuleShapes kRuleShapes = rule_shapes(ADD);


}  // namespace kcr

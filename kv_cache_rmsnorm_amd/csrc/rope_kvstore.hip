// rope_kvstore.hip -- rotate-half RoPE of Q and K fused with the paged
// KV-cache store of rotated K and V (kcr_rope_kvstore), and the device-side
// cos/sin table build (kcr_rope_cos_sin).
//
// The op is the fused kernel of the koas-w.github.io 2026-03-31 post,
// section 1 ("Fused RoPE & Paged KV Cache Store"): Q, K, V, cos and sin are
// read once, rotated in registers, Q goes back to contiguous memory and the
// rotated K and V go straight to the cache slots named by slot_mapping.
// Cache layout [2, num_blocks, block_size, kv_heads, head_dim] as in mer.dev
// "AsyncT vLLM notes (1)", section 1.1.
//
// gfx950 design
//  * Virtual heads: following the GQA mapping of the same section,
//    kv_head = head / (n_head / n_kv_head), KV group g is the query heads
//    g*G .. g*G+G-1 (G = n_head / n_kv_head, contiguous in memory), then K
//    head g, then V head g -- G + 2 heads of equal cost.
//  * LPU lanes per virtual head (the number of 16-byte chunks in half a
//    head, rounded up to a power of two: 8 for bf16 head_dim 128). Lane c
//    owns chunk c of the first half AND chunk c of the second half, so each
//    rotation pair (i, i + d/2) sits in one lane and needs no shuffle.
//  * One workgroup per token (rope_token_kernel) wherever half a head is a
//    power-of-two number of chunks and the token's heads fit 1024 lanes:
//    the token's position and slot are then scalar loads. Other head
//    layouts take the unit kernel (rope_kvstore_kernel): a unit is a run of
//    HPU consecutive virtual heads of one token (1 for decode batches, 2 for
//    prefill), so every unit does the same work and no lane idles on K/V.
//  * cos/sin for the lane's frequencies are loaded once per token or unit
//    (fp32 table rows, L2-resident across tokens); all heads are loaded
//    before any is stored. One-pass grid, nontemporal loads and stores of
//    the streamed heads.
//  * K_rot and V are written with 16-byte stores at
//    ((which * n_slots + slot) * n_kv_head + g) * head_dim: the cache's
//    (block, offset) pair flattens to the slot, so no division is needed.
//    V is moved as raw bits (bit-exact); Q and K go through fp32.
#include "kcr_device.h"
#include "kcr_host.h"

namespace kcr {

struct RopeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* q_out;
    void* cache;
    const int64_t* pos;
    const int64_t* slots;
    const float* cos_t;
    const float* sin_t;
    const void* q_w;  // qk-norm weights [dh] (QKN only)
    const void* k_w;
    float eps;
    int64_t q_ts, q_hs, k_ts, k_hs, v_ts, v_hs;  // elements
    int64_t max_pos, n_slots;
    uint32_t units;   // T * units per token
    FastDiv upt;      // units per token: ceil(n_virtual_heads / HPU)
    FastDiv gsize;    // virtual heads per KV group: G + 2
    int32_t nvh;      // virtual heads per token: n_kv_head * (G + 2)
    int32_t hq, hkv, group, dh;
};

// Launch shape: LPU lanes per unit (one 16-byte chunk of each half head per
// lane), HPU virtual heads per unit, nontemporal loads (NTL) and stores (NTS)
// for the streamed heads, BLOCK lanes per workgroup.
template <int LPU_, int HPU_, bool NTL_, bool NTS_, int BLOCK_ = 256>
struct RopeCfg {
    static constexpr int LPU = LPU_, HPU = HPU_, BLOCK = BLOCK_;
    static constexpr bool NTL = NTL_, NTS = NTS_;
};

// Virtual heads of a token, in KV-group order: for group g (kv_head g), the
// query heads g*G .. g*G+G-1 (exactly those with head / G == g), then K head
// g, then V head g. With QKN every Q and K head is first RMS-normalised with
// its weight (the qk-norm of the Q/K views of a fused QKV projection, mer.dev
// "AsyncT vLLM notes (1)", sections 0 and 3.3): the unit's lanes reduce the
// head's sum of squares with DPP, so all of them stay active (lanes past the
// head's last chunk read chunk 0 and count zero).
template <typename T, typename C, bool QKN>
__global__ __launch_bounds__(C::BLOCK) void rope_kvstore_kernel(const RopeArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec, LPU = C::LPU, HPU = C::HPU;
    constexpr int UPW = C::BLOCK / LPU;  // units per workgroup
    const int c = threadIdx.x % LPU;
    const int half = a.dh >> 1;
    const bool lane_on = c * kVec < half;
    if (!QKN && !lane_on) return;
    const int64_t c0 = lane_on ? (int64_t)c * kVec : 0;
    // One pass, no loop: unit u of the grid (a loop over several units per
    // lane measured slower on the row kernels).
    const uint32_t u = blockIdx.x * UPW + threadIdx.x / LPU;
    if (u >= a.units) return;  // all lanes of a unit leave together
    {
        const uint32_t t = fastdiv(u, a.upt);
        const int j0 = (int)(u - t * a.upt.d) * HPU;
        // Position and slot first, then every head of the unit: the head
        // loads do not depend on the position, so they are in flight while
        // the position arrives and only the (L2-resident) cos/sin rows wait
        // for it.
        const int64_t p = a.pos[t];
        const int64_t slot = a.slots[t];
        // Loads are unconditional (a head index past the token's last head
        // is clamped to it and its result discarded), and the q/k/v choice is
        // made with selects, so no branch merge forces an early wait.
        u32x4 x1[HPU], x2[HPU];
        int kind[HPU];  // 0: query head, 1: K, 2: V, -1: past the token's heads
        int gg[HPU], hh[HPU];
#pragma unroll
        for (int h = 0; h < HPU; ++h) {
            const int j = j0 + h;
            const int jc = j < a.nvh ? j : a.nvh - 1;
            const int g = (int)fastdiv((uint32_t)jc, a.gsize);
            const int r = jc - g * (int)a.gsize.d;
            const bool isq = r < a.group, isk = r == a.group;
            kind[h] = j < a.nvh ? (isq ? 0 : (isk ? 1 : 2)) : -1;
            hh[h] = g * a.group + r;
            gg[h] = g;
            const S* base = static_cast<const S*>(isq ? a.q : (isk ? a.k : a.v));
            const int64_t ts = isq ? a.q_ts : (isk ? a.k_ts : a.v_ts);
            const int64_t hs = isq ? a.q_hs : (isk ? a.k_hs : a.v_hs);
            const S* src = base + t * ts + (int64_t)(isq ? hh[h] : g) * hs;
            x1[h] = C::NTL ? ld16_nt<T>(src, c0) : ld16<T>(src, c0);
            x2[h] = C::NTL ? ld16_nt<T>(src, half + c0) : ld16<T>(src, half + c0);
        }
        // Compiler-only barrier: keeps the head loads issued here, ahead of
        // the position-dependent branches below (emits no instruction).
        asm volatile("" ::: "memory");
        // A token whose position is out of range writes its query heads
        // unrotated and nothing to the cache; its table row is clamped to
        // row 0 and never used. Keeping the query store unconditional also
        // keeps the head loads ahead of the wait for the position.
        const bool p_ok = p >= 0 && p < a.max_pos;
        const int64_t pc = p_ok ? p : 0;
        const bool store_kv = p_ok && slot >= 0 && slot < a.n_slots;

        float wq1[kVec], wq2[kVec], wk1[kVec], wk2[kVec];
        if constexpr (QKN) {
            unpack<T>(ld16<T>(a.q_w, c0), wq1);
            unpack<T>(ld16<T>(a.q_w, half + c0), wq2);
            unpack<T>(ld16<T>(a.k_w, c0), wk1);
            unpack<T>(ld16<T>(a.k_w, half + c0), wk2);
        }

        float cs[kVec], sn[kVec];
        {
            const float* cr = a.cos_t + pc * half + c0;
            const float* sr = a.sin_t + pc * half + c0;
#pragma unroll
            for (int i = 0; i < kVec; i += 4) {
                u32x4 cv = *reinterpret_cast<const u32x4*>(cr + i);
                u32x4 sv = *reinterpret_cast<const u32x4*>(sr + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cs[i + e] = __uint_as_float(cv[e]);
                    sn[i + e] = __uint_as_float(sv[e]);
                }
            }
        }

#pragma unroll
        for (int h = 0; h < HPU; ++h) {
            if (kind[h] < 0) continue;
            // Q and K rotate; V (and Q at an out-of-range position) is copied
            // as is, selected so that its bits pass through untouched.
            float f1[kVec], f2[kVec], r1[kVec], r2[kVec];
            unpack<T>(x1[h], f1);
            unpack<T>(x2[h], f2);
            if constexpr (QKN) {
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < kVec; ++e) ss += f1[e] * f1[e] + f2[e] * f2[e];
                ss = group_sum<LPU>(lane_on ? ss : 0.0f);
                const float r = __builtin_amdgcn_rsqf(ss * inv_width(a.dh) + a.eps);
                const bool isk = kind[h] == 1;
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    f1[e] = f1[e] * r * (isk ? wk1[e] : wq1[e]);
                    f2[e] = f2[e] * r * (isk ? wk2[e] : wq2[e]);
                }
            }
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                r1[e] = f1[e] * cs[e] - f2[e] * sn[e];
                r2[e] = f2[e] * cs[e] + f1[e] * sn[e];
            }
            const u32x4 p1 = pack<T>(r1), p2 = pack<T>(r2);
            const bool rot = kind[h] < 2 && p_ok;
            const u32x4 o1 = rot ? p1 : x1[h], o2 = rot ? p2 : x2[h];
            if (!lane_on || (kind[h] != 0 && !store_kv)) continue;
            S* dst = kind[h] == 0
                         ? static_cast<S*>(a.q_out) + ((int64_t)t * a.hq + hh[h]) * a.dh
                         : static_cast<S*>(a.cache) +
                               (((int64_t)(kind[h] - 1) * a.n_slots + slot) * a.hkv + gg[h]) * (int64_t)a.dh;
            if (C::NTS) {
                st16_nt<T>(dst, c0, o1);
                st16_nt<T>(dst, half + c0, o2);
            } else {
                st16<T>(dst, c0, o1);
                st16<T>(dst, half + c0, o2);
            }
        }
    }
}

// One workgroup per UPW units. A grid holds at most 2^32 - 1 work-items, so
// a call with more tokens than that covers is split into launches over
// consecutive token ranges (q, k, v, q_out, positions and slots offset).
template <typename T, typename C, bool QKN>
static int launch_rope(RopeArgs a, int64_t T_tokens, void* stream) {
    using S = typename T::storage;
    constexpr int UPW = C::BLOCK / C::LPU;
    const int64_t upt = (a.nvh + C::HPU - 1) / C::HPU;
    a.upt = make_fastdiv((uint32_t)upt);
    const int64_t max_tokens = ((int64_t)0xFFFFFFFFu / C::BLOCK) * UPW / upt;
    for (int64_t t0 = 0; t0 < T_tokens; t0 += max_tokens) {
        RopeArgs c = a;
        const int64_t n = T_tokens - t0 < max_tokens ? T_tokens - t0 : max_tokens;
        c.q = static_cast<const S*>(a.q) + t0 * a.q_ts;
        c.k = static_cast<const S*>(a.k) + t0 * a.k_ts;
        c.v = static_cast<const S*>(a.v) + t0 * a.v_ts;
        c.q_out = static_cast<S*>(a.q_out) + t0 * (int64_t)a.hq * a.dh;
        c.pos = a.pos + t0;
        c.slots = a.slots + t0;
        c.units = (uint32_t)(n * upt);
        const dim3 grid((uint32_t)((c.units + UPW - 1) / UPW));
        const int rc = launch(rope_kvstore_kernel<T, C, QKN>, grid, dim3(C::BLOCK), stream, c);
        if (rc != KCR_OK) return rc;
    }
    return KCR_OK;
}

template <typename T, int HPU, bool QKN, int BLOCK>
static int dispatch_rope_lpu(const RopeArgs& a, int64_t T_tokens, void* stream) {
    const int chunks = (a.dh / 2) / T::kVec;
    if (chunks <= 1) return launch_rope<T, RopeCfg<1, HPU, true, true, BLOCK>, QKN>(a, T_tokens, stream);
    if (chunks <= 2) return launch_rope<T, RopeCfg<2, HPU, true, true, BLOCK>, QKN>(a, T_tokens, stream);
    if (chunks <= 4) return launch_rope<T, RopeCfg<4, HPU, true, true, BLOCK>, QKN>(a, T_tokens, stream);
    if (chunks <= 8) return launch_rope<T, RopeCfg<8, HPU, true, true, BLOCK>, QKN>(a, T_tokens, stream);
    if (chunks <= 16) return launch_rope<T, RopeCfg<16, HPU, true, true, BLOCK>, QKN>(a, T_tokens, stream);
    if (chunks <= 32) return launch_rope<T, RopeCfg<32, HPU, true, true, BLOCK>, QKN>(a, T_tokens, stream);
    // 64 chunks of half a head: only fp32 reaches it under KCR_ROPE_MAX_HEAD_DIM.
    if constexpr (T::kVec * 64 * 2 <= KCR_ROPE_MAX_HEAD_DIM) {
        if (chunks <= 64) return launch_rope<T, RopeCfg<64, HPU, true, true, BLOCK>, QKN>(a, T_tokens, stream);
    }
    return KCR_ERR_SHAPE;
}

// Decode batches: one workgroup per token, LPU = the chunks of half a head
// (a power of two), lanes u * LPU .. u * LPU + LPU - 1 on virtual head u in
// KV-group order. The token index is the workgroup index, so its position
// and slot are scalar loads and every lane's addresses follow from the
// lane number alone; lanes past the token's last head (the workgroup is a
// whole number of waves) repeat its last head and store nothing. Straight-
// line code with no early exit: in the 28-layer, batch-256 decode chain on
// MI355X this took the step 5-7 us below the unit kernel above at the same
// work split.
//
// DH: head_dim when fixed at compile time (0: a.dh). FUSED: q, k and v are
// head ranges of one row per token -- k = q + n_head heads, v = k +
// n_kv_head heads, one token stride and one head stride -- the layout of a
// fused QKV projection's output (mer.dev "AsyncT vLLM notes (1)", section
// 3.3), so every lane reads from one base pointer. Both only shorten the
// address arithmetic ahead of the first load: together 4-5 us per step of
// the 28-layer, batch-256 decode chain on MI355X.
template <typename T, int LPU, bool QKN, int DH = 0, bool FUSED = false>
__global__ __launch_bounds__(1024) void rope_token_kernel(const RopeArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec;
    const int tid = threadIdx.x, c = tid % LPU, u0 = tid / LPU;
    const bool on = u0 < a.nvh;
    const int u = on ? u0 : a.nvh - 1;
    const int dh = DH ? DH : a.dh;
    const int half = dh >> 1;
    const int64_t t = blockIdx.x;
    const int g = (int)fastdiv((uint32_t)u, a.gsize);
    const int r = u - g * (int)a.gsize.d;
    const int kind = r < a.group ? 0 : (r == a.group ? 1 : 2);  // query, K, V
    const int hh = g * a.group + r;
    const S* src;
    if constexpr (FUSED) {
        const int head = kind == 0 ? hh : (kind == 1 ? a.hq + g : a.hq + a.hkv + g);
        src = static_cast<const S*>(a.q) + t * a.q_ts + (int64_t)head * a.q_hs;
    } else {
        const S* base = static_cast<const S*>(kind == 0 ? a.q : (kind == 1 ? a.k : a.v));
        const int64_t ts = kind == 0 ? a.q_ts : (kind == 1 ? a.k_ts : a.v_ts);
        const int64_t hs = kind == 0 ? a.q_hs : (kind == 1 ? a.k_hs : a.v_hs);
        src = base + t * ts + (int64_t)(kind == 0 ? hh : g) * hs;
    }
    const int64_t p = a.pos[t], slot = a.slots[t];
    const int c0 = c * kVec;
    const u32x4 x1 = ld16_nt<T>(src, c0), x2 = ld16_nt<T>(src, half + c0);
    // The head loads stay ahead of everything that waits for the position:
    // no memory access moves across (the compiler barrier) and no
    // instruction either (the scheduling barrier; without it the scheduler
    // hoisted the position checks above the head loads, which then waited
    // for the position's scalar load).
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    float w1[kVec], w2[kVec];
    if constexpr (QKN) {
        const void* wp = kind == 1 ? a.k_w : a.q_w;
        unpack<T>(ld16<T>(wp, c0), w1);
        unpack<T>(ld16<T>(wp, half + c0), w2);
    }
    const bool p_ok = p >= 0 && p < a.max_pos;
    const int64_t pc = p_ok ? p : 0;
    const float* cr = a.cos_t + pc * half + c0;
    const float* sr = a.sin_t + pc * half + c0;
    float cs[kVec], sn[kVec];
#pragma unroll
    for (int i = 0; i < kVec; i += 4) {
        const u32x4 cv = *reinterpret_cast<const u32x4*>(cr + i);
        const u32x4 sv = *reinterpret_cast<const u32x4*>(sr + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            cs[i + e] = __uint_as_float(cv[e]);
            sn[i + e] = __uint_as_float(sv[e]);
        }
    }
    float f1[kVec], f2[kVec], r1[kVec], r2[kVec];
    unpack<T>(x1, f1);
    unpack<T>(x2, f2);
    if constexpr (QKN) {
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < kVec; ++e) ss += f1[e] * f1[e] + f2[e] * f2[e];
        ss = group_sum<LPU>(ss);
        const float rs = __builtin_amdgcn_rsqf(ss * inv_width(dh) + a.eps);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            f1[e] = f1[e] * rs * w1[e];
            f2[e] = f2[e] * rs * w2[e];
        }
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        r1[e] = f1[e] * cs[e] - f2[e] * sn[e];
        r2[e] = f2[e] * cs[e] + f1[e] * sn[e];
    }
    // Q and K rotate; V (and Q at an out-of-range position) keep their bits.
    const bool rot = kind < 2 && p_ok;
    const u32x4 o1 = rot ? pack<T>(r1) : x1, o2 = rot ? pack<T>(r2) : x2;
    const bool store_kv = p_ok && slot >= 0 && slot < a.n_slots;
    S* dst = kind == 0 ? static_cast<S*>(a.q_out) + (t * a.hq + hh) * dh
                       : static_cast<S*>(a.cache) +
                             (((int64_t)(kind - 1) * a.n_slots + (store_kv ? slot : 0)) * a.hkv + g) * (int64_t)dh;
    if (on && (kind == 0 || store_kv)) {
        st16_nt<T>(dst, c0, o1);
        st16_nt<T>(dst, half + c0, o2);
    }
}

// One workgroup per token when half a head is a power-of-two number of
// chunks and the token's virtual heads fit one workgroup; returns 1 when the
// call does not qualify.
template <typename T, bool QKN>
static int launch_rope_token(const RopeArgs& a, int64_t T_tokens, void* stream) {
    const int chunks = (a.dh / 2) / T::kVec;
    const int lanes = a.nvh * chunks;
    if ((chunks & (chunks - 1)) != 0 || lanes > 1024) return 1;
    const int64_t block_lanes = (lanes + 63) / 64 * 64;
    if (T_tokens * block_lanes > (int64_t)0xFFFFFFFFu) return 1;  // one grid: under 2^32 work-items
    const dim3 grid((uint32_t)T_tokens), block((uint32_t)block_lanes);
    using S = typename T::storage;
    const bool fused = a.k == static_cast<const S*>(a.q) + (int64_t)a.hq * a.q_hs &&
                       a.v == static_cast<const S*>(a.k) + (int64_t)a.hkv * a.q_hs && a.k_ts == a.q_ts &&
                       a.v_ts == a.q_ts && a.k_hs == a.q_hs && a.v_hs == a.q_hs;
    if (a.dh == 128) {
        constexpr int L = 64 / T::kVec;
        return fused ? launch(rope_token_kernel<T, L, QKN, 128, true>, grid, block, stream, a)
                     : launch(rope_token_kernel<T, L, QKN, 128, false>, grid, block, stream, a);
    }
    // Every other power-of-two chunk count up to KCR_ROPE_MAX_HEAD_DIM (the
    // count of head_dim 128 took the fixed-size form above).
    auto generic = [&](auto lpu) -> int {
        constexpr int L = decltype(lpu)::value;
        if constexpr (L == 64 / T::kVec || T::kVec * L * 2 > KCR_ROPE_MAX_HEAD_DIM) return 1;
        else return launch(rope_token_kernel<T, L, QKN>, grid, block, stream, a);
    };
    switch (chunks) {
        case 1: return generic(std::integral_constant<int, 1>{});
        case 2: return generic(std::integral_constant<int, 2>{});
        case 4: return generic(std::integral_constant<int, 4>{});
        case 8: return generic(std::integral_constant<int, 8>{});
        case 16: return generic(std::integral_constant<int, 16>{});
        case 32: return generic(std::integral_constant<int, 32>{});
        case 64: return generic(std::integral_constant<int, 64>{});
    }
    return 1;
}

// Decode batches (up to 4096 tokens): one virtual head per unit spreads the
// work over the most workgroups, and 128-lane workgroups measured 2.8 us
// faster per step than 256-lane ones in the 28-layer, batch-256 decode chain
// on MI355X. Prefill-sized batches take two heads per unit, which reuses
// each cos/sin load once, in 256-lane workgroups (64 and 128 lanes measured
// the same there). Stores stay nontemporal at every size: cached stores of
// q_out and the cache rows made the decode chain 28 us slower per step
// (each kernel then writes its dirty L2 lines back before the next starts).
constexpr int64_t kRopeSmallBatch = 4096;

// Every call whose token fits one workgroup takes the token kernel: in the
// decode chain it measured 5-7 us per step below the unit kernel, and at the
// 64-sequence prefill shape (70k tokens) 0.5-1.3% above the two-head unit
// kernel (96.0-96.5 against 97.0-97.3 us, two runs; with the Q/K norm the
// same). The unit kernels remain for head layouts the token kernel does not
// take (half a head not a power-of-two number of chunks, or more than 1024
// lanes of heads per token).
template <typename T, bool QKN>
static int dispatch_rope(const RopeArgs& a, int64_t T_tokens, void* stream) {
    const int rc = launch_rope_token<T, QKN>(a, T_tokens, stream);
    if (rc <= 0) return rc;
    return T_tokens <= kRopeSmallBatch ? dispatch_rope_lpu<T, 1, QKN, 128>(a, T_tokens, stream)
                                       : dispatch_rope_lpu<T, 2, QKN, 256>(a, T_tokens, stream);
}

// ---------------------------------------------------------- cos/sin tables
struct TableArgs {
    float* cos_t;
    float* sin_t;
    int64_t n;  // max_pos * half
    int32_t half, head_dim;
    double theta;
};

// cos/sin(p * theta^(-2i/d)) in fp64, rounded once to fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(const TableArgs a) {
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < a.n;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t p = idx / a.half;
        const int i = (int)(idx - p * a.half);
        const double ang = (double)p * pow(a.theta, -2.0 * (double)i / (double)a.head_dim);
        a.cos_t[idx] = (float)cos(ang);
        a.sin_t[idx] = (float)sin(ang);
    }
}

}  // namespace kcr

using namespace kcr;

// Validates the arguments shared by the two RoPE + store entry points and
// fills the kernel arguments; KCR_OK with *work == false means nothing to do.
static int rope_prepare(const void* q, int64_t q_tok_stride, int64_t q_head_stride, const void* k,
                        int64_t k_tok_stride, int64_t k_head_stride, const void* v,
                        int64_t v_tok_stride, int64_t v_head_stride, void* q_out,
                        const int64_t* positions, const float* cos_tab, const float* sin_tab,
                        int64_t max_pos, void* kv_cache, const int64_t* slot_mapping, int64_t T,
                        int n_head, int n_kv_head, int head_dim, int block_size, int64_t num_blocks,
                        int dtype, RopeArgs* out, bool* work) {
    *work = false;
    if (!dtype_ok(dtype)) return KCR_ERR_DTYPE;
    if (n_kv_head < 1 || n_head < 1) return KCR_ERR_SHAPE;
    if (n_head % n_kv_head != 0) return KCR_ERR_HEADS;
    const size_t es = dtype_size(dtype);
    const int vec = (int)(16 / es);
    if (head_dim < 2 || head_dim % 2 != 0 || (head_dim / 2) % vec != 0 ||
        head_dim > KCR_ROPE_MAX_HEAD_DIM)
        return KCR_ERR_SHAPE;
    if (T < 0 || block_size < 1 || num_blocks < 0 || max_pos < 1) return KCR_ERR_SHAPE;
    if (T * (int64_t)n_kv_head * (n_head / n_kv_head + 2) >= (int64_t(1) << 31)) return KCR_ERR_SHAPE;
    if (T == 0) return KCR_OK;
    if (!q || !k || !v || !q_out || !positions || !cos_tab || !sin_tab || !slot_mapping)
        return KCR_ERR_NULL;
    if (!kv_cache && num_blocks > 0) return KCR_ERR_NULL;
    if (q_head_stride < head_dim || k_head_stride < head_dim || v_head_stride < head_dim ||
        q_tok_stride < 0 || k_tok_stride < 0 || v_tok_stride < 0)
        return KCR_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_out) ||
        !aligned16(cos_tab) || !aligned16(sin_tab) || (kv_cache && !aligned16(kv_cache)) ||
        !stride_ok(q_tok_stride, es) || !stride_ok(q_head_stride, es) ||
        !stride_ok(k_tok_stride, es) || !stride_ok(k_head_stride, es) ||
        !stride_ok(v_tok_stride, es) || !stride_ok(v_head_stride, es) ||
        (reinterpret_cast<uintptr_t>(positions) & 7u) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
        return KCR_ERR_ALIGN;

    const int64_t n_slots = num_blocks * (int64_t)block_size;
    const Span sq = span3d(q, T, q_tok_stride, n_head, q_head_stride, head_dim, es);
    const Span sk = span3d(k, T, k_tok_stride, n_kv_head, k_head_stride, head_dim, es);
    const Span sv = span3d(v, T, v_tok_stride, n_kv_head, v_head_stride, head_dim, es);
    const Span so = span2d(q_out, 1, 0, T * n_head * (int64_t)head_dim, es);
    const Span sc = span2d(kv_cache, 1, 0, 2 * n_slots * n_kv_head * (int64_t)head_dim, es);
    const Span st = span2d(cos_tab, 1, 0, max_pos * (head_dim / 2), 4);
    const Span ss = span2d(sin_tab, 1, 0, max_pos * (head_dim / 2), 4);
    const Span sp = span2d(positions, 1, 0, T, 8), sl = span2d(slot_mapping, 1, 0, T, 8);
    const bool q_contig = q_head_stride == head_dim && q_tok_stride == (int64_t)n_head * head_dim;
    const bool in_place = q == q_out && q_contig;
    if ((!in_place && overlap(so, sq)) || overlap(so, sk) || overlap(so, sv) || overlap(so, sc) ||
        overlap(so, st) || overlap(so, ss) || overlap(so, sp) || overlap(so, sl) || overlap(sc, sq) ||
        overlap(sc, sk) || overlap(sc, sv) || overlap(sc, st) || overlap(sc, ss) || overlap(sc, sp) ||
        overlap(sc, sl))
        return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;

    const int group = n_head / n_kv_head;
    *out = RopeArgs{q, k, v, q_out, kv_cache, positions, slot_mapping, cos_tab, sin_tab,
                    nullptr, nullptr, 0.0f,
                    q_tok_stride, q_head_stride, k_tok_stride, k_head_stride, v_tok_stride, v_head_stride,
                    max_pos, n_slots, 0u, make_fastdiv(1u), make_fastdiv((uint32_t)(group + 2)),
                    n_kv_head * (group + 2), n_head, n_kv_head, group, head_dim};
    *work = true;
    return KCR_OK;
}

extern "C" int kcr_rope_kvstore(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                                const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                                const void* v, int64_t v_tok_stride, int64_t v_head_stride,
                                void* q_out, const int64_t* positions, const float* cos_tab,
                                const float* sin_tab, int64_t max_pos, void* kv_cache,
                                const int64_t* slot_mapping, int64_t T, int n_head, int n_kv_head,
                                int head_dim, int block_size, int64_t num_blocks, int dtype,
                                void* stream) {
    RopeArgs a;
    bool work;
    const int rc = rope_prepare(q, q_tok_stride, q_head_stride, k, k_tok_stride, k_head_stride, v,
                                v_tok_stride, v_head_stride, q_out, positions, cos_tab, sin_tab,
                                max_pos, kv_cache, slot_mapping, T, n_head, n_kv_head, head_dim,
                                block_size, num_blocks, dtype, &a, &work);
    if (rc != KCR_OK || !work) return rc;
    return by_dtype(dtype, [&](auto t) { return dispatch_rope<decltype(t), false>(a, T, stream); });
}

extern "C" int kcr_qknorm_rope_kvstore(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                                       const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                                       const void* v, int64_t v_tok_stride, int64_t v_head_stride,
                                       const void* q_norm_w, const void* k_norm_w, float eps,
                                       void* q_out, const int64_t* positions, const float* cos_tab,
                                       const float* sin_tab, int64_t max_pos, void* kv_cache,
                                       const int64_t* slot_mapping, int64_t T, int n_head,
                                       int n_kv_head, int head_dim, int block_size,
                                       int64_t num_blocks, int dtype, void* stream) {
    RopeArgs a;
    bool work;
    const int rc = rope_prepare(q, q_tok_stride, q_head_stride, k, k_tok_stride, k_head_stride, v,
                                v_tok_stride, v_head_stride, q_out, positions, cos_tab, sin_tab,
                                max_pos, kv_cache, slot_mapping, T, n_head, n_kv_head, head_dim,
                                block_size, num_blocks, dtype, &a, &work);
    if (rc != KCR_OK || !work) return rc;
    if (!q_norm_w || !k_norm_w) return KCR_ERR_NULL;
    if (!aligned16(q_norm_w) || !aligned16(k_norm_w)) return KCR_ERR_ALIGN;
    const size_t es = dtype_size(dtype);
    const Span so = span2d(q_out, 1, 0, T * n_head * (int64_t)head_dim, es);
    const Span sc = span2d(kv_cache, 1, 0, 2 * a.n_slots * n_kv_head * (int64_t)head_dim, es);
    const Span wq = span2d(q_norm_w, 1, 0, head_dim, es), wk = span2d(k_norm_w, 1, 0, head_dim, es);
    if (overlap(so, wq) || overlap(so, wk) || overlap(sc, wq) || overlap(sc, wk)) return KCR_ERR_ALIAS;
    a.q_w = q_norm_w;
    a.k_w = k_norm_w;
    a.eps = eps;
    return by_dtype(dtype, [&](auto t) { return dispatch_rope<decltype(t), true>(a, T, stream); });
}

extern "C" int kcr_rope_cos_sin(float* cos_tab, float* sin_tab, int64_t max_pos, int head_dim,
                                double theta, void* stream) {
    if (max_pos < 0 || head_dim < 2 || head_dim % 2 != 0 || !(theta > 0.0)) return KCR_ERR_SHAPE;
    if (max_pos == 0) return KCR_OK;
    if (!cos_tab || !sin_tab) return KCR_ERR_NULL;
    if (!aligned16(cos_tab) || !aligned16(sin_tab)) return KCR_ERR_ALIGN;
    const int half = head_dim / 2;
    const int64_t n = max_pos * half;
    if (overlap(span2d(cos_tab, 1, 0, n, 4), span2d(sin_tab, 1, 0, n, 4))) return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;
    const TableArgs a{cos_tab, sin_tab, n, half, head_dim, theta};
    return launch(rope_table_kernel, dim3(grid_for(n, 256, device_cus(), 8)), dim3(256), stream, a);
}

// The host form of the same tables: one fp64 angle per (position,
// frequency), its cos and sin each rounded once to fp32.
extern "C" int kcr_rope_cos_sin_host(float* cos_tab, float* sin_tab, int64_t max_pos, int head_dim,
                                     double theta) {
    if (max_pos < 0 || head_dim < 2 || head_dim % 2 != 0 || !(theta > 0.0)) return KCR_ERR_SHAPE;
    if (max_pos == 0) return KCR_OK;
    if (!cos_tab || !sin_tab) return KCR_ERR_NULL;
    const int half = head_dim / 2;
    const int64_t n = max_pos * half;
    if (overlap(span2d(cos_tab, 1, 0, n, 4), span2d(sin_tab, 1, 0, n, 4))) return KCR_ERR_ALIAS;
    for (int i = 0; i < half; ++i) {
        const double inv_freq = pow(theta, -2.0 * (double)i / (double)head_dim);
        for (int64_t p = 0; p < max_pos; ++p) {
            const double ang = (double)p * inv_freq;
            cos_tab[p * half + i] = (float)cos(ang);
            sin_tab[p * half + i] = (float)sin(ang);
        }
    }
    return KCR_OK;
}

// decode_chain.hip -- the per-layer chain of one decode step in a single
// launch (kcr_decode_chain_batch, and kcr_decode_chain_b1 for one token):
// for every layer, in order, residual add + RMSNorm (the koas-w.github.io
// 2026-03-31 post, section 4), RoPE + paged store (section 1), residual
// add + RMSNorm, SwiGLU (section 2).
//
// gfx950 design
//  * Only the residual carries a dependency from op to op: each add reads
//    the h the previous one wrote. RoPE and SwiGLU read only the layer's own
//    inputs, which nothing in the chain writes. So one launch holds three
//    kinds of 256-lane workgroup, chosen by workgroup index: one per token
//    runs the token's residual chain (2 add+norms per layer, h in registers,
//    the next layers' deltas and weights in flight); per token, workgroups
//    of query heads and of key/value heads run every layer's RoPE and store
//    in layer order; and one per (layer, token, 256 vectors) runs a SwiGLU
//    chunk. The step's time is then that of the residual chain at small
//    batches and that of the stream of bytes at large ones, instead of the
//    sum of every op of every layer on one workgroup per token.
//  * Workgroups never wait for one another, and only the residual
//    workgroups use barriers: one per layer, for the sums of squares of the
//    layer's two rows across their 4 waves (no norm needs another's result,
//    only the adds chain, so the adds come first), or one per pair of layers
//    in the deep form at one vector per lane.
//  * Each role's layer loop is software-pipelined: the inputs of the next
//    PD (residual) or PDR (RoPE) layers are loaded before the current layer
//    computes, in a ring of register sets; a scheduling barrier between
//    layers keeps each layer's arithmetic waiting on its own inputs only.
//    Batches up to 64 tokens take deeper rings (the residual chain's
//    latency bounds the step); larger batches shallower ones, since the
//    kernel's register count sets how many SwiGLU waves a CU holds.
//  * The per-layer pointer table travels in the argument block; the
//    looping roles read it into the scalar cache at their start.
//  * RoPE lane mapping as in rope_kvstore.hip: LPU lanes per head, lane c
//    owning chunk c of both halves.
#include <algorithm>

#include "kcr_device.h"
#include "kcr_host.h"

namespace kcr {

// Shape limits of the entry points (vectors of 16 bytes): hidden <= 1024,
// inter <= 4096, and the token's virtual heads (query, key and value heads,
// each head_dim/2 elements wide in units of LPU lanes) <= 1024 lanes.
constexpr int kChainMaxHiddenVec = 1024;
constexpr int kChainMaxInterVec = 4096;
constexpr int kChainMaxRopeLanes = 1024;
// Lanes per workgroup, for every role.
constexpr int kFlowThreads = 256;
// The residual role holds ceil(hidden vectors / 256) vectors per lane.
constexpr int kFlowMaxHpl = kChainMaxHiddenVec / kFlowThreads;
// Batches up to this size take the deeply prefetched form (the residual
// chain's latency bounds the step); larger ones the lean form (the SwiGLU
// stream's occupancy does).
constexpr int64_t kFlowDeepMaxBatch = 64;
// SwiGLU workgroups in one grid; beyond this many chunks each loops.
constexpr int64_t kFlowMaxSwigluGroups = int64_t(1) << 22;
// Tokens per launch: the grid (batch * (1 + query and key/value groups)
// plus the SwiGLU groups) times 256 lanes stays below 2^32.
constexpr int64_t kChainMaxBatch = (int64_t(1) << 20) - 1;

struct ChainArgs {
    kcr_chain_layer layers[KCR_B1_MAX_LAYERS];
    void* h;  // [batch, hidden]; token b's rows of every per-token tensor at b * width
    const int64_t* pos;
    const int64_t* slots;
    const float* cos_t;
    const float* sin_t;
    int64_t max_pos, n_slots;
    int32_t n_layers, hidden, inter, hq, hkv, dh, group, lpu;
    int64_t qkv_w;  // (hq + 2 hkv) * dh
    float eps;
    // grid layout: [0, batch) residual groups, then batch * (n_rq + n_rkv)
    // RoPE groups, then s_groups SwiGLU groups covering s_total chunks
    int64_t batch, s_total, s_groups;
    int32_t n_rq, n_rkv, n_s;
};

// The argument-block warm-up in the kernel relies on this entry layout.
static_assert(sizeof(kcr_chain_layer) == 88 && offsetof(kcr_chain_layer, kv_cache) == 40 &&
                  offsetof(kcr_chain_layer, act) == 80,
              "kcr_chain_layer: 11 pointers");

// The layer table sits in the kernel's argument block and each layer's
// pointers are first read at that layer's start, where a scalar-cache miss
// stalls the wave. Bring the whole table into the scalar cache: the fields
// read here (bytes 0, 40 and 80 of each 88-byte, 8-byte-aligned entry) leave
// no gap of 64 bytes, so every 64-byte line of the table holds one of them.
// The block always holds KCR_B1_MAX_LAYERS entries (unused ones zero), so
// every read is in bounds.
__device__ __forceinline__ void warm_layer_table(const ChainArgs& a) {
    uintptr_t acc = 0;
#pragma unroll
    for (int l = 0; l < KCR_B1_MAX_LAYERS; ++l) {
        const kcr_chain_layer& E = a.layers[l];
        acc |= reinterpret_cast<uintptr_t>(E.d_attn) | reinterpret_cast<uintptr_t>(E.kv_cache) |
               reinterpret_cast<uintptr_t>(E.act);
    }
    asm volatile("" ::"s"(acc));
}

// Ends one layer of a role's software pipeline: no memory access moves
// across (the compiler barrier) and no instruction at all (the scheduling
// barrier), so each layer's arithmetic waits only for its own inputs, which
// were loaded PD layers earlier.
__device__ __forceinline__ void layer_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The chain in one launch as three kinds of workgroup, picked by the
// workgroup index. Only the residual depends on the previous op; RoPE and
// SwiGLU read nothing the chain writes. So the residual chain (the step's
// one dependency chain) runs in one workgroup per token, and every layer's
// RoPE and SwiGLU run beside it, all at once.
//  * Residual (one per token): h in registers for the whole step, lane l
//    owning vectors l, l + 256, ...; per layer the two add+norms, storing
//    y_attn and y_mlp; h itself is stored once, at the end (a caller sees
//    only the final residual: every buffer that could observe an earlier
//    one is refused as an overlap). The inputs of the next PD layers are in
//    flight at all times.
//  * RoPE (per token, n_rq groups of query heads, then n_rkv of key and
//    value heads): every layer in order, the next PDR layers' q/k/v chunks
//    in flight. A token's cache rows are written by the same lanes layer
//    after layer, so with layers that share a cache the last layer's rows
//    remain.
//  * SwiGLU (per layer, token and chunk of 256 vectors).
template <typename T, int HPL, bool DEEP>
__global__ __launch_bounds__(kFlowThreads) void decode_chain_kernel(const ChainArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec;
    constexpr int kWaves = kFlowThreads / 64;
    // layers in flight: the residual's inputs take 16 VGPRs per layer and
    // vector per lane, so PD is 4 (deep) or 2 (lean) divided by the vectors
    // per lane, and at least 1
    constexpr int PD = (DEEP ? 4 : 2) / HPL > 1 ? (DEEP ? 4 : 2) / HPL : 1;
    constexpr int PDR = DEEP ? 4 : 2;
    __shared__ float4 part[2][kWaves];  // per wave: sums of squares of up to four rows
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int n = a.n_layers;
    const int64_t bid = blockIdx.x;
    const int64_t nR = a.batch * (a.n_rq + a.n_rkv);

    if (bid < a.batch) {
        // ------------------------------------------------------ residual
        const int64_t hrow = bid * a.hidden;
        const int hv = a.hidden / kVec;
        const float inv_h = inv_width(a.hidden);
        S* const h = static_cast<S*>(a.h) + hrow;
        bool own[HPL], won[HPL];
        int64_t ec[HPL];  // in-bounds element offset for every lane
        float hf[HPL][kVec];  // the residual, each value exactly its stored rounding
#pragma unroll
        for (int k = 0; k < HPL; ++k) {
            const int v = tid + k * kFlowThreads;
            own[k] = v < hv;
            ec[k] = own[k] ? (int64_t)v * kVec : 0;
            unpack<T>(ld16<T>(h, ec[k]), hf[k]);
            // whether this wave owns any of slot k (uniform: a scalar branch)
            won[k] = __builtin_amdgcn_readfirstlane((int)(wave * 64 + k * kFlowThreads < hv)) != 0;
        }
        struct Set {
            u32x4 dA[HPL], wA[HPL], dM[HPL], wM[HPL];
        };
        Set s[PD];
        auto load = [&](Set& st, int l) {
            const kcr_chain_layer& L = a.layers[l];
#pragma unroll
            for (int k = 0; k < HPL; ++k) {
                st.dA[k] = ld16_nt<T>(static_cast<const S*>(L.d_attn) + hrow, ec[k]);
                st.wA[k] = ld16<T>(L.w_attn, ec[k]);
                st.dM[k] = ld16_nt<T>(static_cast<const S*>(L.d_mlp) + hrow, ec[k]);
                st.wM[k] = ld16<T>(L.w_mlp, ec[k]);
            }
        };
#pragma unroll
        for (int j = 0; j < PD; ++j) load(s[j], j < n ? j : n - 1);
        warm_layer_table(a);
        layer_fence();
        // One layer: h <- round(h + d_attn), y_attn = rmsnorm(h) * w_attn,
        // h <- round(h + d_mlp), y_mlp = rmsnorm(h) * w_mlp. The second add
        // needs only the first add's h, not its norm, so both adds come
        // first and the two rows' sums of squares cross the waves in one
        // exchange (one barrier per layer, two alternating slots).
        auto layer = [&](Set& st, int l) {
            const kcr_chain_layer& L = a.layers[l];
            S* const y_attn = static_cast<S*>(L.y_attn) + hrow;
            S* const y_mlp = static_cast<S*>(L.y_mlp) + hrow;
            u32x4 xr[2][HPL];  // the rounded sums, packed
            float ss[2] = {0.0f, 0.0f};
#pragma unroll
            for (int nn = 0; nn < 2; ++nn) {
#pragma unroll
                for (int k = 0; k < HPL; ++k) {
                    if (won[k]) {
                        float df[kVec];
                        unpack<T>(nn == 0 ? st.dA[k] : st.dM[k], df);
#pragma unroll
                        for (int e = 0; e < kVec; ++e) hf[k][e] += df[e];
                        xr[nn][k] = pack<T>(hf[k]);
                        unpack<T>(xr[nn][k], hf[k]);  // the rounded sum is what the norm sees
                        float sk = 0.0f;
#pragma unroll
                        for (int e = 0; e < kVec; ++e) sk = __builtin_fmaf(hf[k][e], hf[k][e], sk);
                        ss[nn] += own[k] ? sk : 0.0f;
                    }
                }
            }
            // each wave's two sums, whole in lane 63
            const float w0 = wave_total_lane63(ss[0]), w1 = wave_total_lane63(ss[1]);
            const int slot = l & 1;
            if (lane == 63) part[slot][wave] = make_float4(w0, w1, 0.0f, 0.0f);
            __syncthreads();
            float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) {
                const float4 v = part[slot][i];
                t0 += v.x;
                t1 += v.y;
            }
            const float rs0 = __builtin_amdgcn_rsqf(t0 * inv_h + a.eps);
            const float rs1 = __builtin_amdgcn_rsqf(t1 * inv_h + a.eps);
#pragma unroll
            for (int nn = 0; nn < 2; ++nn) {
#pragma unroll
                for (int k = 0; k < HPL; ++k) {
                    if (won[k]) {
                        float xf[kVec], wf[kVec], yf[kVec];
                        unpack<T>(xr[nn][k], xf);
                        unpack<T>(nn == 0 ? st.wA[k] : st.wM[k], wf);
                        const float rs = nn == 0 ? rs0 : rs1;
#pragma unroll
                        for (int e = 0; e < kVec; ++e) yf[e] = xf[e] * rs * wf[e];
                        const u32x4 yv = pack<T>(yf);
                        if (own[k]) st16_nt<T>(nn == 0 ? y_attn : y_mlp, ec[k], yv);
                    }
                }
            }
        };
        if constexpr (DEEP && HPL == 1) {
            // Pairs of layers share one exchange (four sums per wave), and the
            // ring holds two pairs, so a pair's inputs were loaded a whole
            // pair earlier. One pair: layers l0 and l0 + 1 from sets base and
            // base + 1. The last n % 4 layers go one at a time, as below (a
            // pair with a run-time layer count made the compiler copy the
            // whole argument block to scratch memory: LLVM folds away its
            // private copy of a by-value kernel argument only while that
            // copy has at most a few hundred users, and the larger unrolled
            // forms pass that count).
            static_assert(PD == 4, "two pairs of layers in flight");
            auto pair = [&](auto base_c, int l0, int slot) {
                constexpr int base = decltype(base_c)::value;
                // [layer][norm]: the rounded sums, unpacked (kept rather than
                // unpacked again for the norms: the residual chain is bound by
                // instruction issue)
                float xs[2][2][kVec];
                float ss[4];
                // Every wave does the adds, also one that owns no vector of the
                // row (its lanes sit on vector 0 and add zero to the sums): a
                // branch around them cost the other waves register moves at
                // the merge, about a tenth of the loop's instructions.
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    ss[2 * j] = 0.0f;
                    ss[2 * j + 1] = 0.0f;
#pragma unroll
                    for (int nn = 0; nn < 2; ++nn) {
                        float df[kVec];
                        unpack<T>(nn == 0 ? s[base + j].dA[0] : s[base + j].dM[0], df);
#pragma unroll
                        for (int e = 0; e < kVec; ++e) hf[0][e] += df[e];
                        unpack<T>(pack<T>(hf[0]), hf[0]);
#pragma unroll
                        for (int e = 0; e < kVec; ++e) xs[j][nn][e] = hf[0][e];
                        float sk = 0.0f;
#pragma unroll
                        for (int e = 0; e < kVec; ++e) sk = __builtin_fmaf(hf[0][e], hf[0][e], sk);
                        ss[2 * j + nn] = own[0] ? sk : 0.0f;
                    }
                }
                const float4 w4 = make_float4(wave_total_lane63(ss[0]), wave_total_lane63(ss[1]),
                                              wave_total_lane63(ss[2]), wave_total_lane63(ss[3]));
                if (lane == 63) part[slot][wave] = w4;
                __syncthreads();
                float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int i = 0; i < kWaves; ++i) {
                    const float4 v = part[slot][i];
                    t[0] += v.x;
                    t[1] += v.y;
                    t[2] += v.z;
                    t[3] += v.w;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (won[0]) {
                        const kcr_chain_layer& L = a.layers[l0 + j];
                        S* const y_attn = static_cast<S*>(L.y_attn) + hrow;
                        S* const y_mlp = static_cast<S*>(L.y_mlp) + hrow;
#pragma unroll
                        for (int nn = 0; nn < 2; ++nn) {
                            const float rs = __builtin_amdgcn_rsqf(t[2 * j + nn] * inv_h + a.eps);
                            float wf[kVec], yf[kVec];
                            unpack<T>(nn == 0 ? s[base + j].wA[0] : s[base + j].wM[0], wf);
#pragma unroll
                            for (int e = 0; e < kVec; ++e) yf[e] = xs[j][nn][e] * rs * wf[e];
                            const u32x4 yv = pack<T>(yf);
                            if (own[0]) st16_nt<T>(nn == 0 ? y_attn : y_mlp, ec[0], yv);
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) load(s[base + j], l0 + j + PD < n ? l0 + j + PD : n - 1);
                layer_fence();
            };
            int l = 0;
            for (; l + PD <= n; l += PD) {
                pair(std::integral_constant<int, 0>{}, l, 0);
                pair(std::integral_constant<int, 2>{}, l + 2, 1);
            }
            // (each exchange still alternates slots: l is even here)
#pragma unroll
            for (int j = 0; j < PD - 1; ++j)
                if (l + j < n) layer(s[j], l + j);
        } else {
            // whole groups of PD layers, then the rest (each set already
            // holds its layer)
            int l = 0;
            for (; l + PD <= n; l += PD) {
#pragma unroll
                for (int j = 0; j < PD; ++j) {
                    layer(s[j], l + j);
                    load(s[j], l + j + PD < n ? l + j + PD : n - 1);
                    layer_fence();
                }
            }
#pragma unroll
            for (int j = 0; j < PD - 1; ++j)
                if (l + j < n) layer(s[j], l + j);
        }
#pragma unroll
        for (int k = 0; k < HPL; ++k)
            if (own[k]) st16_nt<T>(h, ec[k], pack<T>(hf[k]));
        return;
    }

    if (bid < a.batch + nR) {
        // ------------------------------------------------------ RoPE
        // No barriers in this role: lanes without work leave at once.
        const int64_t r = bid - a.batch;
        const int per_tok = a.n_rq + a.n_rkv;
        // uniform by construction; said so, so that no index into the
        // argument block becomes a per-lane one (the block would then be
        // copied to scratch to be indexed)
        const int64_t tok = __builtin_amdgcn_readfirstlane((int)(r / per_tok));
        const int chunk = __builtin_amdgcn_readfirstlane((int)(r - tok * per_tok));
        const bool is_q = chunk < a.n_rq;  // uniform
        const int half = a.dh >> 1;
        // unit = head: query heads, or key heads [0, hkv) then value heads
        const int unit = (is_q ? chunk : chunk - a.n_rq) * (kFlowThreads / a.lpu) + tid / a.lpu;
        const int c = tid % a.lpu;  // lane c owns chunk c of both halves
        if (unit >= (is_q ? a.hq : 2 * a.hkv) || c * kVec >= half) return;
        const int64_t p = a.pos[tok];
        const int64_t slot = a.slots[tok];
        const bool p_ok = p >= 0 && p < a.max_pos;
        const bool store_kv = p_ok && slot >= 0 && slot < a.n_slots;
        if (!is_q && !store_kv) return;
        const bool is_v = !is_q && unit >= a.hkv;
        const int g = is_v ? unit - a.hkv : unit;  // KV head of a key or value unit
        const int src_head = is_q ? unit : a.hq + unit;
        const int64_t c0 = (int64_t)c * kVec;
        // query and key heads rotate at a valid position; value heads and
        // query heads at an invalid one are copied
        const bool rot = p_ok && !is_v;
        const int64_t dst_off = is_q ? tok * (int64_t)a.hq * a.dh + (int64_t)unit * a.dh
                                     : (((int64_t)(is_v ? 1 : 0) * a.n_slots + slot) * a.hkv + g) * (int64_t)a.dh;
        float cs[kVec], sn[kVec];
        {
            const float* cr = a.cos_t + (p_ok ? p : 0) * half + c0;
            const float* sr = a.sin_t + (p_ok ? p : 0) * half + c0;
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
        }
        struct Set {
            u32x4 x1, x2;
        };
        Set s[PDR];
        auto load = [&](Set& st, int l) {
            const S* src = static_cast<const S*>(a.layers[l].qkv) + tok * a.qkv_w + (int64_t)src_head * a.dh;
            st.x1 = ld16_nt<T>(src, c0);
            st.x2 = ld16_nt<T>(src, half + c0);
        };
        // (the table rows first: the loop's first wait covers them alone)
#pragma unroll
        for (int j = 0; j < PDR; ++j) load(s[j], j < n ? j : n - 1);
        warm_layer_table(a);
        layer_fence();
        auto layer = [&](Set& st, int l) {
            const kcr_chain_layer& L = a.layers[l];
            float f1[kVec], f2[kVec], r1[kVec], r2[kVec];
            unpack<T>(st.x1, f1);
            unpack<T>(st.x2, f2);
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                r1[e] = __builtin_fmaf(f1[e], cs[e], -(f2[e] * sn[e]));
                r2[e] = __builtin_fmaf(f2[e], cs[e], f1[e] * sn[e]);
            }
            const u32x4 p1 = pack<T>(r1), p2 = pack<T>(r2);
            u32x4 o1, o2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o1[i] = rot ? p1[i] : st.x1[i];
                o2[i] = rot ? p2[i] : st.x2[i];
            }
            // the destination's base pointer is uniform (is_q is): a scalar load
            S* const dst = static_cast<S*>(is_q ? L.q_out : L.kv_cache) + dst_off;
            st16_nt<T>(dst, c0, o1);
            st16_nt<T>(dst, half + c0, o2);
        };
        int l = 0;
        for (; l + PDR <= n; l += PDR) {
#pragma unroll
            for (int j = 0; j < PDR; ++j) {
                layer(s[j], l + j);
                load(s[j], l + j + PDR < n ? l + j + PDR : n - 1);
                layer_fence();
            }
        }
#pragma unroll
        for (int j = 0; j < PDR - 1; ++j)
            if (l + j < n) layer(s[j], l + j);
        return;
    }

    // ---------------------------------------------------------- SwiGLU
    // chunk index = (layer * batch + token) * n_s + chunk of 256 vectors
    const int iv = a.inter / kVec;
    for (int64_t sx = bid - a.batch - nR; sx < a.s_total; sx += a.s_groups) {
        // (all uniform, and said so: see the RoPE role)
        const int64_t row = sx / a.n_s;  // layer * batch + token
        const int chunk = __builtin_amdgcn_readfirstlane((int)(sx - row * a.n_s));
        const int l = __builtin_amdgcn_readfirstlane((int)(row / a.batch));
        const int64_t tok = __builtin_amdgcn_readfirstlane((int)(row - (int64_t)l * a.batch));
        const kcr_chain_layer& L = a.layers[l];
        const int v = chunk * kFlowThreads + tid;
        const int64_t e = v < iv ? (int64_t)v * kVec : 0;
        const S* const gate_up = static_cast<const S*>(L.gate_up) + tok * 2 * (int64_t)a.inter;
        const u32x4 gv = ld16_nt<T>(gate_up, e);
        const u32x4 uv = ld16_nt<T>(gate_up, (int64_t)a.inter + e);
        if (v < iv) {
            float gf[kVec], uf[kVec], of[kVec];
            unpack<T>(gv, gf);
            unpack<T>(uv, uf);
#pragma unroll
            for (int i = 0; i < kVec; ++i) {
                const float ex = __builtin_amdgcn_exp2f(gf[i] * -1.4426950408889634f);
                of[i] = gf[i] * __builtin_amdgcn_rcpf(1.0f + ex) * uf[i];
            }
            st16_nt<T>(static_cast<S*>(L.act) + tok * (int64_t)a.inter, (int64_t)v * kVec, pack<T>(of));
        }
    }
}

template <typename T, bool DEEP>
static int launch_chain_t(const ChainArgs& a, int hpl, void* stream) {
    const int64_t groups = a.batch * (1 + a.n_rq + a.n_rkv) + a.s_groups;
    const dim3 grid((uint32_t)groups), block(kFlowThreads);
    switch (hpl) {
        case 1: return launch(decode_chain_kernel<T, 1, DEEP>, grid, block, stream, a);
        case 2: return launch(decode_chain_kernel<T, 2, DEEP>, grid, block, stream, a);
        case 3: return launch(decode_chain_kernel<T, 3, DEEP>, grid, block, stream, a);
        default: return launch(decode_chain_kernel<T, kFlowMaxHpl, DEEP>, grid, block, stream, a);
    }
}

// Completes the grid layout in `a` and launches.
template <typename T>
static int launch_chain(ChainArgs& a, void* stream) {
    constexpr int kVec = T::kVec;
    const int hpl = (a.hidden / kVec + kFlowThreads - 1) / kFlowThreads;
    const int per_group = kFlowThreads / a.lpu;  // heads per RoPE workgroup
    a.n_rq = (a.hq + per_group - 1) / per_group;
    a.n_rkv = (2 * a.hkv + per_group - 1) / per_group;
    a.n_s = (a.inter / kVec + kFlowThreads - 1) / kFlowThreads;
    a.s_total = (int64_t)a.n_layers * a.batch * a.n_s;
    a.s_groups = std::min(a.s_total, kFlowMaxSwigluGroups);
    return a.batch <= kFlowDeepMaxBatch ? launch_chain_t<T, true>(a, hpl, stream)
                                        : launch_chain_t<T, false>(a, hpl, stream);
}

// One per-layer buffer of a chain call: its byte range, its layer, its
// role (the order of the span lists in kcr_decode_chain_batch: d_attn,
// w_attn, qkv, d_mlp, w_mlp, gate_up, then y_attn, q_out, kv_cache, y_mlp,
// act) and whether the chain writes it.
struct LayerSpan {
    Span s;
    int layer, role;
    bool written;
};
constexpr int kLayerInputs = 6, kLayerBufs = 11, kRoleCache = 8;

// Cross-layer rule of the one-launch chain: each layer's inputs are read
// ahead of the previous layer's ops, so a buffer one layer writes may not
// overlap any buffer of another layer. Inputs may be shared (e.g. one
// weight for several layers), and so may a cache, when the layers name the
// same cache range: the chain never reads the cache, and each token's cache
// rows are written by the same lanes layer after layer, so the last layer's
// rows land there, as with the separate calls. Overlaps within a layer are
// checked by the caller. Sort-and-sweep over the ranges, O(n log n) plus the
// overlapping pairs.
static bool layers_disjoint(LayerSpan* v, int n) {
    std::sort(v, v + n, [](const LayerSpan& x, const LayerSpan& y) { return x.s.lo < y.s.lo; });
    for (int i = 0; i < n; ++i) {
        if (v[i].s.lo == v[i].s.hi) continue;
        for (int j = i + 1; j < n && v[j].s.lo < v[i].s.hi; ++j) {
            if (v[j].s.lo == v[j].s.hi || v[i].layer == v[j].layer) continue;
            if (!v[i].written && !v[j].written) continue;
            const bool same_cache = v[i].role == kRoleCache && v[j].role == kRoleCache &&
                                    v[i].s.lo == v[j].s.lo && v[i].s.hi == v[j].s.hi;
            if (!same_cache) return false;
        }
    }
    return true;
}

}  // namespace kcr

using namespace kcr;

extern "C" int kcr_decode_chain_batch(const kcr_chain_layer* layers, int n_layers, int64_t batch, void* h,
                                      int hidden, int inter, int n_head, int n_kv_head, int head_dim,
                                      const int64_t* positions, const int64_t* slot_mapping,
                                      const float* cos_tab, const float* sin_tab, int64_t max_pos,
                                      int block_size, int64_t num_blocks, float eps, int dtype,
                                      void* stream) {
    if (!dtype_ok(dtype)) return KCR_ERR_DTYPE;
    if (n_layers < 0 || n_layers > KCR_B1_MAX_LAYERS) return KCR_ERR_SHAPE;
    if (batch < 0 || batch > kChainMaxBatch) return KCR_ERR_SHAPE;
    if (n_kv_head < 1 || n_head < 1) return KCR_ERR_SHAPE;
    if (n_head % n_kv_head != 0) return KCR_ERR_HEADS;
    const size_t es = dtype_size(dtype);
    const int vec = (int)(16 / es);
    if (hidden < 1 || hidden % vec != 0 || hidden / vec > kChainMaxHiddenVec) return KCR_ERR_SHAPE;
    if (inter < 1 || inter % vec != 0 || inter / vec > kChainMaxInterVec) return KCR_ERR_SHAPE;
    if (head_dim < 2 || head_dim % 2 != 0 || (head_dim / 2) % vec != 0 || head_dim > KCR_ROPE_MAX_HEAD_DIM)
        return KCR_ERR_SHAPE;
    if (block_size < 1 || num_blocks < 0 || max_pos < 1) return KCR_ERR_SHAPE;
    const int group = n_head / n_kv_head;
    int lpu = 1;
    while (lpu * vec < head_dim / 2) lpu *= 2;
    if ((int64_t)n_kv_head * (group + 2) * lpu > kChainMaxRopeLanes) return KCR_ERR_SHAPE;
    if (n_layers == 0 || batch == 0) return KCR_OK;
    if (!layers || !h || !positions || !slot_mapping || !cos_tab || !sin_tab) return KCR_ERR_NULL;
    if (!aligned16(h) || !aligned16(cos_tab) || !aligned16(sin_tab) ||
        (reinterpret_cast<uintptr_t>(positions) & 7u) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
        return KCR_ERR_ALIGN;

    const int64_t n_slots = num_blocks * (int64_t)block_size;
    const int64_t qkv_elems = (int64_t)(n_head + 2 * n_kv_head) * head_dim;
    const int64_t B = batch;
    const Span sh = span2d(h, B, hidden, hidden, es);
    const Span st = span2d(cos_tab, 1, 0, max_pos * (head_dim / 2), 4);
    const Span ss = span2d(sin_tab, 1, 0, max_pos * (head_dim / 2), 4);
    const Span sp = span2d(positions, 1, 0, B, 8), sm = span2d(slot_mapping, 1, 0, B, 8);
    ChainArgs a{};
    // Every layer's buffers, for the cross-layer check below.
    LayerSpan all[KCR_B1_MAX_LAYERS * kLayerBufs];
    int n_all = 0;
    for (int l = 0; l < n_layers; ++l) {
        const kcr_chain_layer& L = layers[l];
        const void* ptrs[] = {L.d_attn, L.w_attn, L.y_attn, L.qkv, L.q_out, L.d_mlp, L.w_mlp, L.y_mlp,
                              L.gate_up, L.act};
        for (const void* p : ptrs) {
            if (!p) return KCR_ERR_NULL;
            if (!aligned16(p)) return KCR_ERR_ALIGN;
        }
        if (!L.kv_cache && n_slots > 0) return KCR_ERR_NULL;
        if (L.kv_cache && !aligned16(L.kv_cache)) return KCR_ERR_ALIGN;
        const Span in[] = {span2d(L.d_attn, B, hidden, hidden, es), span2d(L.w_attn, 1, 0, hidden, es),
                           span2d(L.qkv, B, qkv_elems, qkv_elems, es), span2d(L.d_mlp, B, hidden, hidden, es),
                           span2d(L.w_mlp, 1, 0, hidden, es),
                           span2d(L.gate_up, B, 2 * (int64_t)inter, 2 * (int64_t)inter, es),
                           st, ss, sp, sm};
        // h is read and written: it may overlap neither an input nor an output.
        const Span out[] = {sh, span2d(L.y_attn, B, hidden, hidden, es),
                            span2d(L.q_out, B, (int64_t)n_head * head_dim, (int64_t)n_head * head_dim, es),
                            span2d(L.kv_cache, 1, 0, 2 * n_slots * n_kv_head * (int64_t)head_dim, es),
                            span2d(L.y_mlp, B, hidden, hidden, es), span2d(L.act, B, inter, inter, es)};
        constexpr int n_in = sizeof(in) / sizeof(in[0]), n_out = sizeof(out) / sizeof(out[0]);
        for (int i = 0; i < n_out; ++i) {
            for (int j = 0; j < n_in; ++j)
                if (overlap(out[i], in[j])) return KCR_ERR_ALIAS;
            for (int j = i + 1; j < n_out; ++j)
                if (overlap(out[i], out[j])) return KCR_ERR_ALIAS;
        }
        const Span mine[kLayerBufs] = {in[0], in[1], in[2], in[3], in[4], in[5],
                                       out[1], out[2], out[3], out[4], out[5]};
        for (int i = 0; i < kLayerBufs; ++i)
            all[n_all++] = LayerSpan{mine[i], l, i, i >= kLayerInputs};
        a.layers[l] = L;
    }
    if (!layers_disjoint(all, n_all)) return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;
    a.h = h;
    a.pos = positions;
    a.slots = slot_mapping;
    a.cos_t = cos_tab;
    a.sin_t = sin_tab;
    a.max_pos = max_pos;
    a.n_slots = n_slots;
    a.n_layers = n_layers;
    a.hidden = hidden;
    a.inter = inter;
    a.hq = n_head;
    a.hkv = n_kv_head;
    a.dh = head_dim;
    a.group = group;
    a.lpu = lpu;
    a.eps = eps;
    a.qkv_w = qkv_elems;
    a.batch = batch;
    return by_dtype(dtype, [&](auto t) { return launch_chain<decltype(t)>(a, stream); });
}

extern "C" int kcr_decode_chain_b1(const kcr_chain_layer* layers, int n_layers, void* h, int hidden,
                                   int inter, int n_head, int n_kv_head, int head_dim,
                                   const int64_t* positions, const int64_t* slot_mapping,
                                   const float* cos_tab, const float* sin_tab, int64_t max_pos,
                                   int block_size, int64_t num_blocks, float eps, int dtype,
                                   void* stream) {
    return kcr_decode_chain_batch(layers, n_layers, 1, h, hidden, inter, n_head, n_kv_head, head_dim,
                                  positions, slot_mapping, cos_tab, sin_tab, max_pos, block_size,
                                  num_blocks, eps, dtype, stream);
}

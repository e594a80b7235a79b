// decode_chain.hip -- the per-layer chain of one decode step in a single
// launch (kcr_decode_chain_batch, and kcr_decode_chain_b1 for one token):
// for every layer, in order, residual add + RMSNorm (the koas-w.github.io
// 2026-03-31 post, section 4), RoPE + paged store (section 1), residual
// add + RMSNorm, SwiGLU (section 2).
//
// gfx950 design
//  * One workgroup per token (512 lanes where the token's row, RoPE units
//    and SwiGLU vectors fit, else 1024) runs every op of every layer in
//    turn; ops are separated by workgroup barriers only, so the 4 launches
//    per layer of the separate entry points (and their graph-node or host
//    launch cost) become one launch per step. Every op of the chain is
//    row-wise (a token's outputs depend on that token's inputs alone), so
//    the tokens' workgroups never wait for one another: no device-wide
//    barrier is needed at any batch size. A batch of 256 fills the 256 CUs
//    with one workgroup each.
//  * The residual h lives in registers for the whole step: lane l owns
//    16-byte vector l of the row, adds delta to it, stores the rounded sum
//    (the in-place update of each add) and normalises it. The row's sum of
//    squares is reduced in-wave with DPP, then across the waves through
//    two alternating LDS slot arrays (one barrier per norm).
//  * Loads are software-pipelined by half layers. The MLP half's inputs
//    (delta, weight, the gate/up vectors) are issued together before the
//    layer's first op; the attention half's (delta, weight, the token's
//    q/k/v chunks) one layer ahead, as soon as the previous layer's RoPE has
//    consumed its own. Each half's loads are therefore in flight while the
//    other half computes, in the registers the layer already holds. The
//    cos/sin rows of the token's position are the same for every layer and
//    are read once.
//  * The per-layer pointer table travels in the argument block; it is read
//    into the scalar cache at kernel start, so no layer's start waits on a
//    scalar-cache miss for its pointers.
//  * RoPE lane mapping as in rope_kvstore.hip: a unit of LPU lanes per
//    virtual head in KV-group order, lane c owning chunk c of both halves.
#include <algorithm>

#include "kcr_device.h"
#include "kcr_host.h"

namespace kcr {

// Lanes per token: 1024 at most (the shape limits below), 512 where the
// row, the RoPE units and the SwiGLU fit (fewer waves per barrier; measured
// faster at every batch).
constexpr int kChainThreads = 1024;
constexpr int kChainSmallThreads = 512;
constexpr int kChainMaxSwigluIters = 4;  // inter <= 4096 vectors at 1024 lanes
// Tokens per launch: batch * 1024 lanes must stay below 2^32.
constexpr int64_t kChainMaxBatch = (int64_t(1) << 22) - 1;

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
};

// The argument-block warm-up in the kernel relies on this entry layout.
static_assert(sizeof(kcr_chain_layer) == 88 && offsetof(kcr_chain_layer, kv_cache) == 40 &&
                  offsetof(kcr_chain_layer, act) == 80,
              "kcr_chain_layer: 11 pointers");

// Sum over the workgroup's lanes, every lane gets the result. `slot`
// alternates between the two norms of a layer: a lane rewrites slot s only
// after passing the barrier of the other slot, which every lane reaches
// after its last read of slot s.
template <int WAVES>
__device__ __forceinline__ float block_sum(float v, float (*part)[WAVES], int slot, int wave, int lane) {
    v = wave_sum(v);
    if (lane == 0) part[slot][wave] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) t += part[slot][i];
    return t;
}

template <typename T, int SWI, int THREADS>
__global__ __launch_bounds__(THREADS) void decode_chain_kernel(const ChainArgs a) {
    using S = typename T::storage;
    constexpr int kVec = T::kVec;
    constexpr int kWaves = THREADS / 64;
    __shared__ float part[2][kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    // This workgroup's token and its row offsets (uniform).
    const int64_t tok = blockIdx.x;
    const int64_t hrow = tok * a.hidden;

    // residual: lane tid owns vector tid of the token's row of h
    const int hv = a.hidden / kVec;
    const bool own_h = tid < hv;
    const int64_t he = (int64_t)tid * kVec;
    const int64_t he_c = own_h ? he : 0;  // in-bounds load address for every lane
    S* const h = static_cast<S*>(a.h) + hrow;
    u32x4 hreg = ld16<T>(h, he_c);

    // RoPE: unit = virtual head (KV-group order), lane c = chunk c of both halves
    const int half = a.dh >> 1;
    const int unit = tid / a.lpu, c = tid % a.lpu;
    const int nvh = a.hkv * (a.group + 2);
    const bool rope_on = unit < nvh && c * kVec < half;
    const int g = rope_on ? unit / (a.group + 2) : 0;
    const int r = rope_on ? unit - g * (a.group + 2) : 0;
    const int kind = r < a.group ? 0 : (r == a.group ? 1 : 2);  // query, K, V
    const int src_head = kind == 0 ? g * a.group + r : (kind == 1 ? a.hq + g : a.hq + a.hkv + g);
    const int64_t c0 = rope_on ? (int64_t)c * kVec : 0;
    const int64_t p = a.pos[tok];
    const int64_t slot = a.slots[tok];
    const bool p_ok = p >= 0 && p < a.max_pos;
    const bool store_kv = p_ok && slot >= 0 && slot < a.n_slots;
    float cs[kVec], sn[kVec];
    if (rope_on) {
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
    const int iv = a.inter / kVec;

    // The attention half's inputs of layer l (delta, weight, the token's
    // q/k/v chunks). They are loaded one layer ahead: layer l + 1's are
    // issued once layer l's RoPE has consumed its own, so they are in flight
    // during layer l's MLP half. Every load is unconditional: lanes with
    // nothing to load read an in-bounds clamped address and ignore the
    // result. In straight-line code the compiler waits for exactly the loads
    // each op needs; loads under lane-dependent branches made it wait for all
    // of them, and for earlier stores, before every op.
    u32x4 dA, wA, x1, x2;
    auto load_attn = [&](int l) {
        const kcr_chain_layer& L = a.layers[l];
        dA = ld16_nt<T>(static_cast<const S*>(L.d_attn) + hrow, he_c);
        wA = ld16<T>(L.w_attn, he_c);
        const S* src = static_cast<const S*>(L.qkv) + tok * a.qkv_w + (int64_t)src_head * a.dh;
        x1 = ld16_nt<T>(src, c0);
        x2 = ld16_nt<T>(src, half + c0);
    };
    load_attn(0);
    // The layer table sits in the kernel's argument block and each layer's
    // pointers are first read at that layer's start, where a scalar-cache
    // miss stalls every wave. Bring the whole table into the scalar cache
    // now, behind the first layer's loads: the fields read here (bytes 0,
    // 40 and 80 of each 88-byte, 8-byte-aligned entry) leave no gap of 64
    // bytes, so every 64-byte line of the table holds one of them. The
    // block always holds KCR_B1_MAX_LAYERS entries (unused ones zero), so
    // every read is in bounds.
    {
        uintptr_t acc = 0;
#pragma unroll
        for (int l = 0; l < KCR_B1_MAX_LAYERS; ++l) {
            const kcr_chain_layer& E = a.layers[l];
            acc |= reinterpret_cast<uintptr_t>(E.d_attn) | reinterpret_cast<uintptr_t>(E.kv_cache) |
                   reinterpret_cast<uintptr_t>(E.act);
        }
        asm volatile("" ::"s"(acc));
    }

    for (int l = 0; l < a.n_layers; ++l) {
        const kcr_chain_layer& L = a.layers[l];
        // The token's rows of the layer's per-token tensors (uniform).
        const S* const d_mlp = static_cast<const S*>(L.d_mlp) + hrow;
        const S* const gate_up = static_cast<const S*>(L.gate_up) + tok * 2 * (int64_t)a.inter;
        // The MLP half's inputs, issued together before the layer's first op.
        const u32x4 dM = ld16_nt<T>(d_mlp, he_c);
        const u32x4 wM = ld16<T>(L.w_mlp, he_c);
        u32x4 gr[SWI], ur[SWI];
#pragma unroll
        for (int k = 0; k < SWI; ++k) {
            const int v = tid + k * THREADS;
            const int64_t e = v < iv ? (int64_t)v * kVec : 0;
            gr[k] = ld16_nt<T>(gate_up, e);
            ur[k] = ld16_nt<T>(gate_up, (int64_t)a.inter + e);
        }
        // The layer's output pointers, read while the loads are in flight
        // (uniform; a per-lane choice between two fields of the argument
        // block would be a vector load that every later wait must cover).
        S* const q_out = static_cast<S*>(L.q_out) + tok * (int64_t)a.hq * a.dh;
        S* const kv_cache = static_cast<S*>(L.kv_cache);
        S* const y_attn = static_cast<S*>(L.y_attn) + hrow;
        S* const y_mlp = static_cast<S*>(L.y_mlp) + hrow;
        S* const act = static_cast<S*>(L.act) + tok * (int64_t)a.inter;
        // Compiler-only barrier: keeps every load above issued here, ahead of
        // the lane-dependent branches that use them (the compiler otherwise
        // sinks a load into its only user and then waits for all loads).
        asm volatile("" ::: "memory");

        // 1. h <- round(h + d_attn); y_attn = rmsnorm(h) * w_attn
        for (int n = 0; n < 2; ++n) {
            const u32x4 dv = n == 0 ? dA : dM;
            const u32x4 wv = n == 0 ? wA : wM;
            float ss = 0.0f;
            float xf[kVec];
            if (own_h) {
                float df[kVec];
                unpack<T>(hreg, xf);
                unpack<T>(dv, df);
#pragma unroll
                for (int e = 0; e < kVec; ++e) xf[e] += df[e];
                hreg = pack<T>(xf);
                st16_nt<T>(h, he, hreg);
                unpack<T>(hreg, xf);  // the rounded sum is what the norm sees
#pragma unroll
                for (int e = 0; e < kVec; ++e) ss += xf[e] * xf[e];
            }
            const float tot = block_sum<kWaves>(ss, part, n, wave, lane);
            if (own_h) {
                const float rs = __builtin_amdgcn_rsqf(tot / (float)a.hidden + a.eps);
                float wf[kVec], yf[kVec];
                unpack<T>(wv, wf);
#pragma unroll
                for (int e = 0; e < kVec; ++e) yf[e] = xf[e] * rs * wf[e];
                st16_nt<T>(n == 0 ? y_attn : y_mlp, he, pack<T>(yf));
            }
            if (n == 1) break;

            // 2. RoPE of the token's query and key heads, K_rot and V to the cache
            if (rope_on && (kind == 0 || store_kv)) {
                u32x4 o1 = x1, o2 = x2;
                if (kind < 2 && p_ok) {
                    float f1[kVec], f2[kVec], r1[kVec], r2[kVec];
                    unpack<T>(x1, f1);
                    unpack<T>(x2, f2);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        r1[e] = f1[e] * cs[e] - f2[e] * sn[e];
                        r2[e] = f2[e] * cs[e] + f1[e] * sn[e];
                    }
                    o1 = pack<T>(r1);
                    o2 = pack<T>(r2);
                }
                S* dst = kind == 0
                             ? q_out + (int64_t)src_head * a.dh
                             : kv_cache + (((int64_t)(kind - 1) * a.n_slots + slot) * a.hkv + g) * (int64_t)a.dh;
                st16_nt<T>(dst, c0, o1);
                st16_nt<T>(dst, half + c0, o2);
            }
            // The next layer's attention-half inputs (the last layer reads its
            // own again and ignores them).
            load_attn(l + 1 < a.n_layers ? l + 1 : l);
            asm volatile("" ::: "memory");
        }

        // 4. act = silu(gate) * up
#pragma unroll
        for (int k = 0; k < SWI; ++k) {
            const int v = tid + k * THREADS;
            if (v < iv) {
                float gf[kVec], uf[kVec], of[kVec];
                unpack<T>(gr[k], gf);
                unpack<T>(ur[k], uf);
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    const float ex = __builtin_amdgcn_exp2f(gf[e] * -1.4426950408889634f);
                    of[e] = gf[e] * __builtin_amdgcn_rcpf(1.0f + ex) * uf[e];
                }
                st16_nt<T>(act, (int64_t)v * kVec, pack<T>(of));
            }
        }
    }
}

template <typename T, int THREADS>
static int launch_chain_t(const ChainArgs& a, int64_t batch, void* stream) {
    const int iters = (a.inter / T::kVec + THREADS - 1) / THREADS;
    const dim3 grid((uint32_t)batch), block(THREADS);
    switch (iters) {
        case 1: return launch(decode_chain_kernel<T, 1, THREADS>, grid, block, stream, a);
        case 2: return launch(decode_chain_kernel<T, 2, THREADS>, grid, block, stream, a);
        case 3: return launch(decode_chain_kernel<T, 3, THREADS>, grid, block, stream, a);
        default: return launch(decode_chain_kernel<T, kChainMaxSwigluIters, THREADS>, grid, block, stream, a);
    }
}

// 512 lanes when the token's row, its RoPE units and its SwiGLU vectors (at
// most 4 per lane) fit, else 1024.
template <typename T>
static int launch_chain(const ChainArgs& a, int64_t batch, void* stream) {
    const bool small = a.hidden / T::kVec <= kChainSmallThreads &&
                       a.hkv * (a.group + 2) * a.lpu <= kChainSmallThreads &&
                       a.inter / T::kVec <= kChainMaxSwigluIters * kChainSmallThreads;
    return small ? launch_chain_t<T, kChainSmallThreads>(a, batch, stream)
                 : launch_chain_t<T, kChainThreads>(a, batch, stream);
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
    if (hidden < 1 || hidden % vec != 0 || hidden / vec > kChainThreads) return KCR_ERR_SHAPE;
    if (inter < 1 || inter % vec != 0 || inter / vec > kChainMaxSwigluIters * kChainThreads) return KCR_ERR_SHAPE;
    if (head_dim < 2 || head_dim % 2 != 0 || (head_dim / 2) % vec != 0 || head_dim > KCR_ROPE_MAX_HEAD_DIM)
        return KCR_ERR_SHAPE;
    if (block_size < 1 || num_blocks < 0 || max_pos < 1) return KCR_ERR_SHAPE;
    const int group = n_head / n_kv_head;
    int lpu = 1;
    while (lpu * vec < head_dim / 2) lpu *= 2;
    if ((int64_t)n_kv_head * (group + 2) * lpu > kChainThreads) return KCR_ERR_SHAPE;
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
    return by_dtype(dtype, [&](auto t) { return launch_chain<decltype(t)>(a, batch, stream); });
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

// kcr_device.h -- device-side building blocks shared by the gfx950 kernels:
// 16-byte vector loads and stores with an element-wise tail, bf16 and fp16
// <-> fp32 conversion, and the wave64 sum reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kcr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// The same 16 bytes at 4-byte alignment: global_load/store_dwordx4 need
// only dword alignment, so rows that start 4 or 8 bytes past a 16-byte
// boundary (e.g. 8196 bf16 elements per row) still move as whole vectors.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Storage types. kVec is the number of elements in one 16-byte vector, the
// unit of every global load and store (global_load_dwordx4 /
// global_store_dwordx4).
struct Bf16 {
    using storage = uint16_t;
    static constexpr int kVec = 8;
};
struct F32 {
    using storage = float;
    static constexpr int kVec = 4;
};
struct F16 {
    using storage = uint16_t;
    static constexpr int kVec = 8;
};

// ---------------------------------------------------------------- codec
// bf16 is the top half of an fp32, so widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> two bf16, round to nearest even, one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// IEEE binary16: widening to fp32 is exact (subnormals included); narrowing
// rounds to nearest even, overflowing to inf, in the default float mode.
__device__ __forceinline__ f32x2 f16x2_to_f32(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Unpack a 16-byte vector into kVec floats, and pack back.
template <typename T>
__device__ __forceinline__ void unpack(const u32x4& v, float* f);
template <>
__device__ __forceinline__ void unpack<Bf16>(const u32x4& v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = bf16_lo(v[j]);
        f[2 * j + 1] = bf16_hi(v[j]);
    }
}
template <>
__device__ __forceinline__ void unpack<F16>(const u32x4& v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x2 p = f16x2_to_f32(v[j]);
        f[2 * j] = p[0];
        f[2 * j + 1] = p[1];
    }
}
template <>
__device__ __forceinline__ void unpack<F32>(const u32x4& v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(v[j]);
}

template <typename T>
__device__ __forceinline__ u32x4 pack(const float* f);
template <>
__device__ __forceinline__ u32x4 pack<Bf16>(const float* f) {
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
    return v;
}
template <>
__device__ __forceinline__ u32x4 pack<F16>(const float* f) {
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = pack_f16x2(f[2 * j], f[2 * j + 1]);
    return v;
}
template <>
__device__ __forceinline__ u32x4 pack<F32>(const float* f) {
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __float_as_uint(f[j]);
    return v;
}

// Single elements, for the ragged tail of a row.
template <typename T>
__device__ __forceinline__ float load_one(const void* base, int64_t i);
template <>
__device__ __forceinline__ float load_one<Bf16>(const void* base, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
}
template <>
__device__ __forceinline__ float load_one<F16>(const void* base, int64_t i) {
    return f16_to_f32(static_cast<const uint16_t*>(base)[i]);
}
template <>
__device__ __forceinline__ float load_one<F32>(const void* base, int64_t i) {
    return static_cast<const float*>(base)[i];
}
template <typename T>
__device__ __forceinline__ void store_one(void* base, int64_t i, float v);
template <>
__device__ __forceinline__ void store_one<Bf16>(void* base, int64_t i, float v) {
    static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
}
template <>
__device__ __forceinline__ void store_one<F16>(void* base, int64_t i, float v) {
    static_cast<uint16_t*>(base)[i] = f32_to_f16(v);
}
template <>
__device__ __forceinline__ void store_one<F32>(void* base, int64_t i, float v) {
    static_cast<float*>(base)[i] = v;
}

// ------------------------------------------------------------ vector I/O
// `elem` is an element offset that is a multiple of kVec, so the address is
// 16-byte aligned whenever the base and the row stride are.
template <typename T>
__device__ __forceinline__ u32x4 ld16(const void* base, int64_t elem) {
    return *reinterpret_cast<const u32x4_a4*>(static_cast<const typename T::storage*>(base) + elem);
}
template <typename T>
__device__ __forceinline__ u32x4 ld16_nt(const void* base, int64_t elem) {
    return __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_a4*>(static_cast<const typename T::storage*>(base) + elem));
}
template <typename T>
__device__ __forceinline__ void st16(void* base, int64_t elem, const u32x4& v) {
    *reinterpret_cast<u32x4_a4*>(static_cast<typename T::storage*>(base) + elem) = v;
}
template <typename T>
__device__ __forceinline__ void st16_nt(void* base, int64_t elem, const u32x4& v) {
    const u32x4_a4 w = v;
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_a4*>(static_cast<typename T::storage*>(base) + elem));
}

// Raw-bit variants: the vector starting at element `elem` of a row of `n`
// elements, as it sits in memory. `vec` says whether the row's base address
// is dword aligned (vec_ok); when it is, every vector wholly inside the row
// moves with one 16-byte access, and otherwise (and for the vector that
// straddles the end of the row) element by element. Elements past the end of the row
// read as zero bits (+0.0 in every dtype) and are never written.
__host__ __device__ __forceinline__ bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}
// Whether a row starting at `p` can move as 16-byte vectors (dword-aligned).
__host__ __device__ __forceinline__ bool vec_ok(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 3u) == 0;
}

// The elements [elem, min(elem + kVec, n)) one by one, zero bits past n.
// Every element load is issued, from an in-bounds address (clamped to the
// row's last element), before any is used.
template <typename T>
__device__ __forceinline__ u32x4 load_elems(const void* base, int64_t elem, int64_t n) {
    const typename T::storage* p = static_cast<const typename T::storage*>(base);
    uint32_t bits[T::kVec];
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
        const int64_t i = elem + e < n ? elem + e : n - 1;
        if constexpr (T::kVec == 8) bits[e] = (uint32_t)p[i];
        else bits[e] = __float_as_uint(p[i]);
    }
    u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
        const uint32_t b = elem + e < n ? bits[e] : 0u;
        if constexpr (T::kVec == 8) v[e >> 1] |= b << (16 * (e & 1));
        else v[e] = b;
    }
    return v;
}

// Lanes at or past the end of the row take the element path, where the
// compiler waits for every load the wave has in flight before it goes on,
// so each wave's requests are spaced out. The throughput-bound large-call
// row-norm shapes were tuned with this form and measured faster with it on
// MI355X: bf16 [131072, 2176] streams at 6.46-6.48 TB/s this way against
// 6.31-6.33 with every load issued first. Latency-bound small calls whose
// shape leaves lanes past the row's end take load_whole and load_tail below
// instead ([512, 2176] bf16: 3.22 against 3.77 us per launch).
template <typename T, bool NT>
__device__ __forceinline__ u32x4 load_raw(const void* base, int64_t elem, int64_t n, bool vec = true) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!vec) {  // a row that is not dword aligned: element access throughout
        if (elem < n) v = load_elems<T>(base, elem, n);
        return v;
    }
    if (elem + T::kVec <= n) return NT ? ld16_nt<T>(base, elem) : ld16<T>(base, elem);
    const typename T::storage* p = static_cast<const typename T::storage*>(base) + elem;
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
        if (elem + e < n) {
            if constexpr (T::kVec == 8) v[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
            else v[e] = __float_as_uint(p[e]);
        }
    }
    return v;
}

// Whole 16-byte vectors only: lanes whose vector is not wholly inside the
// row read zero bits, and the vector that straddles the end is left to
// load_tail, which the caller runs once every load of the wave is in flight
// (so the wait its element loads need delays nothing). The result is zero
// bits in its registers before the vector load is issued (the empty asm
// keeps the compiler from sinking the zeros into a branch): were the zeros
// written on their own path, they would overwrite the destination of the
// vector load still in flight in other lanes, and the compiler would wait
// there for every load in flight.
template <typename T, bool NT>
__device__ __forceinline__ u32x4 load_whole(const void* base, int64_t elem, int64_t n) {
    u32x4 v = {0u, 0u, 0u, 0u};
    asm volatile("" : "+v"(v));
    if (elem + T::kVec <= n) v = NT ? ld16_nt<T>(base, elem) : ld16<T>(base, elem);
    return v;
}
template <typename T>
__device__ __forceinline__ void load_tail(const void* base, int64_t elem, int64_t n, u32x4& v) {
    if (elem < n && elem + T::kVec > n) v = load_elems<T>(base, elem, n);
}

template <typename T, bool NT>
__device__ __forceinline__ void store_raw(void* base, int64_t elem, int64_t n, const u32x4& v,
                                          bool vec = true) {
    if (vec && elem + T::kVec <= n) {
        if (NT) st16_nt<T>(base, elem, v); else st16<T>(base, elem, v);
        return;
    }
    typename T::storage* p = static_cast<typename T::storage*>(base) + elem;
#pragma unroll
    for (int e = 0; e < T::kVec; ++e) {
        if (elem + e < n) {
            if constexpr (T::kVec == 8) p[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            else p[e] = __uint_as_float(v[e]);
        }
    }
}

// ------------------------------------------------------------ reductions
// DPP lane permutations within rows of 16 lanes (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm:[1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each half row
constexpr int kDppRowMirror = 0x140;    // lane i <- lane 15-i within each row

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over all 64 lanes of a wave, whole in lane 63 only (the other lanes
// hold partial sums); every lane must be active. Four DPP steps leave each
// 16-lane row's sum r0..r3 in all its lanes; then gfx9's row broadcasts add
// row 0's sum into row 1 and row 2's into row 3 (from lanes 15 and 47), and
// rows 0 + 1 into row 3 (from lane 31), so lane 63 holds (r3 + r2) + (r1 + r0).
// For a reduction whose result one lane stores: no lane reads.
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row -> the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 -> rows 2 and 3

__device__ __forceinline__ float wave_total_lane63(float v) {
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppRowHalfMirror>(v);
    v += dpp<kDppRowMirror>(v);
    // rows outside the row mask take the 0 passed as the old value
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast15, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast31, 0xC, 0xF, false));
    return v;
}

// The same sum made wave-uniform (the same value, bit for bit, in every
// lane): lane 63's total, read out once. Each addition in lane 63 is one of
// (r0 + r1) + (r2 + r3) with its operands swapped, so the result has the
// bits of that order.
__device__ __forceinline__ float wave_sum(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_total_lane63(v)), 63));
}

// Sum over each aligned group of N consecutive lanes (N a power of two up to
// 64); every lane of a group must be active and each gets its group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<kDppQuadXor1>(v);
    if constexpr (N >= 4) v += dpp<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp<kDppRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp<kDppRowMirror>(v);
    if constexpr (N >= 32) v += __shfl_xor(v, 16);
    if constexpr (N >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Every row norm takes its mean square as the sum of squares times the
// width's reciprocal, 1/d rounded once to fp32 (one rounding more than a
// division). Computed at a kernel's start, the reciprocal stays off the path
// from a row's last load to its stores, where a division's dozen dependent
// instructions would sit.
__device__ __forceinline__ float inv_width(int32_t d) { return 1.0f / (float)d; }

// Wave index made explicitly uniform, so that row and unit indices derived
// from it live in scalar registers.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace kcr

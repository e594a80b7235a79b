/*
 * oracle.c -- plain, slow, fp64 CPU definitions of the four per-token ops of
 * small-LLM decode: RMSNorm, residual-add + RMSNorm, rotate-half RoPE with a
 * paged KV-cache store, and SwiGLU.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the HIP library never
 * does, and the two share no source, header, table or helper.
 *
 * Every op is written as its textbook definition in double precision, with
 * no blocking, fusion or reordering, so that each loop can be read against
 * the pages:
 *   - RMSNorm: koas-w.github.io 2026-03-31 post, section 3 ("Triton RMSNorm":
 *     the unfused chain pow -> mean -> add eps -> rsqrt -> mul x -> mul w,
 *     computed in float32 internally and cast back once on write), and
 *     m.lsln.cn/news/61269 section 2.3 (var = sum(x^2)/n_cols,
 *     rstd = 1/sqrt(var + eps), y = x * rstd * w).
 *   - add + RMSNorm: koas-w post, section 4 ("Fused Add Norm"): x is
 *     updated in place to x + residual and the normalised sum is returned.
 *   - RoPE + store: koas-w post, section 1 ("Fused RoPE & Paged KV Cache
 *     Store"): rotate-half RoPE (the halves are sliced, negated and
 *     concatenated), Q written to contiguous memory, rotated K and V written
 *     straight into the paged cache at the slots given by slot_mapping;
 *     cache layout [2, num_blocks, block_size, kv_heads, head_dim] from
 *     mer.dev "AsyncT vLLM notes (1)", section 1.1; slot = block *
 *     block_size + offset from section 1.4 of the same page. The rotation
 *     frequencies are the RoFormer ones, base^(-2i/d).
 *   - SwiGLU: koas-w post, section 2 ("Fused SwiGLU"): silu(gate) * up with
 *     silu(g) = g * sigmoid(g).
 *   - Variants from mer.dev "AsyncT vLLM notes (1)": per-head Q/K RMSNorm
 *     before RoPE (sections 0, 3.3), the paged gather (section 1.4), ReGLU
 *     and the DyHT clip norm (sections 0, 3.3).
 *
 * Inputs arrive in their storage dtype (bf16 or fp16 bit patterns, or fp32) and are
 * widened exactly to double. Results are returned in double, except values
 * that the op itself defines as stored data (the updated residual, the cache
 * image), which are rounded once, to nearest with ties to even, into the
 * storage dtype by this file's own encoder.
 *
 * Parity: every function is pinned by closed forms, invariants, hand-worked
 * cases and independent library cross-checks in the CPU test suite.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F16 = 2 };

/* ------------------------------------------------------------ dtype codec */

/* bf16 is the top half of an IEEE binary32: widening is exact. */
static double bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in one step (no
 * detour through float, which would round twice). bf16 keeps 8 significant
 * bits and binary32's exponent range, subnormals included. */
static uint16_t double_to_bf16(double v) {
    uint64_t bits;
    memcpy(&bits, &v, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (a == 0.0) return sign;
    /* Largest finite bf16 is (2 - 2^-7) * 2^127. Halfway to the next step
     * (2^128) lies at (2 - 2^-8) * 2^127; from there on the result is inf
     * (the tie goes to the even neighbour, which is inf). */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7F80u);
    int e;
    frexp(a, &e);             /* a in [2^(e-1), 2^e) */
    int lg = e - 1;           /* floor(log2(a)) */
    if (lg < -126) lg = -126; /* subnormal range: fixed spacing 2^-133 */
    double q = ldexp(1.0, lg - 7); /* spacing of bf16 values around a */
    double n = rint(a / q);   /* a/q is exact; rint rounds half to even */
    float f = (float)(n * q); /* exact: n*q is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 holds zero and the subnormals (fraction * 2^-24), field
 * 31 the infinities and NaNs. */
static double f16_to_double(uint16_t h) {
    int ex = (h >> 10) & 0x1F;
    int fr = h & 0x3FF;
    double mag;
    if (ex == 0) mag = ldexp((double)fr, -24);
    else if (ex == 31) mag = fr ? NAN : INFINITY;
    else mag = ldexp((double)(1024 + fr), ex - 25);
    return (h & 0x8000u) ? -mag : mag;
}

/* Round a double to the nearest binary16 value, ties to even, in one step.
 * binary16 keeps 11 significant bits; its normals start at 2^-14, below
 * which the spacing is fixed at 2^-24. */
static uint16_t double_to_f16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs(v);
    if (a == 0.0) return sign;
    /* Largest finite value (2 - 2^-10) * 2^15 = 65504; the midpoint to the
     * next step 2^16 is 65520, and from there on the result is inf. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    int e;
    frexp(a, &e);
    int lg = e - 1;
    if (lg < -14) lg = -14;
    double q = ldexp(1.0, lg - 10);
    double r = rint(a / q) * q; /* exact: a binary16 value */
    if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    frexp(r, &e);               /* r in [2^(e-1), 2^e) */
    uint16_t frac = (uint16_t)(ldexp(r, 11 - e) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((e - 1 + 15) << 10) | frac);
}

static double load(const void* base, int64_t i, int dtype) {
    if (dtype == ORC_BF16) return bf16_to_double(((const uint16_t*)base)[i]);
    if (dtype == ORC_F16) return f16_to_double(((const uint16_t*)base)[i]);
    return (double)((const float*)base)[i];
}

/* C's double -> float conversion rounds to nearest even in one step. */
static void store(void* base, int64_t i, double v, int dtype) {
    if (dtype == ORC_BF16) ((uint16_t*)base)[i] = double_to_bf16(v);
    else if (dtype == ORC_F16) ((uint16_t*)base)[i] = double_to_f16(v);
    else ((float*)base)[i] = (float)v;
}

static void copy_bits(void* dst, int64_t di, const void* src, int64_t si, int dtype) {
    if (dtype == ORC_F32) ((uint32_t*)dst)[di] = ((const uint32_t*)src)[si];
    else ((uint16_t*)dst)[di] = ((const uint16_t*)src)[si];
}

void orc_encode(const double* in, void* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) store(out, i, in[i], dtype);
}

void orc_decode(const void* in, double* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = load(in, i, dtype);
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* --------------------------------------------------------------- RMSNorm */

/* One row: ms = sum_j x_j^2 / D over the D real columns; r = 1/sqrt(ms+eps);
 * y_j = x_j * r * w_j. */
static void rmsnorm_row(const void* x, int64_t x_off, const void* w, double* y,
                        int64_t d, double eps, int dtype) {
    double sum_sq = 0.0;
    for (int64_t j = 0; j < d; ++j) {
        double xj = load(x, x_off + j, dtype);
        sum_sq += xj * xj;
    }
    double ms = sum_sq / (double)d;
    double r = 1.0 / sqrt(ms + eps);
    for (int64_t j = 0; j < d; ++j)
        y[j] = load(x, x_off + j, dtype) * r * load(w, j, dtype);
}

void orc_rmsnorm(const void* x, int64_t x_stride, const void* w, double* y, int64_t y_stride,
                 int64_t rows, int64_t d, double eps, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        rmsnorm_row(x, r * x_stride, w, y + r * y_stride, d, eps, dtype);
}

/* x <- round(x + delta) in place, then y = rmsnorm(x_new) * w. The sum of two
 * bf16 or two fp32 values is formed in double and rounded once to the storage
 * dtype; the norm reads the stored (rounded) sum, exactly as the unfused
 * sequence "x = x + attn_out; y = rmsnorm(x)" would. */
void orc_add_rmsnorm(void* x, int64_t x_stride, const void* delta, int64_t delta_stride,
                     const void* w, double* y, int64_t y_stride, int64_t rows, int64_t d,
                     double eps, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < d; ++j) {
            double s = load(x, r * x_stride + j, dtype) + load(delta, r * delta_stride + j, dtype);
            store(x, r * x_stride + j, s, dtype);
        }
        rmsnorm_row(x, r * x_stride, w, y + r * y_stride, d, eps, dtype);
    }
}

/* ------------------------------------------------------------------ RoPE */

/* Angle of frequency i at position p: p * base^(-2i/d). */
static double rope_angle(int64_t p, int i, int d, double base) {
    return (double)p * pow(base, -2.0 * (double)i / (double)d);
}

void orc_rope_angles(double* cos_out, double* sin_out, int64_t max_pos, int head_dim,
                     double base) {
    int half = head_dim / 2;
    for (int64_t p = 0; p < max_pos; ++p)
        for (int i = 0; i < half; ++i) {
            double a = rope_angle(p, i, head_dim, base);
            cos_out[p * half + i] = cos(a);
            sin_out[p * half + i] = sin(a);
        }
}

/* Rotate-half RoPE of one head given in double: element i pairs with
 * element i + d/2;
 *   out_i       = x_i * cos - x_{i+d/2} * sin
 *   out_{i+d/2} = x_{i+d/2} * cos + x_i * sin                              */
static void rotate_half(const double* x, double* out, int64_t p, int d, double base) {
    int half = d / 2;
    for (int i = 0; i < half; ++i) {
        double a = rope_angle(p, i, d, base);
        double c = cos(a), s = sin(a);
        double x1 = x[i];
        double x2 = x[i + half];
        out[i] = x1 * c - x2 * s;
        out[i + half] = x2 * c + x1 * s;
    }
}

/* One head read from its storage dtype and rotated. d <= 1024. */
static void rope_head(const void* x, int64_t x_off, double* out, int64_t p, int d, double base,
                      int dtype) {
    double v[1024];
    for (int e = 0; e < d; ++e) v[e] = load(x, x_off + e, dtype);
    rotate_half(v, out, p, d, base);
}

/* The store: for each token whose slot is in [0, num_blocks * block_size):
 * block = slot / block_size, offset = slot % block_size,
 * cache[0, block, offset, h, :] = round(k_rot) and cache[1, block, offset, h,
 * :] = v (bit copy). Negative slots mark padding tokens and are skipped; the
 * scatter runs in token order, so with repeated slots the last token wins.
 * No other cache element is touched. */
static void scatter_kv(const double* k_rot, const void* v, int64_t v_ts, int64_t v_hs, void* cache,
                       const int64_t* slot_mapping, int64_t T, int hkv, int d, int block_size,
                       int64_t num_blocks, int dtype) {
    int64_t n_slots = num_blocks * (int64_t)block_size;
    for (int64_t t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= n_slots) continue;
        int64_t block = slot / block_size, offset = slot % block_size;
        for (int h = 0; h < hkv; ++h) {
            int64_t k_dst = (((0 * num_blocks + block) * block_size + offset) * hkv + h) * d;
            int64_t v_dst = (((1 * num_blocks + block) * block_size + offset) * hkv + h) * d;
            for (int e = 0; e < d; ++e) {
                store(cache, k_dst + e, k_rot[(t * hkv + h) * d + e], dtype);
                copy_bits(cache, v_dst + e, v, t * v_ts + h * v_hs + e, dtype);
            }
        }
    }
}

/* Q and K heads rotated at positions[t]; q_rot [T, hq, d] and k_rot
 * [T, hkv, d] in double; then the store above when a cache is given. */
void orc_rope_kvstore(const void* q, int64_t q_ts, int64_t q_hs,
                      const void* k, int64_t k_ts, int64_t k_hs,
                      const void* v, int64_t v_ts, int64_t v_hs,
                      const int64_t* positions, double base,
                      double* q_rot, double* k_rot,
                      void* cache, const int64_t* slot_mapping,
                      int64_t T, int hq, int hkv, int d, int block_size,
                      int64_t num_blocks, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int64_t p = positions[t];
        for (int h = 0; h < hq; ++h)
            rope_head(q, t * q_ts + h * q_hs, q_rot + (t * hq + h) * d, p, d, base, dtype);
        for (int h = 0; h < hkv; ++h)
            rope_head(k, t * k_ts + h * k_hs, k_rot + (t * hkv + h) * d, p, d, base, dtype);
    }
    if (cache != 0)
        scatter_kv(k_rot, v, v_ts, v_hs, cache, slot_mapping, T, hkv, d, block_size, num_blocks, dtype);
}

/* Per-head RMSNorm of a query or key head (the qk-norm applied to the
 * narrow Q/K views of a fused QKV projection, mer.dev notes sections 0 and
 * 3.3; RMSNorm as in the koas-w post, section 3):
 * n_e = x_e / sqrt(sum_e x_e^2 / d + eps) * w_e. */
static void rms_norm_head(const void* x, int64_t x_off, const void* w, double eps, int d, int dtype,
                          double* n) {
    double sum_sq = 0.0;
    for (int e = 0; e < d; ++e) {
        double v = load(x, x_off + e, dtype);
        sum_sq += v * v;
    }
    double r = 1.0 / sqrt(sum_sq / (double)d + eps);
    for (int e = 0; e < d; ++e) n[e] = load(x, x_off + e, dtype) * r * load(w, e, dtype);
}

/* As orc_rope_kvstore, with every query head normalised by q_w and every
 * key head by k_w (each [d], eps added to the mean square) before the
 * rotation; V is stored unchanged. d <= 1024. */
void orc_qknorm_rope_kvstore(const void* q, int64_t q_ts, int64_t q_hs,
                             const void* k, int64_t k_ts, int64_t k_hs,
                             const void* v, int64_t v_ts, int64_t v_hs,
                             const void* q_w, const void* k_w, double eps,
                             const int64_t* positions, double base,
                             double* q_rot, double* k_rot,
                             void* cache, const int64_t* slot_mapping,
                             int64_t T, int hq, int hkv, int d, int block_size,
                             int64_t num_blocks, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int64_t p = positions[t];
        double n[1024];
        for (int h = 0; h < hq; ++h) {
            rms_norm_head(q, t * q_ts + h * q_hs, q_w, eps, d, dtype, n);
            rotate_half(n, q_rot + (t * hq + h) * d, p, d, base);
        }
        for (int h = 0; h < hkv; ++h) {
            rms_norm_head(k, t * k_ts + h * k_hs, k_w, eps, d, dtype, n);
            rotate_half(n, k_rot + (t * hkv + h) * d, p, d, base);
        }
    }
    if (cache != 0)
        scatter_kv(k_rot, v, v_ts, v_hs, cache, slot_mapping, T, hkv, d, block_size, num_blocks, dtype);
}

/* GQA: query head h reads the KV head h / (hq / hkv) (koas-w post,
 * section 1). */
int orc_gqa_kv_head(int h, int hq, int hkv) {
    return h / (hq / hkv);
}

/* Paged gather, the inverse of the store: for each token of a sequence,
 * slot = block_table[pos / block_size] * block_size + pos % block_size
 * (mer.dev notes, section 1.4), and out[t, h, :] = cache[which, block,
 * offset, h, :] as a bit copy. */
void orc_paged_gather(const void* cache, int which, const int64_t* block_table, int64_t n_tok,
                      int hkv, int d, int block_size, int64_t num_blocks, void* out, int dtype) {
    for (int64_t t = 0; t < n_tok; ++t) {
        int64_t block = block_table[t / block_size], offset = t % block_size;
        for (int h = 0; h < hkv; ++h)
            for (int e = 0; e < d; ++e)
                copy_bits(out, (t * hkv + h) * d + e, cache,
                          ((((int64_t)which * num_blocks + block) * block_size + offset) * hkv + h) * d + e,
                          dtype);
    }
}

/* ---------------------------------------------------------------- SwiGLU */

/* out = silu(g) * u = g / (1 + exp(-g)) * u. */
void orc_swiglu(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
                double* out, int64_t out_stride, int64_t rows, int64_t cols, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double g = load(gate, r * gate_stride + c, dtype);
            double u = load(up, r * up_stride + c, dtype);
            double sigmoid = 1.0 / (1.0 + exp(-g));
            out[r * out_stride + c] = g * sigmoid * u;
        }
}

/* ----------------------------------------------------------------- ReGLU */

/* out = relu(g) * u, relu(g) = g if g > 0 else 0 (the ReGLU of the mer.dev
 * AsyncT notes, section 0, fused as relu_and_mul in section 3.3). */
void orc_reglu(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
               double* out, int64_t out_stride, int64_t rows, int64_t cols, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double g = load(gate, r * gate_stride + c, dtype);
            double u = load(up, r * up_stride + c, dtype);
            double relu = g > 0.0 ? g : 0.0;
            out[r * out_stride + c] = relu * u;
        }
}

/* ------------------------------------------------------------ DyHT / clip */

/* y[t, h, e] = clamp(alpha_e * x[t, h, e], lo, hi) * gamma_e over an
 * [n_tok, n_head, d] view with token and head strides (the DyHT norm of the
 * mer.dev AsyncT notes, section 0, y * clamp(a x, -1, 1), and its clip-norm
 * kernel in section 3.3 with per-channel or scalar a and gamma: a scalar
 * parameter is read at index 0 for every channel). */
void orc_clip_norm(const void* x, int64_t x_ts, int64_t x_hs, const void* alpha, int alpha_per_ch,
                   const void* gamma, int gamma_per_ch, double lo, double hi, double* y,
                   int64_t n_tok, int n_head, int d, int dtype) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t)
        for (int h = 0; h < n_head; ++h)
            for (int e = 0; e < d; ++e) {
                double a = load(alpha, alpha_per_ch ? e : 0, dtype);
                double g = load(gamma, gamma_per_ch ? e : 0, dtype);
                double v = a * load(x, t * x_ts + h * x_hs + e, dtype);
                if (v < lo) v = lo;
                if (v > hi) v = hi;
                y[(t * n_head + h) * d + e] = v * g;
            }
}

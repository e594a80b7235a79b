/*
 * kcr.h -- C ABI of libkcr: hand-written HIP kernels for AMD MI355X (gfx950)
 * covering the memory-bound per-token ops of small-LLM decode.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor arguments are DEVICE pointers into memory the caller allocated on
 *    the current HIP device; the library never allocates, frees, copies to
 *    the host or synchronizes. Work is enqueued on `stream` (a hipStream_t
 *    passed as void*; NULL means the default stream) and the call returns
 *    as soon as the kernel is queued.
 *  - Strides are in ELEMENTS, not bytes. The innermost dimension of every
 *    tensor is contiguous.
 *  - `dtype` is one of kcr_dtype. Weights, activations and the KV cache of
 *    one call share that dtype; arithmetic is done in fp32 and every output
 *    element is rounded once (to nearest, ties to even) into the dtype.
 *  - Alignment: every pointer must be aligned to its element size
 *    (KCR_ERR_ALIGN otherwise). Rows whose base address is 4-byte aligned
 *    move with 16-byte vector loads and stores; other rows (a 2-byte dtype
 *    at an odd element offset, e.g. the rows of a densely packed tensor of
 *    odd width) are accessed element by element, correct but slower.
 *    kcr_rope_kvstore is stricter, see there.
 *  - Arguments are validated on the host before anything is launched; a
 *    negative return code means nothing was enqueued. A call with no work
 *    (rows == 0, T == 0) returns KCR_OK and launches nothing, and NULL
 *    pointers are accepted then.
 *  - Data-dependent indices (positions, slots) are bounds-checked inside the
 *    kernels: an out-of-range index skips that token's writes instead of
 *    touching memory outside the caller's buffers.
 *  - Calls are thread-safe. The only library state is set once: per device,
 *    the compute-unit count, the LDS per workgroup and whether the wide-row
 *    kernel's LDS limit has been raised; per thread, the events armed by
 *    kcr_time_next_launch.
 *  - Debug mode: with the environment variable KCR_DEBUG set to a non-zero
 *    integer when the library first launches, every call synchronizes its
 *    stream after the launch (except while the stream is being captured into
 *    a graph) and returns KCR_ERR_LAUNCH if the kernel failed.
 *
 * Citations name the web page and the section that defines each operation.
 */
#ifndef KCR_H
#define KCR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kcr_dtype {
    KCR_BF16 = 0, /* bfloat16 storage, fp32 arithmetic */
    KCR_F32 = 1,  /* float32 storage and arithmetic */
    KCR_F16 = 2   /* IEEE binary16 storage, fp32 arithmetic */
} kcr_dtype;

enum kcr_status {
    KCR_OK = 0,
    KCR_ERR_NULL = -1,   /* a required pointer is NULL while there is work to do */
    KCR_ERR_SHAPE = -2,  /* a size is negative, zero where it must not be, or above a limit */
    KCR_ERR_DTYPE = -3,  /* dtype is not a kcr_dtype */
    KCR_ERR_ALIGN = -4,  /* a base pointer or a stride breaks 16-byte vector alignment */
    KCR_ERR_HEADS = -5,  /* n_head is not a multiple of n_kv_head */
    KCR_ERR_ALIAS = -6,  /* an output overlaps an input in a way the op does not allow */
    KCR_ERR_LAUNCH = -7, /* the HIP runtime refused the launch, or (KCR_DEBUG) the kernel failed */
    KCR_ERR_DEVICE = -8  /* no usable HIP device is current */
};

/* Row widths of kcr_rmsnorm / kcr_add_rmsnorm. Rows of up to 4096 16-byte
 * vectors (32768 bf16/fp16 or 16384 fp32 elements) are held in registers
 * and read from HBM once. Wider rows take a two-pass form, one workgroup per
 * row: rows of up to about 160 KB are staged in LDS and still read once;
 * wider rows are read twice. KCR_NORM_MAX_D bounds every dtype. */
#define KCR_NORM_REG_MAX_D_16 32768
#define KCR_NORM_REG_MAX_D_F32 16384
#define KCR_NORM_MAX_D (1 << 30)
/* Largest head_dim accepted by kcr_rope_kvstore. */
#define KCR_ROPE_MAX_HEAD_DIM 512

/*
 * kcr_rmsnorm -- row-wise RMSNorm with fp32 accumulation.
 *
 *   for each row r < rows:
 *     ms   = sum_{j<d} x[r,j]^2 / d          (fp32 sum of the d real columns,
 *                                             times 1/d rounded once to fp32)
 *     y[r,j] = x[r,j] * (ms + eps)^(-1/2) * w[j]
 *
 * Defined in the koas-w.github.io 2026-03-31 post, section 3 ("Triton
 * RMSNorm": pow, mean, add eps, rsqrt, mul x, mul weight in one pass, fp32
 * inside, cast back to the input dtype on write) and in m.lsln.cn/news/61269
 * section 2.3 (var = sum(x^2)/n_cols, rstd = 1/sqrt(var + eps),
 * y = x * rstd * w); the one-pass, register-resident form follows the csdn
 * "Qwen3 from scratch (4-2): RMSNorm in Triton" page.
 *
 *   x    [rows, d] at row stride x_stride (>= d)          input
 *   w    [d]       contiguous                              input
 *   y    [rows, d] at row stride y_stride (>= d)          output
 *   eps  added to the mean square before the reciprocal square root
 *
 * y may be x itself (same pointer and stride: in-place); any other overlap
 * of y with x or w is KCR_ERR_ALIAS. 1 <= d <= KCR_NORM_MAX_D else
 * KCR_ERR_SHAPE.
 */
int kcr_rmsnorm(const void* x, int64_t x_stride, const void* w, void* y, int64_t y_stride,
                int64_t rows, int64_t d, float eps, int dtype, void* stream);

/*
 * kcr_add_rmsnorm -- residual add fused with RMSNorm.
 *
 *   x[r,j] <- round(x[r,j] + delta[r,j])            (x is updated in place)
 *   y[r,:]  = rmsnorm(x[r,:]) * w                   (norm of the rounded sum)
 *
 * Defined in the koas-w.github.io 2026-03-31 post, section 4 ("Fused Add
 * Norm"): x + residual is formed in registers, x is updated in place to the
 * sum and the normalised sum is returned (one read of each input, two
 * writes). The stored sum is what the norm sees, so the result equals the
 * unfused "x = x + delta; y = rmsnorm(x)" and the updated x is bit-exact.
 *
 *   x     [rows, d] at x_stride       input and output (the residual stream)
 *   delta [rows, d] at delta_stride   input (attention or MLP output)
 *   w, y, eps, rows, d                as for kcr_rmsnorm
 *
 * y must not overlap x, delta or w, and delta must not overlap x
 * (KCR_ERR_ALIAS). Limits as for kcr_rmsnorm.
 */
int kcr_add_rmsnorm(void* x, int64_t x_stride, const void* delta, int64_t delta_stride,
                    const void* w, void* y, int64_t y_stride, int64_t rows, int64_t d,
                    float eps, int dtype, void* stream);

/*
 * kcr_rope_kvstore -- rotate-half RoPE of Q and K fused with the paged
 * KV-cache store of the rotated K and of V.
 *
 * For each token t with p = positions[t] and each frequency i < head_dim/2,
 * with c = cos_tab[p, i] and s = sin_tab[p, i]:
 *     out[i]              = x[i] * c - x[i + head_dim/2] * s
 *     out[i + head_dim/2] = x[i + head_dim/2] * c + x[i] * s
 * for every query head (written to q_out) and every KV head (written to the
 * cache). Then, if 0 <= slot = slot_mapping[t] < num_blocks * block_size,
 * with block = slot / block_size and offset = slot % block_size:
 *     kv_cache[0, block, offset, h, :] = rotated k[t, h, :]
 *     kv_cache[1, block, offset, h, :] = v[t, h, :]           (bit copy)
 *
 * Defined in the koas-w.github.io 2026-03-31 post, section 1 ("Fused RoPE &
 * Paged KV Cache Store": Q, K, V, cos and sin read once, the rotation done in
 * registers, Q written back to contiguous memory, rotated K and V written
 * directly to the cache slots named by slot_mapping; query heads share KV
 * heads through kv_head = head / (n_head / n_kv_head)); rotate-half pairing
 * from the same section's description of the unfused version (slice the
 * halves, negate, concatenate); cache layout from mer.dev "AsyncT vLLM notes
 * (1)", section 1.1, and slot = block * block_size + offset from its
 * section 1.4; precomputed cos/sin tables from m.lsln.cn/news/61269
 * section 2.3.
 *
 *   q   [T, n_head, head_dim]     strides (q_tok_stride, q_head_stride)   input
 *   k   [T, n_kv_head, head_dim]  strides (k_tok_stride, k_head_stride)   input
 *   v   [T, n_kv_head, head_dim]  strides (v_tok_stride, v_head_stride)   input
 *       (q, k and v may be narrow views of one fused QKV projection buffer)
 *   q_out [T, n_head, head_dim] contiguous                                output
 *       may be q itself only when q is contiguous; no other overlap
 *   positions [T] int64; a token with p outside [0, max_pos) gets its
 *       query heads copied to q_out unrotated and writes nothing to the cache
 *   cos_tab, sin_tab [max_pos, head_dim/2] fp32, contiguous (for example
 *       from kcr_rope_cos_sin)
 *   kv_cache [2, num_blocks, block_size, n_kv_head, head_dim] contiguous
 *   slot_mapping [T] int64; a negative slot marks a padding token whose K
 *       and V are not stored; slots must be distinct (with repeats, which
 *       token's data lands in the slot is unspecified)
 *
 * Alignment: q, k, v, q_out, the tables and the cache must be 16-byte
 * aligned and every head and token stride a multiple of 16 bytes
 * (KCR_ERR_ALIGN); positions and slot_mapping 8-byte aligned.
 *
 * Errors: KCR_ERR_HEADS when n_head % n_kv_head != 0; KCR_ERR_SHAPE unless
 * head_dim is even, head_dim/2 is a multiple of 16 bytes' worth of elements
 * (8 bf16, 4 fp32), head_dim <= KCR_ROPE_MAX_HEAD_DIM, n_kv_head >= 1,
 * block_size >= 1, num_blocks >= 0, max_pos >= 1; KCR_ERR_ALIAS when q_out
 * overlaps k, v, the tables, positions, slot_mapping or the cache, or the
 * cache overlaps q, k, v, the tables, positions or slot_mapping.
 */
int kcr_rope_kvstore(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                     const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                     const void* v, int64_t v_tok_stride, int64_t v_head_stride,
                     void* q_out, const int64_t* positions, const float* cos_tab,
                     const float* sin_tab, int64_t max_pos, void* kv_cache,
                     const int64_t* slot_mapping, int64_t T, int n_head, int n_kv_head,
                     int head_dim, int block_size, int64_t num_blocks, int dtype, void* stream);

/*
 * kcr_qknorm_rope_kvstore -- kcr_rope_kvstore with a per-head RMSNorm of
 * every query and key head before the rotation:
 *     x <- x * (sum_e x_e^2 / head_dim + eps)^(-1/2) * w
 * with w = q_norm_w [head_dim] for query heads and k_norm_w [head_dim] for
 * key heads (activation dtype, 16-byte aligned); V is stored unchanged. The
 * normalised head stays in fp32 through the rotation and is rounded once.
 *
 * The qk-norm that mer.dev "AsyncT vLLM notes (1)" counts among the model's
 * RMSNorms (section 0) and runs on the narrow [N, H, D] Q/K views of the
 * fused QKV projection (section 3.3); RMSNorm as in the koas-w.github.io
 * 2026-03-31 post, section 3. Every other argument, limit and error is as
 * for kcr_rope_kvstore; the weights may not overlap q_out or the cache.
 */
int kcr_qknorm_rope_kvstore(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                            const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                            const void* v, int64_t v_tok_stride, int64_t v_head_stride,
                            const void* q_norm_w, const void* k_norm_w, float eps, void* q_out,
                            const int64_t* positions, const float* cos_tab, const float* sin_tab,
                            int64_t max_pos, void* kv_cache, const int64_t* slot_mapping, int64_t T,
                            int n_head, int n_kv_head, int head_dim, int block_size,
                            int64_t num_blocks, int dtype, void* stream);

/*
 * kcr_rope_cos_sin -- fill the RoPE tables on the device:
 *     cos_tab[p, i] = cos(p * theta^(-2i/head_dim)),  sin_tab likewise,
 * for p < max_pos and i < head_dim/2, evaluated in fp64 and rounded once
 * to fp32. The tables are precomputed once rather than evaluated per token
 * (m.lsln.cn/news/61269, section 2.3) and kept in fp32 because low-precision
 * trigonometry loses accuracy as positions grow (same page, section 1.1).
 * Frequencies are the RoFormer ones.
 *
 *   cos_tab, sin_tab [max_pos, head_dim/2] fp32 device outputs, 16-byte
 *   aligned; head_dim even and >= 2; max_pos >= 0; theta > 0 (KCR_ERR_SHAPE
 *   otherwise).
 */
int kcr_rope_cos_sin(float* cos_tab, float* sin_tab, int64_t max_pos, int head_dim,
                     double theta, void* stream);

/*
 * kcr_rope_cos_sin_host -- the same tables, computed on the host into HOST
 * memory (for callers that build them once and copy them to the device
 * themselves): cos_tab[p, i] = cos(p * theta^(-2i/head_dim)), sin_tab
 * likewise, in fp64 rounded once to fp32, with the precompute and fp32
 * reasons of m.lsln.cn/news/61269, sections 2.3 and 1.1.
 *
 *   cos_tab, sin_tab [max_pos, head_dim/2] fp32 host outputs (caller-owned,
 *   not overlapping); head_dim even and >= 2; max_pos >= 0; theta > 0
 *   (KCR_ERR_SHAPE otherwise). Synchronous; touches no device.
 */
int kcr_rope_cos_sin_host(float* cos_tab, float* sin_tab, int64_t max_pos, int head_dim,
                          double theta);

/*
 * kcr_swiglu -- SwiGLU activation: out = silu(gate) * up, with
 * silu(g) = g / (1 + exp(-g)), in fp32, rounded once.
 *
 * Defined in the koas-w.github.io 2026-03-31 post, section 2 ("Fused
 * SwiGLU": gate and up loaded together, sigmoid, gate * sigmoid and the
 * product with up done in registers, one write); the flattened (row x
 * column) work split follows the same section.
 *
 *   gate [rows, cols] at gate_stride   input
 *   up   [rows, cols] at up_stride     input
 *   out  [rows, cols] at out_stride    output
 *
 * For a fused gate_up [rows, 2*cols] buffer (gate first): up = gate + cols
 * and gate_stride = up_stride = 2*cols. out may be gate or up itself (same
 * pointer and stride); any other overlap is KCR_ERR_ALIAS. rows * ceil(cols
 * / (16 bytes' worth of elements)) must stay below 2^31 (KCR_ERR_SHAPE).
 */
int kcr_swiglu(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride,
               void* out, int64_t out_stride, int64_t rows, int64_t cols, int dtype,
               void* stream);

/*
 * kcr_reglu -- ReGLU activation: out = relu(gate) * up, relu(g) = max(g, 0),
 * in fp32, rounded once. The ReGLU that replaces SwiGLU in the AsyncT model
 * (mer.dev "AsyncT vLLM notes (1)", section 0), fused as relu_and_mul
 * (section 3.3). Arguments, layouts, limits and errors as for kcr_swiglu.
 */
int kcr_reglu(const void* gate, int64_t gate_stride, const void* up, int64_t up_stride, void* out,
              int64_t out_stride, int64_t rows, int64_t cols, int dtype, void* stream);

/*
 * kcr_clip_norm -- the DyHT clip norm over a strided [n_tok, n_head, d] view:
 *     y[t, h, e] = clamp(alpha_e * x[t, h, e], lo, hi) * gamma_e
 * in fp32, rounded once. alpha and gamma are per channel ([d]) when their
 * *_per_channel flag is nonzero, else one scalar ([1]).
 *
 * DyHT(x) = y * clamp(a x, -1, 1) replaces every RMSNorm of the AsyncT model
 * (mer.dev "AsyncT vLLM notes (1)", section 0); the page's clip-norm kernel
 * (section 3.3) takes per-channel or scalar a and g and clip bounds, and the
 * same section warns that Q/K norms run on narrow [N, H, D] views of the
 * fused QKV projection, so both the token and the head stride are taken.
 *
 *   x [n_tok, n_head, d] at (x_tok_stride, x_head_stride)   input
 *   y [n_tok, n_head, d] at (y_tok_stride, y_head_stride)   output; may be x
 *       itself (same pointer and strides), no other overlap with x, alpha,
 *       gamma
 *   lo <= hi (KCR_ERR_SHAPE otherwise; DyHT uses -1, 1)
 */
int kcr_clip_norm(const void* x, int64_t x_tok_stride, int64_t x_head_stride, void* y,
                  int64_t y_tok_stride, int64_t y_head_stride, int64_t n_tok, int n_head, int d,
                  const void* alpha, int alpha_per_channel, const void* gamma,
                  int gamma_per_channel, float lo, float hi, int dtype, void* stream);

/*
 * kcr_paged_kv_gather -- read the paged KV cache back into contiguous
 * per-sequence K and V:
 *     for b < n_seqs, t < min(seq_lens[b], max_len), with
 *     slot = block_tables[b, t / block_size] * block_size + t % block_size:
 *       k_out[b, t, :, :] = kv_cache[0, slot / block_size, slot % block_size, :, :]
 *       v_out[b, t, :, :] = kv_cache[1, ...]                        (bit copies)
 *
 * The read side of the cache: op 19 (cache_kv_read) of the op list in
 * m.lsln.cn/news/61269 section 2.1, and the vectorized gather of mer.dev
 * "AsyncT vLLM notes (1)" section 1.4 (token index = block_table *
 * block_size + offset).
 *
 *   kv_cache [2, num_blocks, block_size, n_kv_head, head_dim] contiguous   input
 *   block_tables [n_seqs, max_blocks_per_seq] int64, row-major             input
 *   seq_lens [n_seqs] int64                                                input
 *   k_out, v_out [n_seqs, max_len, n_kv_head, head_dim] contiguous         outputs
 *
 * Rows at t >= seq_lens[b], and rows whose block id is outside
 * [0, num_blocks), are left untouched. n_kv_head * head_dim must be a
 * multiple of 16 bytes' worth of elements and max_len <= max_blocks_per_seq
 * * block_size (KCR_ERR_SHAPE); kv_cache, k_out and v_out 16-byte aligned
 * (KCR_ERR_ALIGN); outputs may not overlap each other or any input
 * (KCR_ERR_ALIAS).
 */
int kcr_paged_kv_gather(const void* kv_cache, int64_t num_blocks, int block_size, int n_kv_head,
                        int head_dim, const int64_t* block_tables, int64_t max_blocks_per_seq,
                        const int64_t* seq_lens, int64_t n_seqs, int64_t max_len, void* k_out,
                        void* v_out, int dtype, void* stream);

/*
 * kcr_decode_chain_b1 -- the whole per-layer chain of one batch-1 decode
 * step in a single launch:
 *
 *   for each layer l < n_layers, in order:
 *     h <- round(h + d_attn);  y_attn = rmsnorm(h) * w_attn      (kcr_add_rmsnorm)
 *     rope + store of the token's q/k/v (from the layer's fused qkv) at
 *       positions[0] into the layer's cache at slot_mapping[0]    (kcr_rope_kvstore)
 *     h <- round(h + d_mlp);   y_mlp  = rmsnorm(h) * w_mlp       (kcr_add_rmsnorm)
 *     act = silu(gate) * up, from the layer's fused gate_up     (kcr_swiglu)
 *
 * Each op is the one defined above (the koas-w.github.io 2026-03-31 post,
 * sections 1, 2 and 4) and its results are those of the separate calls made
 * in this order (the residual and the cache's V rows bit for bit; the
 * norms' outputs up to the order in which a row's squares are summed, within
 * the same tolerances): the launch-overhead elimination (one launch instead of four
 * per layer) that m.lsln.cn/news/61269 section 4 seeks with CUDA Graph. Only
 * the residual passes from op to op, so inside the launch one workgroup runs
 * the token's residual chain (h in registers) while other workgroups run
 * every layer's RoPE + store and SwiGLU at the same time. Batch 1 only: the
 * ops' GEMMs and attention (not part of this library) are not in between.
 *
 *   layers [n_layers]  HOST array of per-layer device pointers (read during
 *        the call; 0 <= n_layers <= KCR_B1_MAX_LAYERS):
 *          d_attn, w_attn, d_mlp, w_mlp [hidden]       inputs
 *          y_attn, y_mlp [hidden]                      outputs
 *          qkv [(n_head + 2 n_kv_head) * head_dim]     input, heads in that order
 *          q_out [n_head * head_dim]                   output
 *          kv_cache [2, num_blocks, block_size, n_kv_head, head_dim]  in/out
 *          gate_up [2 * inter] (gate first)            input
 *          act [inter]                                 output
 *   h [hidden]                  device, input and output (the residual)
 *   positions, slot_mapping [1] int64 device; cos_tab, sin_tab as for
 *        kcr_rope_kvstore (slot < 0 or out of range: nothing stored)
 *
 * Limits (KCR_ERR_SHAPE): hidden and inter multiples of 16 bytes' worth of
 * elements, hidden <= 1024 such vectors, inter <= 4096 of them, head_dim as
 * for kcr_rope_kvstore with (n_head + 2 n_kv_head) heads of at most 1024
 * lanes in all. Every pointer 16-byte aligned (KCR_ERR_ALIGN); a layer's
 * outputs and h may not overlap one another or that layer's inputs, the
 * tables, positions or slot_mapping (KCR_ERR_ALIAS).
 */
#define KCR_B1_MAX_LAYERS 32
typedef struct kcr_chain_layer {
    const void* d_attn;
    const void* w_attn;
    void* y_attn;
    const void* qkv;
    void* q_out;
    void* kv_cache;
    const void* d_mlp;
    const void* w_mlp;
    void* y_mlp;
    const void* gate_up;
    void* act;
} kcr_chain_layer;

int kcr_decode_chain_b1(const kcr_chain_layer* layers, int n_layers, void* h, int hidden,
                        int inter, int n_head, int n_kv_head, int head_dim,
                        const int64_t* positions, const int64_t* slot_mapping,
                        const float* cos_tab, const float* sin_tab, int64_t max_pos,
                        int block_size, int64_t num_blocks, float eps, int dtype, void* stream);

/*
 * kcr_decode_chain_batch -- the same chain for `batch` tokens in one launch:
 * kcr_decode_chain_b1 is this call with batch = 1. Every op of the chain is
 * row-wise, so token b's outputs depend on token b's inputs alone (and on
 * the shared weights and tables); one workgroup per token runs its residual
 * chain, other workgroups its RoPE + stores and every (layer, token) SwiGLU,
 * and no workgroup waits for another. The results are those of the
 * separate calls, each over the whole batch, in the order above.
 *
 *   batch        0 <= batch < 2^20 tokens (0: nothing is launched)
 *   layers       as for kcr_decode_chain_b1, each per-token tensor with
 *        `batch` contiguous rows (token b's row at b times the row width):
 *        d_attn, y_attn, d_mlp, y_mlp [batch, hidden];
 *        qkv [batch, (n_head + 2 n_kv_head) * head_dim];
 *        q_out [batch, n_head * head_dim]; gate_up [batch, 2 * inter];
 *        act [batch, inter]. w_attn, w_mlp [hidden] and the cache are shared.
 *   h [batch, hidden]           device, input and output (the residual)
 *   positions, slot_mapping [batch] int64 device. Two tokens with the same
 *        valid slot store into one cache row; which one lands there is
 *        unspecified (as for kcr_rope_kvstore).
 *
 * For both entry points, a buffer that one layer writes may not overlap any
 * buffer of another layer, since the layers' ops run concurrently
 * (KCR_ERR_ALIAS, checked before anything is launched).
 * Inputs may be shared between layers (e.g. one weight), and so may a
 * cache when the layers name exactly the same cache range: the chain never
 * reads the cache, and the last layer's K/V rows land there, as with the
 * separate calls.
 *
 * Limits, alignment and aliasing as for kcr_decode_chain_b1, over the
 * batch's whole rows; batch out of range is KCR_ERR_SHAPE.
 */
int kcr_decode_chain_batch(const kcr_chain_layer* layers, int n_layers, int64_t batch, void* h,
                           int hidden, int inter, int n_head, int n_kv_head, int head_dim,
                           const int64_t* positions, const int64_t* slot_mapping,
                           const float* cos_tab, const float* sin_tab, int64_t max_pos,
                           int block_size, int64_t num_blocks, float eps, int dtype, void* stream);

/*
 * kcr_copy -- plain streaming copy of `bytes` bytes (a multiple of 16, both
 * pointers 16-byte aligned, no overlap). It moves data with the same 16-byte
 * vector loads and stores as the kernels above and serves as the measured
 * bandwidth ceiling and as the reference for hardware byte counters. A copy
 * of more than 2^32 - 64 vectors (64 GiB) runs as several launches over
 * consecutive ranges; a timing arming (kcr_time_next_launch) then stamps
 * the first of them only.
 */
int kcr_copy(void* dst, const void* src, int64_t bytes, void* stream);

/* Measurement hook: the calling thread's next kernel launch through this
 * library records `start_event` when the kernel begins executing and
 * `stop_event` when it ends (hipExtLaunchKernel), so their elapsed time is
 * the kernel's own duration, free of launch gaps. Both are hipEvent_t
 * handles created by the caller with timing enabled (either may be NULL).
 * The arming is consumed by that one launch. */
int kcr_time_next_launch(void* start_event, void* stop_event);

/* Number of compute units of the current device (0 if none is usable). */
int kcr_device_cus(void);

/* Checks the host-side helper arithmetic (fast integer division constants,
 * dispatch bucket choice) exhaustively on small ranges and by sampling on
 * large ones. Needs no GPU. Returns 0 on success, else the number of the
 * first failing check. */
int kcr_selftest_host(void);

/* Human-readable message for a kcr_status value. */
const char* kcr_strerror(int status);

/* Library version string. */
const char* kcr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KCR_H */

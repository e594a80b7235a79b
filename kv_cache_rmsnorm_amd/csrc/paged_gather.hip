// paged_gather.hip -- read a paged KV cache back into contiguous per-sequence
// K and V (kcr_paged_kv_gather).
//
// The read side of the cache write: op 19 (cache_kv_read) of the 21-op list
// in m.lsln.cn/news/61269 section 2.1 ("just pointer offsets"), and the
// vectorized gather of mer.dev "AsyncT vLLM notes (1)" section 1.4: the
// physical slot of position t of a sequence is
// block_table[t / block_size] * block_size + t % block_size.
//
// gfx950 design: one wave per (sequence, position), four per workgroup (one
// per workgroup measured 6% slower on MI355X, two the same), a one-pass
// grid; the length and block id are wave-uniform scalar loads and
// the lanes copy the token's K and V rows with nontemporal 16-byte loads and
// stores. Lengths and block ids are checked in the kernel, so a bad table
// entry skips its row instead of reading outside the cache.
#include "kcr_device.h"
#include "kcr_host.h"

namespace kcr {

struct GatherArgs {
    const void* cache;
    void* k_out;
    void* v_out;
    const int64_t* block_tables;
    const int64_t* seq_lens;
    int64_t bt_stride;    // entries per sequence in block_tables
    int64_t num_blocks;
    int64_t row_elems;    // n_kv_head * head_dim
    int64_t kv_elems;     // num_blocks * block_size * row_elems: offset of the V half
    uint32_t tokens;      // n_seqs * max_len
    uint32_t cpt;         // 16-byte chunks per token (K row and V row)
    uint32_t k_chunks;    // chunks in one K row
    FastDiv len;          // max_len
    FastDiv bs;           // block_size
};

// One wave per (sequence, position), WAVES per workgroup: the wave-uniform
// length and block-id reads become scalar loads, and the lanes copy the
// token's K and V rows (for 2 KV heads of 128 bf16 that is exactly one
// 16-byte chunk per lane). The block id is read together with the length:
// t < max_len <= max_blocks_per_seq * block_size (checked on the host), so
// its table entry exists even for a position past the sequence's length.
template <typename T, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void paged_gather_kernel(const GatherArgs a) {
    using S = typename T::storage;
    const uint32_t tok = blockIdx.x * (uint32_t)WAVES + (uint32_t)wave_id();
    if (tok >= a.tokens) return;
    const uint32_t b = fastdiv(tok, a.len);
    const uint32_t t = tok - b * a.len.d;
    const uint32_t lb = fastdiv(t, a.bs);
    const int64_t len = a.seq_lens[b];
    const int64_t blk = a.block_tables[(int64_t)b * a.bt_stride + lb];
    if ((int64_t)t >= len) return;
    if (blk < 0 || blk >= a.num_blocks) return;
    const int64_t slot = blk * a.bs.d + (t - lb * a.bs.d);
    const S* ksrc = static_cast<const S*>(a.cache) + slot * a.row_elems;
    const S* vsrc = ksrc + a.kv_elems;
    S* kdst = static_cast<S*>(a.k_out) + (int64_t)tok * a.row_elems;
    S* vdst = static_cast<S*>(a.v_out) + (int64_t)tok * a.row_elems;
    for (uint32_t c = threadIdx.x & 63; c < a.cpt; c += 64) {
        const bool is_v = c >= a.k_chunks;
        const int64_t cc = (int64_t)(is_v ? c - a.k_chunks : c) * T::kVec;
        st16_nt<T>(is_v ? vdst : kdst, cc, ld16_nt<T>(is_v ? vsrc : ksrc, cc));
    }
}

}  // namespace kcr

using namespace kcr;

extern "C" int kcr_paged_kv_gather(const void* kv_cache, int64_t num_blocks, int block_size,
                                   int n_kv_head, int head_dim, const int64_t* block_tables,
                                   int64_t max_blocks_per_seq, const int64_t* seq_lens,
                                   int64_t n_seqs, int64_t max_len, void* k_out, void* v_out,
                                   int dtype, void* stream) {
    if (!dtype_ok(dtype)) return KCR_ERR_DTYPE;
    const size_t es = dtype_size(dtype);
    const int64_t vec = (int64_t)(16 / es);
    if (num_blocks < 0 || block_size < 1 || n_kv_head < 1 || head_dim < 1 || n_seqs < 0 ||
        max_len < 0 || max_blocks_per_seq < 0)
        return KCR_ERR_SHAPE;
    const int64_t row = (int64_t)n_kv_head * head_dim;
    if (row % vec != 0) return KCR_ERR_SHAPE;
    if (max_len > max_blocks_per_seq * block_size) return KCR_ERR_SHAPE;
    const int64_t cpt = 2 * row / vec;
    if (n_seqs * max_len * cpt >= (int64_t(1) << 31)) return KCR_ERR_SHAPE;
    if (n_seqs == 0 || max_len == 0) return KCR_OK;
    if (!kv_cache || !block_tables || !seq_lens || !k_out || !v_out) return KCR_ERR_NULL;
    if (!aligned16(kv_cache) || !aligned16(k_out) || !aligned16(v_out) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 7u) || (reinterpret_cast<uintptr_t>(seq_lens) & 7u))
        return KCR_ERR_ALIGN;
    const int64_t out_elems = n_seqs * max_len * row;
    const Span sc = span2d(kv_cache, 1, 0, 2 * num_blocks * block_size * row, es);
    const Span sk = span2d(k_out, 1, 0, out_elems, es), sv = span2d(v_out, 1, 0, out_elems, es);
    const Span sb = span2d(block_tables, 1, 0, n_seqs * max_blocks_per_seq, 8);
    const Span sl = span2d(seq_lens, 1, 0, n_seqs, 8);
    if (overlap(sk, sv) || overlap(sk, sc) || overlap(sv, sc) || overlap(sk, sb) || overlap(sv, sb) ||
        overlap(sk, sl) || overlap(sv, sl))
        return KCR_ERR_ALIAS;
    if (device_cus() <= 0) return KCR_ERR_DEVICE;
    const uint32_t tokens = (uint32_t)(n_seqs * max_len);
    GatherArgs a{kv_cache, k_out, v_out, block_tables, seq_lens, max_blocks_per_seq, num_blocks, row,
                 num_blocks * block_size * row, tokens, (uint32_t)cpt, (uint32_t)(row / vec),
                 make_fastdiv((uint32_t)max_len), make_fastdiv((uint32_t)block_size)};
    constexpr int kWaves = 4;
    const dim3 grid((tokens + kWaves - 1) / kWaves);
    // The gather moves bits: both 2-byte dtypes take the same kernel.
    return dtype == KCR_F32 ? launch(paged_gather_kernel<F32, kWaves>, grid, dim3(64 * kWaves), stream, a)
                            : launch(paged_gather_kernel<Bf16, kWaves>, grid, dim3(64 * kWaves), stream, a);
}

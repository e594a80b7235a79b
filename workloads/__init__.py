"""Seeded synthetic inputs for the four per-token decode ops.

This module only draws and lays out input data. It holds none of the
arithmetic of RMSNorm, RoPE, the cache scatter or SwiGLU, so both the CPU
oracle (``oracle/``) and the HIP library can consume what it produces
without sharing any of the method's code.

All draws use a CPU ``torch.Generator`` with an explicit seed, so the same
call gives the same bits on any machine. Values are drawn in float32 and
rounded to the storage dtype by torch's round-to-nearest-even cast.

Shapes follow the workloads the pages describe:
  * Qwen2.5-1.5B decode shapes (hidden 1536, 12 query heads, 2 KV heads,
    28 layers) from the koas-w.github.io 2026-03-31 post, sections 1 and 3;
  * head_dim 128, intermediate 8960, RoPE base 1e6, eps 1e-6 and block size
    16 are the Qwen2.5-1.5B model constants (the pages do not print them);
  * the FlashAttention paged-cache layout [2, num_blocks, block_size,
    kv_heads, head_dim] from mer.dev "AsyncT vLLM notes (1)", section 1.1;
  * slots from block tables as block * block_size + offset, as in section 1.4
    (Vectorized Gather) of the same page.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Qwen2.5-1.5B shapes.
HIDDEN = 1536
N_HEAD = 12
N_KV_HEAD = 2
HEAD_DIM = 128
INTER = 8960
N_LAYERS = 28
ROPE_THETA = 1.0e6
EPS = 1.0e-6
BLOCK_SIZE = 16

# Fill pattern for cache bytes that a call must leave alone: all-ones bits,
# a NaN in bf16, fp16 and fp32, so an accidental read-modify-write shows up.
SENTINEL_BITS = {torch.bfloat16: 0xFFFF, torch.float16: 0xFFFF, torch.float32: 0xFFFFFFFF}

_DT = {"bf16": torch.bfloat16, "f32": torch.float32, "f16": torch.float16,
       torch.bfloat16: torch.bfloat16, torch.float32: torch.float32, torch.float16: torch.float16}


def as_dtype(dt) -> torch.dtype:
    return _DT[dt]


def gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(shape, g: torch.Generator, std: float = 1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def sentinel_cache(shape, dtype) -> torch.Tensor:
    """A cache tensor whose every element holds the all-ones bit pattern."""
    dtype = as_dtype(dtype)
    t = torch.empty(shape, dtype=dtype)
    if dtype.itemsize == 2:
        t.view(torch.int16).fill_(-1)
    else:
        t.view(torch.int32).fill_(-1)
    return t


# ---------------------------------------------------------------- RMSNorm
def rmsnorm_rows(rows: int = 512, d: int = 2176, dtype="bf16", seed: int = 0,
                 outlier_frac: float = 0.01, outlier_scale: float = 100.0):
    """x ~ N(0,1) with round(outlier_frac*rows) rows scaled by outlier_scale
    (chosen by a seeded permutation), w ~ U(0.5, 1.5), eps 1e-6."""
    dt = as_dtype(dtype)
    g = gen(seed)
    x = randn([rows, d], g)
    n_out = int(round(outlier_frac * rows))
    out_rows = torch.randperm(rows, generator=g)[:n_out] if n_out else torch.empty(0, dtype=torch.long)
    if n_out:
        x[out_rows] *= outlier_scale
    w = 0.5 + torch.rand([d], generator=g, dtype=torch.float32)
    return dict(x=x.to(dt), w=w.to(dt), eps=EPS, outlier_rows=out_rows)


def norm_weight(d: int, g: torch.Generator, dtype) -> torch.Tensor:
    """Norm weight 1 + 0.1 N(0,1), the shape of a trained RMSNorm gain."""
    return (1.0 + 0.1 * randn([d], g)).to(as_dtype(dtype))


def add_rmsnorm_rows(rows: int, d: int, dtype="bf16", seed: int = 0):
    dt = as_dtype(dtype)
    g = gen(seed)
    x = randn([rows, d], g).to(dt)
    delta = randn([rows, d], g).to(dt)
    w = norm_weight(d, g, dt)
    return dict(x=x, delta=delta, w=w, eps=EPS)


# ----------------------------------------------------------- RoPE + cache
@dataclass
class PagedBatch:
    """Sequences laid out in a paged KV cache."""
    lens: list
    positions: torch.Tensor          # [T] int64
    slot_mapping: torch.Tensor       # [T] int64
    block_tables: list               # per sequence: LongTensor of physical block ids
    num_blocks: int
    block_size: int
    spare_blocks: torch.Tensor = field(default_factory=lambda: torch.empty(0, dtype=torch.long))


def paged_layout(lens, block_size: int, g: torch.Generator, spare: int = 64,
                 new_token_only: bool = False) -> PagedBatch:
    """Physical blocks are a seeded random permutation handed out in sequence
    order; ``spare`` extra blocks are never named by any slot.

    With ``new_token_only`` each sequence contributes one token, the one at
    position len-1 (a decode step whose earlier context is already cached);
    otherwise every position 0..len-1 is a token (prefill).
    """
    nb_seq = [math.ceil(L / block_size) for L in lens]
    n_used = sum(nb_seq)
    num_blocks = n_used + spare
    perm = torch.randperm(num_blocks, generator=g)
    tables, pos_l, slot_l = [], [], []
    off = 0
    for L, nb in zip(lens, nb_seq):
        bt = perm[off:off + nb]
        off += nb
        tables.append(bt)
        p = torch.arange(L - 1, L) if new_token_only else torch.arange(L)
        pos_l.append(p)
        slot_l.append(bt[p // block_size] * block_size + p % block_size)
    return PagedBatch(lens=list(lens), positions=torch.cat(pos_l).to(torch.int64),
                      slot_mapping=torch.cat(slot_l).to(torch.int64), block_tables=tables,
                      num_blocks=num_blocks, block_size=block_size, spare_blocks=perm[off:])


def qkv_views(qkv: torch.Tensor, hq: int, hkv: int, dh: int):
    """Split a fused [T, (hq+2hkv)*dh] projection output into strided
    [T, H, dh] views of Q, K and V (no copies)."""
    q = qkv[:, : hq * dh].unflatten(1, (hq, dh))
    k = qkv[:, hq * dh:(hq + hkv) * dh].unflatten(1, (hkv, dh))
    v = qkv[:, (hq + hkv) * dh:].unflatten(1, (hkv, dh))
    return q, k, v


def prefill(n_seqs: int = 8, len_lo: int = 128, len_hi: int = 2048, dtype="bf16",
            seed: int = 0, hq: int = N_HEAD, hkv: int = N_KV_HEAD, dh: int = HEAD_DIM,
            block_size: int = BLOCK_SIZE, theta: float = ROPE_THETA):
    """Prefill RoPE + paged store: lengths uniform in [len_lo, len_hi]
    (inclusive), q/k/v as views of one fused projection buffer ~ N(0,1)."""
    dt = as_dtype(dtype)
    g = gen(seed)
    lens = torch.randint(len_lo, len_hi + 1, (n_seqs,), generator=g).tolist()
    layout = paged_layout(lens, block_size, g)
    T = sum(lens)
    qkv = randn([T, (hq + 2 * hkv) * dh], g).to(dt)
    q, k, v = qkv_views(qkv, hq, hkv, dh)
    cache = sentinel_cache([2, layout.num_blocks, block_size, hkv, dh], dt)
    return dict(qkv=qkv, q=q, k=k, v=v, layout=layout, positions=layout.positions,
                slot_mapping=layout.slot_mapping, cache=cache, max_pos=len_hi,
                theta=theta, hq=hq, hkv=hkv, dh=dh, block_size=block_size)


# ---------------------------------------------------------------- SwiGLU
def swiglu_fused(rows: int = 8192, inter: int = INTER, dtype="bf16", seed: int = 0,
                 std: float = 2.0):
    """Fused [rows, 2*inter] gate_up buffer (gate first), entries N(0, std^2)."""
    dt = as_dtype(dtype)
    g = gen(seed)
    gate_up = randn([rows, 2 * inter], g, std=std).to(dt)
    return dict(gate_up=gate_up, gate=gate_up[:, :inter], up=gate_up[:, inter:], inter=inter)


# ------------------------------------------------ batch-1 decode token
def decode_token(seed: int = 0, dtype="bf16"):
    """One Qwen2.5-1.5B decode token: RMSNorm of x[1,1536]; RoPE + store of
    Q[1,12,128], K/V[1,2,128] at position 37 into a 64-block cache at slot
    597; SwiGLU of gate/up[1,8960]."""
    dt = as_dtype(dtype)
    g = gen(seed)
    x = randn([1, HIDDEN], g).to(dt)
    w = norm_weight(HIDDEN, g, dt)
    q = randn([1, N_HEAD, HEAD_DIM], g).to(dt)
    k = randn([1, N_KV_HEAD, HEAD_DIM], g).to(dt)
    v = randn([1, N_KV_HEAD, HEAD_DIM], g).to(dt)
    gate = randn([1, INTER], g).to(dt)
    up = randn([1, INTER], g).to(dt)
    cache = sentinel_cache([2, 64, BLOCK_SIZE, N_KV_HEAD, HEAD_DIM], dt)
    return dict(x=x, w=w, eps=EPS, q=q, k=k, v=v, positions=torch.tensor([37], dtype=torch.int64),
                slot_mapping=torch.tensor([597], dtype=torch.int64), cache=cache, num_blocks=64,
                max_pos=64, theta=ROPE_THETA, gate=gate, up=up)


# ------------------------------------------------ batched decode chain
def decode_chain(layers: int = N_LAYERS, batch: int = 256, ctx: int = 4096, dtype="bf16",
                 seed: int = 0, hidden: int = HIDDEN, inter: int = INTER, hq: int = N_HEAD,
                 hkv: int = N_KV_HEAD, dh: int = HEAD_DIM, block_size: int = BLOCK_SIZE):
    """Per layer: add_rmsnorm(h, d_attn), rope_kvstore(qkv), add_rmsnorm(h,
    d_mlp), swiglu(gate_up). Every sequence has ``ctx`` tokens cached and
    decodes the token at position ``ctx``; each holds ceil((ctx+1)/bs)
    blocks of one random permutation, shared by all layers. Every layer has
    its own inputs, weights and cache."""
    dt = as_dtype(dtype)
    g = gen(seed)
    h = randn([batch, hidden], g).to(dt)
    per_layer = []
    for _ in range(layers):
        per_layer.append(dict(
            w_attn=norm_weight(hidden, g, dt), w_mlp=norm_weight(hidden, g, dt),
            d_attn=randn([batch, hidden], g).to(dt), d_mlp=randn([batch, hidden], g).to(dt),
            qkv=randn([batch, (hq + 2 * hkv) * dh], g).to(dt),
            gate_up=randn([batch, 2 * inter], g).to(dt)))
    layout = paged_layout([ctx + 1] * batch, block_size, g, new_token_only=True)
    return dict(h=h, layers=per_layer, layout=layout, positions=layout.positions,
                slot_mapping=layout.slot_mapping, num_blocks=layout.num_blocks,
                cache_shape=[2, layout.num_blocks, block_size, hkv, dh], max_pos=ctx + 1,
                theta=ROPE_THETA, eps=EPS, hidden=hidden, inter=inter, hq=hq, hkv=hkv, dh=dh,
                block_size=block_size, dtype=dt)

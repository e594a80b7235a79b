"""kv_cache_rmsnorm_amd -- Python binding of libkcr, the gfx950 HIP library of
fused per-token decode ops (C ABI in include/kcr.h).

This module only marshals arguments: it reads pointers, strides and the
current HIP stream off torch tensors and calls the library. Every step of
the computation runs in the library's kernels; there is no fallback path, and
importing this module fails if libkcr.so has not been built
(``python kv_cache_rmsnorm_amd/build.py``).

Ops (names as in the C ABI):
  rmsnorm(x, w, eps)                       y = x * rsqrt(mean(x^2) + eps) * w
  add_rmsnorm(x, delta, w, eps)            x <- x + delta (in place); y = rmsnorm(x) * w
  rope_kvstore(q, k, v, positions, cos, sin, kv_cache, slot_mapping)
                                           rotate-half RoPE of Q/K; q_out; K_rot, V -> cache
  swiglu(gate, up)                         silu(gate) * up
  rope_cos_sin(max_pos, head_dim, theta)   fp32 cos/sin tables built on the device
  rope_cos_sin_host(max_pos, head_dim, theta)  the same tables built on the host
  qknorm_rope_kvstore(q, k, v, wq, wk, eps, ...)  per-head Q/K RMSNorm, then rope_kvstore
  reglu(gate, up)                          relu(gate) * up
  clip_norm(x, alpha, gamma, lo, hi)       clamp(alpha * x, lo, hi) * gamma (DyHT)
  paged_kv_gather(kv_cache, block_tables, seq_lens, max_len)
                                           K, V of each sequence, read back from the cache
  DecodeChainB1(layers, h, ...)            batch-1 decode chain of every layer in one launch
  DecodeChainBatch(layers, h, ...)         the same chain for a batch of tokens in one launch
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkcr.so")

BF16, F32, F16 = 0, 1, 2
_DTYPE = {torch.bfloat16: BF16, torch.float32: F32, torch.float16: F16}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python kv_cache_rmsnorm_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

_P, _I64, _I, _F, _D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
_SIGS = {
    "kcr_rmsnorm": [_P, _I64, _P, _P, _I64, _I64, _I64, _F, _I, _P],
    "kcr_add_rmsnorm": [_P, _I64, _P, _I64, _P, _P, _I64, _I64, _I64, _F, _I, _P],
    "kcr_rope_kvstore": [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _P, _P, _P, _I64, _P,
                         _P, _I64, _I, _I, _I, _I, _I64, _I, _P],
    "kcr_qknorm_rope_kvstore": [_P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _P, _F, _P, _P,
                                _P, _P, _I64, _P, _P, _I64, _I, _I, _I, _I, _I64, _I, _P],
    "kcr_rope_cos_sin": [_P, _P, _I64, _I, _D, _P],
    "kcr_rope_cos_sin_host": [_P, _P, _I64, _I, _D],
    "kcr_swiglu": [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I, _P],
    "kcr_reglu": [_P, _I64, _P, _I64, _P, _I64, _I64, _I64, _I, _P],
    "kcr_clip_norm": [_P, _I64, _I64, _P, _I64, _I64, _I64, _I, _I, _P, _I, _P, _I, _F, _F, _I, _P],
    "kcr_paged_kv_gather": [_P, _I64, _I, _I, _I, _P, _I64, _P, _I64, _I64, _P, _P, _I, _P],
    "kcr_copy": [_P, _P, _I64, _P],
    "kcr_decode_chain_b1": [_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I64, _I, _I64, _F, _I, _P],
    "kcr_decode_chain_batch": [_P, _I, _I64, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I64, _I, _I64, _F, _I, _P],
    "kcr_time_next_launch": [_P, _P],
    "kcr_device_cus": [],
    "kcr_selftest_host": [],
}
for _name, _args in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _I
_lib.kcr_strerror.argtypes = [_I]
_lib.kcr_strerror.restype = ctypes.c_char_p
_lib.kcr_version.argtypes = []
_lib.kcr_version.restype = ctypes.c_char_p


class KcrError(RuntimeError):
    def __init__(self, op: str, status: int):
        self.status = status
        super().__init__(f"{op}: {_lib.kcr_strerror(status).decode()} (status {status})")


def _check(op: str, status: int) -> None:
    if status != 0:
        raise KcrError(op, status)


def _dt(*ts: torch.Tensor) -> int:
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt:
            raise TypeError(f"mixed dtypes {dt} and {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError("kcr ops take device tensors")
    if dt not in _DTYPE:
        raise TypeError(f"unsupported dtype {dt}")
    return _DTYPE[dt]


def _expect(cond: bool, msg: str) -> None:
    """Shape checks the C ABI cannot make: it sees only pointers, so a tensor
    smaller than the sizes passed with it would be read or written past its
    end."""
    if not cond:
        raise ValueError(msg)


def _same(a: torch.Tensor, b: torch.Tensor, what: str) -> None:
    _expect(tuple(a.shape) == tuple(b.shape), f"{what}: shape {tuple(a.shape)} != {tuple(b.shape)}")
    _expect(a.dtype == b.dtype and a.device == b.device, f"{what}: dtype/device mismatch")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _rows(t: torch.Tensor):
    """(rows, cols, row stride) of a tensor viewed as 2-D over its last dim."""
    if t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    cols = t.shape[-1]
    if t.dim() == 1:
        return 1, cols, cols
    flat = t.reshape(-1, cols) if t.dim() > 2 else t
    if flat.data_ptr() != t.data_ptr() or (t.dim() > 2 and not _uniform_rows(t)):
        raise ValueError("leading dimensions must collapse to one row stride")
    return flat.shape[0], cols, (flat.stride(0) if flat.shape[0] > 1 else cols)


def _uniform_rows(t: torch.Tensor) -> bool:
    expect = t.stride(-2)
    for i in range(t.dim() - 2, 0, -1):
        expect *= t.shape[i]
        if t.shape[i - 1] > 1 and t.stride(i - 1) != expect:
            return False
    return True


# ------------------------------------------------------------------- ops
def rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
            out: torch.Tensor | None = None) -> torch.Tensor:
    dt = _dt(x, w)
    rows, d, xs = _rows(x)
    _expect(w.dim() == 1 and w.numel() == d and w.is_contiguous(), "w must be a contiguous [d] vector")
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if out is None else out
    _same(y, x, "rmsnorm out")
    _, _, ys = _rows(y)
    _check("rmsnorm", _lib.kcr_rmsnorm(x.data_ptr(), xs, w.data_ptr(), y.data_ptr(), ys, rows, d,
                                       float(eps), dt, _stream(x)))
    return y


def add_rmsnorm(x: torch.Tensor, delta: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """x is updated in place to x + delta; returns rmsnorm(x + delta) * w."""
    dt = _dt(x, delta, w)
    rows, d, xs = _rows(x)
    _same(delta, x, "add_rmsnorm delta")
    _, _, ds = _rows(delta)
    _expect(w.dim() == 1 and w.numel() == d and w.is_contiguous(), "w must be a contiguous [d] vector")
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if out is None else out
    _same(y, x, "add_rmsnorm out")
    _, _, ys = _rows(y)
    _check("add_rmsnorm", _lib.kcr_add_rmsnorm(x.data_ptr(), xs, delta.data_ptr(), ds, w.data_ptr(),
                                               y.data_ptr(), ys, rows, d, float(eps), dt, _stream(x)))
    return y


def _rope_checks(q, k, v, positions, cos, sin, kv_cache, slot_mapping, q_out):
    dt = _dt(q, k, v, kv_cache)
    _expect(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [T, heads, head_dim]")
    T, hq, hd = q.shape
    hkv = k.shape[1]
    _expect(tuple(k.shape) == (T, hkv, hd) and tuple(v.shape) == (T, hkv, hd),
            "k and v must be [T, n_kv_head, head_dim] with q's T and head_dim")
    _expect(q.stride(2) == 1 and k.stride(2) == 1 and v.stride(2) == 1,
            "the head dimension of q, k, v must be contiguous")
    _expect(positions.dim() == 1 and positions.numel() == T and slot_mapping.dim() == 1
            and slot_mapping.numel() == T, "positions and slot_mapping must be [T]")
    _expect(positions.device == q.device and slot_mapping.device == q.device and cos.device == q.device
            and sin.device == q.device, "all tensors must be on q's device")
    _expect(cos.dim() == 2 and cos.shape[1] == hd // 2 and tuple(sin.shape) == tuple(cos.shape),
            "cos and sin must both be [max_pos, head_dim / 2]")
    if positions.dtype != torch.int64 or slot_mapping.dtype != torch.int64:
        raise TypeError("positions and slot_mapping must be int64")
    if cos.dtype != torch.float32 or sin.dtype != torch.float32:
        raise TypeError("cos/sin tables must be float32")
    if not (cos.is_contiguous() and sin.is_contiguous() and kv_cache.is_contiguous()
            and positions.is_contiguous() and slot_mapping.is_contiguous()):
        raise ValueError("tables, cache, positions and slot_mapping must be contiguous")
    if kv_cache.dim() != 5 or kv_cache.shape[0] != 2 or tuple(kv_cache.shape[3:]) != (hkv, hd):
        raise ValueError("kv_cache must be [2, num_blocks, block_size, n_kv_head, head_dim]")
    if q_out is None:
        q_out = torch.empty((T, hq, hd), dtype=q.dtype, device=q.device)
    _expect(tuple(q_out.shape) == (T, hq, hd) and q_out.is_contiguous() and q_out.dtype == q.dtype
            and q_out.device == q.device, "q_out must be a contiguous [T, n_head, head_dim] tensor like q")
    return dt, T, hq, hkv, hd, q_out


def rope_kvstore(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, positions: torch.Tensor,
                 cos: torch.Tensor, sin: torch.Tensor, kv_cache: torch.Tensor,
                 slot_mapping: torch.Tensor, q_out: torch.Tensor | None = None) -> torch.Tensor:
    """q [T,Hq,D], k/v [T,Hkv,D] (views allowed), positions/slot_mapping [T]
    int64, cos/sin [max_pos, D/2] fp32, kv_cache [2, blocks, block_size, Hkv, D].
    Returns q_out [T,Hq,D] (contiguous); K_rot and V land in kv_cache."""
    dt, T, hq, hkv, hd, q_out = _rope_checks(q, k, v, positions, cos, sin, kv_cache, slot_mapping, q_out)
    _check("rope_kvstore", _lib.kcr_rope_kvstore(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k.stride(0), k.stride(1),
        v.data_ptr(), v.stride(0), v.stride(1), q_out.data_ptr(), positions.data_ptr(),
        cos.data_ptr(), sin.data_ptr(), cos.shape[0], kv_cache.data_ptr(), slot_mapping.data_ptr(),
        T, hq, hkv, hd, kv_cache.shape[2], kv_cache.shape[1], dt, _stream(q)))
    return q_out


def qknorm_rope_kvstore(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_norm_w: torch.Tensor,
                        k_norm_w: torch.Tensor, eps: float, positions: torch.Tensor,
                        cos: torch.Tensor, sin: torch.Tensor, kv_cache: torch.Tensor,
                        slot_mapping: torch.Tensor, q_out: torch.Tensor | None = None) -> torch.Tensor:
    """rope_kvstore with a per-head RMSNorm of every Q head (weight q_norm_w)
    and K head (weight k_norm_w) before the rotation."""
    dt, T, hq, hkv, hd, q_out = _rope_checks(q, k, v, positions, cos, sin, kv_cache, slot_mapping, q_out)
    if q_norm_w.dtype != q.dtype or k_norm_w.dtype != q.dtype:
        raise TypeError("norm weights must have the activation dtype")
    _expect(q_norm_w.numel() == hd and k_norm_w.numel() == hd and q_norm_w.is_contiguous()
            and k_norm_w.is_contiguous() and q_norm_w.device == q.device and k_norm_w.device == q.device,
            "q_norm_w and k_norm_w must be contiguous [head_dim] vectors on q's device")
    _check("qknorm_rope_kvstore", _lib.kcr_qknorm_rope_kvstore(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k.stride(0), k.stride(1),
        v.data_ptr(), v.stride(0), v.stride(1), q_norm_w.data_ptr(), k_norm_w.data_ptr(), float(eps),
        q_out.data_ptr(), positions.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0],
        kv_cache.data_ptr(), slot_mapping.data_ptr(), T, hq, hkv, hd, kv_cache.shape[2],
        kv_cache.shape[1], dt, _stream(q)))
    return q_out


def rope_cos_sin(max_pos: int, head_dim: int, theta: float, device="cuda"):
    cos = torch.empty((max_pos, head_dim // 2), dtype=torch.float32, device=device)
    sin = torch.empty_like(cos)
    _check("rope_cos_sin", _lib.kcr_rope_cos_sin(cos.data_ptr(), sin.data_ptr(), max_pos, head_dim,
                                                 float(theta), _stream(cos)))
    return cos, sin


def _gated_args(gate: torch.Tensor, up: torch.Tensor, out: torch.Tensor | None, what: str):
    dt = _dt(gate, up)
    _same(up, gate, f"{what} up")
    rows, cols, gs = _rows(gate)
    _, _, us = _rows(up)
    if out is None:
        out = torch.empty(gate.shape, dtype=gate.dtype, device=gate.device)
    _same(out, gate, f"{what} out")
    _, _, os_ = _rows(out)
    return dt, rows, cols, gs, us, out, os_


def rope_cos_sin_host(max_pos: int, head_dim: int, theta: float):
    """The cos/sin tables computed on the host: two CPU float32 tensors
    [max_pos, head_dim / 2] (copy them to the device before use)."""
    cos = torch.empty((max_pos, head_dim // 2), dtype=torch.float32)
    sin = torch.empty_like(cos)
    _check("rope_cos_sin_host", _lib.kcr_rope_cos_sin_host(cos.data_ptr(), sin.data_ptr(), max_pos,
                                                           head_dim, float(theta)))
    return cos, sin


def swiglu(gate: torch.Tensor, up: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    dt, rows, cols, gs, us, out, os_ = _gated_args(gate, up, out, "swiglu")
    _check("swiglu", _lib.kcr_swiglu(gate.data_ptr(), gs, up.data_ptr(), us, out.data_ptr(), os_,
                                     rows, cols, dt, _stream(gate)))
    return out


def reglu(gate: torch.Tensor, up: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """relu(gate) * up (same layouts as swiglu)."""
    dt, rows, cols, gs, us, out, os_ = _gated_args(gate, up, out, "reglu")
    _check("reglu", _lib.kcr_reglu(gate.data_ptr(), gs, up.data_ptr(), us, out.data_ptr(), os_,
                                   rows, cols, dt, _stream(gate)))
    return out


def clip_norm(x: torch.Tensor, alpha: torch.Tensor, gamma: torch.Tensor, lo: float = -1.0,
              hi: float = 1.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """clamp(alpha * x, lo, hi) * gamma over x [n_tok, n_head, d] (or [n, d]),
    strided views allowed; alpha/gamma are [d] (per channel) or [1]."""
    dt = _dt(x, alpha, gamma)
    if x.dim() == 2:
        x = x.unsqueeze(1)
        out = out.unsqueeze(1) if out is not None else None
        squeeze = True
    else:
        squeeze = False
    _expect(x.dim() == 3, "x must be [n_tok, n_head, d] or [n, d]")
    n, h, d = x.shape
    if x.stride(2) != 1:
        raise ValueError("the last dimension must be contiguous")
    for name, p in (("alpha", alpha), ("gamma", gamma)):
        _expect(p.numel() in (1, d) and p.is_contiguous(), f"{name} must be a contiguous [d] or [1] tensor")
    y = torch.empty((n, h, d), dtype=x.dtype, device=x.device) if out is None else out
    _same(y, x, "clip_norm out")
    _expect(y.stride(2) == 1, "the last dimension of out must be contiguous")
    _check("clip_norm", _lib.kcr_clip_norm(
        x.data_ptr(), x.stride(0), x.stride(1), y.data_ptr(), y.stride(0), y.stride(1), n, h, d,
        alpha.data_ptr(), int(alpha.numel() > 1), gamma.data_ptr(), int(gamma.numel() > 1),
        float(lo), float(hi), dt, _stream(x)))
    return y.squeeze(1) if squeeze else y


def swiglu_fused(gate_up: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """SwiGLU of a fused [..., 2*I] buffer whose first half is the gate."""
    inter = gate_up.shape[-1] // 2
    return swiglu(gate_up[..., :inter], gate_up[..., inter:], out=out)


def paged_kv_gather(kv_cache: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                    max_len: int, k_out: torch.Tensor | None = None,
                    v_out: torch.Tensor | None = None):
    """K and V of each sequence, gathered from the paged cache through its
    block table: returns (k, v), each [n_seqs, max_len, n_kv_head, head_dim].
    Rows past a sequence's length are left as allocated (uninitialized when
    the outputs are created here)."""
    dt = _dt(kv_cache)
    _expect(kv_cache.dim() == 5 and kv_cache.shape[0] == 2,
            "kv_cache must be [2, num_blocks, block_size, n_kv_head, head_dim]")
    _, nb, bs, hkv, hd = kv_cache.shape
    _expect(block_tables.dim() == 2 and seq_lens.dim() == 1 and seq_lens.numel() == block_tables.shape[0],
            "block_tables must be [n_seqs, max_blocks] and seq_lens [n_seqs]")
    _expect(block_tables.device == kv_cache.device and seq_lens.device == kv_cache.device,
            "all tensors must be on the cache's device")
    n = block_tables.shape[0]
    if block_tables.dtype != torch.int64 or seq_lens.dtype != torch.int64:
        raise TypeError("block_tables and seq_lens must be int64")
    if not (kv_cache.is_contiguous() and block_tables.is_contiguous() and seq_lens.is_contiguous()):
        raise ValueError("kv_cache, block_tables and seq_lens must be contiguous")
    shape = (n, max_len, hkv, hd)
    k_out = torch.empty(shape, dtype=kv_cache.dtype, device=kv_cache.device) if k_out is None else k_out
    v_out = torch.empty(shape, dtype=kv_cache.dtype, device=kv_cache.device) if v_out is None else v_out
    for name, o in (("k_out", k_out), ("v_out", v_out)):
        _expect(tuple(o.shape) == shape and o.is_contiguous() and o.dtype == kv_cache.dtype
                and o.device == kv_cache.device, f"{name} must be a contiguous {shape} tensor like the cache")
    _check("paged_kv_gather", _lib.kcr_paged_kv_gather(
        kv_cache.data_ptr(), nb, bs, hkv, hd, block_tables.data_ptr(), block_tables.shape[1],
        seq_lens.data_ptr(), n, max_len, k_out.data_ptr(), v_out.data_ptr(), dt, _stream(kv_cache)))
    return k_out, v_out


class ChainLayer(ctypes.Structure):
    """kcr_chain_layer: one layer's device pointers for the one-launch chain."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("d_attn", "w_attn", "y_attn", "qkv", "q_out", "kv_cache",
                                                "d_mlp", "w_mlp", "y_mlp", "gate_up", "act")]


class DecodeChainBatch:
    """Marshalled arguments of kcr_decode_chain_batch (one decode step's
    chain for a batch of tokens in one launch), checked and packed once;
    calling the object launches the step on the current stream. `h` is the
    residual [batch, hidden] (or [hidden] for one token), updated in place.
    `layers` is a list of dicts with tensors of `batch` contiguous rows:
    d_attn, y_attn, d_mlp, y_mlp [batch, hidden],
    qkv [batch, (n_head + 2 n_kv_head) * head_dim], q_out [batch, n_head, head_dim],
    gate_up [batch, 2 * inter], act [batch, inter]; and the shared
    w_attn, w_mlp [hidden] and cache [2, blocks, block_size, n_kv_head, head_dim].
    The tensors must stay alive while the object is used."""

    _op = "decode_chain_batch"

    def __init__(self, layers: list, h: torch.Tensor, positions: torch.Tensor, slot_mapping: torch.Tensor,
                 cos: torch.Tensor, sin: torch.Tensor, eps: float, n_head: int, n_kv_head: int):
        hidden = h.shape[-1]
        batch = h.numel() // hidden if hidden else 0
        _expect(h.dim() in (1, 2) and h.is_contiguous(), "h must be a contiguous [batch, hidden] tensor")
        self._check_batch(batch)
        self.dt = _dt(h)
        _expect(all(t.device == h.device for t in (positions, slot_mapping, cos, sin)),
                "positions, slot_mapping and the tables must be on h's device")
        n = len(layers)
        _expect(0 <= n <= 32, "at most 32 layers")
        _expect(cos.dim() == 2 and cos.dtype == torch.float32 and sin.dtype == torch.float32
                and tuple(sin.shape) == tuple(cos.shape) and cos.is_contiguous() and sin.is_contiguous(),
                "cos/sin must be contiguous float32 [max_pos, head_dim / 2]")
        head_dim = cos.shape[1] * 2
        _expect(positions.dtype == torch.int64 and slot_mapping.dtype == torch.int64
                and positions.numel() == batch and slot_mapping.numel() == batch
                and positions.is_contiguous() and slot_mapping.is_contiguous(),
                f"positions and slot_mapping must be contiguous int64 [{batch}]")
        self.table = (ChainLayer * max(n, 1))()
        inter = nb = bs = 0
        for i, L in enumerate(layers):
            cache = L["cache"]
            _expect(cache.dim() == 5 and cache.shape[0] == 2 and cache.shape[3] == n_kv_head
                    and cache.shape[4] == head_dim and cache.is_contiguous() and cache.dtype == h.dtype
                    and cache.device == h.device,
                    "cache must be a contiguous [2, blocks, block_size, n_kv_head, head_dim] tensor like h")
            if i and (cache.shape[1], cache.shape[2], L["act"].shape[-1]) != (nb, bs, inter):
                raise ValueError("every layer must have the same cache shape and intermediate size")
            nb, bs, inter = cache.shape[1], cache.shape[2], L["act"].shape[-1]
            per_tok = dict(d_attn=hidden, y_attn=hidden, d_mlp=hidden, y_mlp=hidden,
                           qkv=(n_head + 2 * n_kv_head) * head_dim, q_out=n_head * head_dim,
                           gate_up=2 * inter, act=inter)
            sizes = dict(w_attn=hidden, w_mlp=hidden, **{k: batch * v for k, v in per_tok.items()})
            for name, size in sizes.items():
                t = L[name]
                _expect(t.numel() == size and t.is_contiguous() and t.dtype == h.dtype and t.device == h.device,
                        f"layer {i} {name} must be a contiguous {size}-element tensor like h")
            self.table[i] = ChainLayer(*[L[f].data_ptr() for f in ("d_attn", "w_attn", "y_attn", "qkv", "q_out")],
                                       cache.data_ptr(),
                                       *[L[f].data_ptr() for f in ("d_mlp", "w_mlp", "y_mlp", "gate_up", "act")])
        self.h = h
        self.batch = batch
        self.args = (ctypes.cast(self.table, ctypes.c_void_p), n, h.data_ptr(), hidden, inter, n_head, n_kv_head,
                     head_dim, positions.data_ptr(), slot_mapping.data_ptr(), cos.data_ptr(), sin.data_ptr(),
                     cos.shape[0], bs, nb, float(eps), self.dt)
        self.n = n

    @staticmethod
    def _check_batch(batch: int) -> None:
        pass

    def _launch(self) -> int:
        return _lib.kcr_decode_chain_batch(self.args[0], self.args[1], self.batch, *self.args[2:],
                                           _stream(self.h))

    def __call__(self) -> None:
        if self.n and self.batch:
            _check(self._op, self._launch())


class DecodeChainB1(DecodeChainBatch):
    """The batch-1 form through kcr_decode_chain_b1: h is one row ([hidden]
    or [1, hidden]) and every per-token tensor holds one token."""

    _op = "decode_chain_b1"

    @staticmethod
    def _check_batch(batch: int) -> None:
        _expect(batch == 1, "h must be one contiguous row")

    def _launch(self) -> int:
        return _lib.kcr_decode_chain_b1(*self.args, _stream(self.h))


def decode_chain_b1(layers: list, h: torch.Tensor, positions: torch.Tensor, slot_mapping: torch.Tensor,
                    cos: torch.Tensor, sin: torch.Tensor, eps: float, n_head: int, n_kv_head: int) -> None:
    """One call of kcr_decode_chain_b1 (see DecodeChainB1)."""
    DecodeChainB1(layers, h, positions, slot_mapping, cos, sin, eps, n_head, n_kv_head)()


def decode_chain_batch(layers: list, h: torch.Tensor, positions: torch.Tensor, slot_mapping: torch.Tensor,
                       cos: torch.Tensor, sin: torch.Tensor, eps: float, n_head: int, n_kv_head: int) -> None:
    """One call of kcr_decode_chain_batch (see DecodeChainBatch)."""
    DecodeChainBatch(layers, h, positions, slot_mapping, cos, sin, eps, n_head, n_kv_head)()


def copy_(dst: torch.Tensor, src: torch.Tensor) -> torch.Tensor:
    """Plain 16-byte streaming copy of src's bytes into dst (bandwidth probe)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("copy_ needs contiguous tensors, dst at least as large as src")
    _expect(dst.device.type == "cuda" and src.device == dst.device, "copy_ takes two tensors on one device")
    _check("copy", _lib.kcr_copy(dst.data_ptr(), src.data_ptr(), n, _stream(src)))
    return dst


def time_next_launch(start: torch.cuda.Event, stop: torch.cuda.Event) -> None:
    """Arm a pair of timing events (already recorded once, so that they
    exist) to be stamped at the start and end of the calling thread's next
    kcr kernel; start.elapsed_time(stop) is then that kernel's duration."""
    _check("time_next_launch", _lib.kcr_time_next_launch(start.cuda_event, stop.cuda_event))


def device_cus() -> int:
    return _lib.kcr_device_cus()


def selftest_host() -> int:
    return _lib.kcr_selftest_host()


def version() -> str:
    return _lib.kcr_version().decode()


def raw_lib():
    """The ctypes handle of libkcr.so, for callers that drive the C ABI directly."""
    return _lib

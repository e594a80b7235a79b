"""CPU fp64 oracle for RMSNorm, add+RMSNorm, RoPE + paged KV store and SwiGLU.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the library in
``kv_cache_rmsnorm_amd`` never does and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, built with
gcc). This module only marshals numpy arrays into it. bf16 data travels as
its raw uint16 bit patterns, fp16 as numpy float16 (only stored and passed on,
never used for arithmetic here), fp32 as float32.

Parity of every function is pinned in the CPU tests (closed forms,
invariants, hand-worked cases in ``tests/golden`` and independent library
cross-checks); none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

BF16, F32, F16 = 0, 1, 2
_STORE = {BF16: np.uint16, F32: np.float32, F16: np.float16}
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    c = ctypes
    P, I64, D, I = c.c_void_p, c.c_int64, c.c_double, c.c_int
    sig = {
        "orc_encode": (None, [P, P, I64, I]),
        "orc_decode": (None, [P, P, I64, I]),
        "orc_num_threads": (I, []),
        "orc_set_num_threads": (None, [I]),
        "orc_rmsnorm": (None, [P, I64, P, P, I64, I64, I64, D, I]),
        "orc_add_rmsnorm": (None, [P, I64, P, I64, P, P, I64, I64, I64, D, I]),
        "orc_rope_angles": (None, [P, P, I64, I, D]),
        "orc_rope_kvstore": (None, [P, I64, I64, P, I64, I64, P, I64, I64, P, D, P, P, P, P,
                                    I64, I, I, I, I, I64, I]),
        "orc_qknorm_rope_kvstore": (None, [P, I64, I64, P, I64, I64, P, I64, I64, P, P, D, P, D, P,
                                           P, P, P, I64, I, I, I, I, I64, I]),
        "orc_gqa_kv_head": (I, [I, I, I]),
        "orc_paged_gather": (None, [P, I, P, I64, I, I, I, I64, P, I]),
        "orc_swiglu": (None, [P, I64, P, I64, P, I64, I64, I64, I]),
        "orc_reglu": (None, [P, I64, P, I64, P, I64, I64, I64, I]),
        "orc_clip_norm": (None, [P, I64, I64, P, I, P, I, D, D, P, I64, I, I, I]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def lib(path: str | None = None):
    """Load the oracle library, building it first if it is not there."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


# ------------------------------------------------------------ marshalling
def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"oracle takes bf16 bits (uint16), float16 or float32, got {a.dtype}")


def _rows(a: np.ndarray):
    """Row-major 2-D array with unit column stride -> (array, row stride)."""
    if a.ndim != 2 or a.strides[1] != a.itemsize:
        a = np.ascontiguousarray(a)
    return a, a.strides[0] // a.itemsize


def _elem_strides(a: np.ndarray):
    assert a.strides[-1] == a.itemsize, "last dim must be contiguous"
    return [s // a.itemsize for s in a.strides]


def encode(x: np.ndarray, dtype: int, L=None) -> np.ndarray:
    """Round float64 values to the storage dtype (nearest, ties to even)."""
    L = L or lib()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=_STORE[dtype])
    L.orc_encode(_ptr(x), _ptr(out), x.size, dtype)
    return out


def decode(x: np.ndarray, L=None) -> np.ndarray:
    L = L or lib()
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, dtype=np.float64)
    L.orc_decode(_ptr(x), _ptr(out), x.size, _code(x))
    return out


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float, L=None) -> np.ndarray:
    L = L or lib()
    x, xs = _rows(x)
    w = np.ascontiguousarray(w)
    rows, d = x.shape
    y = np.empty((rows, d), dtype=np.float64)
    L.orc_rmsnorm(_ptr(x), xs, _ptr(w), _ptr(y), d, rows, d, float(eps), _code(x))
    return y


def add_rmsnorm(x: np.ndarray, delta: np.ndarray, w: np.ndarray, eps: float, L=None):
    """Returns (x_new in the storage dtype, y in float64); x is not modified."""
    L = L or lib()
    xn = np.array(x, copy=True, order="C")
    delta, ds = _rows(delta)
    w = np.ascontiguousarray(w)
    rows, d = xn.shape
    y = np.empty((rows, d), dtype=np.float64)
    L.orc_add_rmsnorm(_ptr(xn), d, _ptr(delta), ds, _ptr(w), _ptr(y), d, rows, d, float(eps),
                      _code(xn))
    return xn, y


def rope_angles(max_pos: int, head_dim: int, theta: float, L=None):
    L = L or lib()
    c = np.empty((max_pos, head_dim // 2), dtype=np.float64)
    s = np.empty_like(c)
    L.orc_rope_angles(_ptr(c), _ptr(s), max_pos, head_dim, float(theta))
    return c, s


def rope_kvstore(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions: np.ndarray,
                 theta: float, cache: np.ndarray | None, slot_mapping: np.ndarray | None,
                 block_size: int = 16, L=None):
    """q [T,hq,d], k and v [T,hkv,d] (strided views allowed, last dim
    contiguous, all sharing one buffer dtype). Returns (q_rot, k_rot) in
    float64; ``cache`` [2,N,bs,hkv,d] is updated in place when given."""
    L = L or lib()
    T, hq, d = q.shape
    hkv = k.shape[1]
    assert d <= 1024
    qs, ks, vs = _elem_strides(q), _elem_strides(k), _elem_strides(v)
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    q_rot = np.empty((T, hq, d), dtype=np.float64)
    k_rot = np.empty((T, hkv, d), dtype=np.float64)
    if cache is not None:
        assert cache.flags.c_contiguous and cache.dtype == q.dtype
        slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        nb = cache.shape[1]
        assert cache.shape[2] == block_size
        cptr, sptr = _ptr(cache), _ptr(slot_mapping)
    else:
        nb, cptr, sptr = 0, None, None
    L.orc_rope_kvstore(_ptr(q), qs[0], qs[1], _ptr(k), ks[0], ks[1], _ptr(v), vs[0], vs[1],
                       _ptr(positions), float(theta), _ptr(q_rot), _ptr(k_rot), cptr, sptr,
                       T, hq, hkv, d, block_size, nb, _code(q))
    return q_rot, k_rot


def qknorm_rope_kvstore(q, k, v, q_w, k_w, eps, positions, theta, cache, slot_mapping,
                        block_size: int = 16, L=None):
    """As rope_kvstore, with per-head RMSNorm of every Q head (weight q_w) and
    K head (weight k_w) before the rotation. Returns (q_rot, k_rot)."""
    L = L or lib()
    T, hq, d = q.shape
    hkv = k.shape[1]
    assert d <= 1024
    qs, ks, vs = _elem_strides(q), _elem_strides(k), _elem_strides(v)
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    q_w, k_w = np.ascontiguousarray(q_w), np.ascontiguousarray(k_w)
    q_rot = np.empty((T, hq, d), dtype=np.float64)
    k_rot = np.empty((T, hkv, d), dtype=np.float64)
    if cache is not None:
        assert cache.flags.c_contiguous and cache.dtype == q.dtype and cache.shape[2] == block_size
        slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        nb, cptr, sptr = cache.shape[1], _ptr(cache), _ptr(slot_mapping)
    else:
        nb, cptr, sptr = 0, None, None
    L.orc_qknorm_rope_kvstore(_ptr(q), qs[0], qs[1], _ptr(k), ks[0], ks[1], _ptr(v), vs[0], vs[1],
                              _ptr(q_w), _ptr(k_w), float(eps), _ptr(positions), float(theta),
                              _ptr(q_rot), _ptr(k_rot), cptr, sptr, T, hq, hkv, d, block_size, nb,
                              _code(q))
    return q_rot, k_rot


def gqa_kv_head(h: int, hq: int, hkv: int, L=None) -> int:
    return (L or lib()).orc_gqa_kv_head(h, hq, hkv)


def paged_gather(cache: np.ndarray, which: int, block_table: np.ndarray, n_tok: int, L=None):
    L = L or lib()
    _, nb, bs, hkv, d = cache.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int64)
    out = np.empty((n_tok, hkv, d), dtype=cache.dtype)
    L.orc_paged_gather(_ptr(cache), which, _ptr(bt), n_tok, hkv, d, bs, nb, _ptr(out),
                       _code(cache))
    return out


def swiglu(gate: np.ndarray, up: np.ndarray, L=None) -> np.ndarray:
    L = L or lib()
    gate, gs = _rows(gate)
    up, us = _rows(up)
    rows, cols = gate.shape
    out = np.empty((rows, cols), dtype=np.float64)
    L.orc_swiglu(_ptr(gate), gs, _ptr(up), us, _ptr(out), cols, rows, cols, _code(gate))
    return out


def reglu(gate: np.ndarray, up: np.ndarray, L=None) -> np.ndarray:
    L = L or lib()
    gate, gs = _rows(gate)
    up, us = _rows(up)
    rows, cols = gate.shape
    out = np.empty((rows, cols), dtype=np.float64)
    L.orc_reglu(_ptr(gate), gs, _ptr(up), us, _ptr(out), cols, rows, cols, _code(gate))
    return out


def clip_norm(x: np.ndarray, alpha: np.ndarray, gamma: np.ndarray, lo: float = -1.0,
              hi: float = 1.0, L=None) -> np.ndarray:
    """x [n_tok, n_head, d] (strided views allowed, last dim contiguous);
    alpha and gamma are [d] (per channel) or [1] (scalar). Returns float64."""
    L = L or lib()
    n_tok, n_head, d = x.shape
    xs = _elem_strides(x)
    alpha, gamma = np.ascontiguousarray(alpha), np.ascontiguousarray(gamma)
    y = np.empty((n_tok, n_head, d), dtype=np.float64)
    L.orc_clip_norm(_ptr(x), xs[0], xs[1], _ptr(alpha), int(alpha.size > 1), _ptr(gamma),
                    int(gamma.size > 1), float(lo), float(hi), _ptr(y), n_tok, n_head, d, _code(x))
    return y


def num_threads(L=None) -> int:
    return (L or lib()).orc_num_threads()


def set_num_threads(n: int, L=None) -> None:
    (L or lib()).orc_set_num_threads(int(n))

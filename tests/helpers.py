"""Test-side helpers: bit views between torch and numpy, and the comparison
rules shared by the parity tests.

Comparison rules (bf16, fp16 and fp32 outputs against the fp64 oracle):
  * bf16: |gpu - ref| <= 2 * ulp_bf16(ref)  or  |gpu - ref| <= 1e-2, with
    ulp_bf16(y) = 2^(floor(log2|y|) - 7) (2^-133 at the bottom of the range);
  * fp16: |gpu - ref| <= 2 * ulp_f16(ref), ulp_f16(y) = 2^(max(floor(log2|y|),
    -14) - 10): the kernels compute in fp32 (relative error ~1e-6 here) and
    round once, so they land within one fp16 ulp; the second ulp is margin;
  * fp32: |gpu - ref| <= 1e-5 * |ref|, with an absolute floor at the fp32
    normal minimum (1.2e-38) for results that underflow;
  * integer, index and copied data: bit-exact;
  * +0 and -0 compare equal.
Pure relative error is never used on its own: it explodes near zero.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

BF16_ATOL = 1e-2
BF16_ULPS = 2.0
F16_ULPS = 2.0
F32_RTOL = 1e-5
F32_FLOOR = 1.1754943508222875e-38


def np_bits(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy view in the oracle's storage convention (bf16 as
    uint16 bit patterns, fp16 as float16, fp32 as float32); strides are kept."""
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.float16):
        return t.numpy()
    raise TypeError(t.dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.exp2(e - 7.0), 2.0 ** -133)


def ulp_f16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e, -14.0) - 10.0)


def tol_violations(got: np.ndarray, ref: np.ndarray, dtype) -> np.ndarray:
    """Boolean mask of elements outside the tolerance for ``dtype``."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    if dtype in (torch.bfloat16, "bf16"):
        ok = (err <= BF16_ULPS * ulp_bf16(ref)) | (err <= BF16_ATOL)
    elif dtype in (torch.float16, "f16"):
        ok = err <= F16_ULPS * ulp_f16(ref)
    else:
        ok = err <= np.maximum(F32_RTOL * np.abs(ref), F32_FLOOR)
    ok |= (got == ref)  # covers matching infinities
    return ~ok


def assert_close(got, ref, dtype, what: str = ""):
    bad = tol_violations(got, ref, dtype)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        g = np.asarray(got, dtype=np.float64)
        r = np.asarray(ref, dtype=np.float64)
        msg = ", ".join(f"{tuple(i)}: got {g[tuple(i)]!r} ref {r[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; {msg}")


def assert_bits_equal(a: torch.Tensor, b: torch.Tensor, what: str = ""):
    ia = a.detach().cpu().contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.detach().cpu().contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    ne = ia != ib
    if bool(ne.any()):
        idx = ne.nonzero()[:5].tolist()
        raise AssertionError(f"{what}: {int(ne.sum())} elements differ bitwise, first at {idx}")


# ------------------------------------------------------- RoPE + KV store
def dev(t):
    return t.to("cuda")


def gpu_qkv(wl):
    """Device q/k/v: narrow views of one fused device QKV buffer when the
    workload has one, else contiguous copies."""
    if "qkv" in wl:
        return workloads.qkv_views(dev(wl["qkv"]), wl["hq"], wl["hkv"], wl["dh"])
    return dev(wl["q"]), dev(wl["k"]), dev(wl["v"])


def assert_rope_close(got, ref, dt, what):
    """bf16: the common rule. fp32: |got - ref| <= 1e-5 * the norm of the
    rotation pair (i, i + d/2), which the rotation preserves; a relative
    bound per element would be meaningless where x_i c - x_{i+d/2} s
    cancels. fp16: 2 fp16 ulps of the result plus the fp32 pair-norm term
    (the rotation is done in fp32 and rounded once)."""
    if dt == torch.bfloat16:
        assert_close(got, ref, dt, what)
        return
    half = ref.shape[-1] // 2
    pn = np.sqrt(ref[..., :half] ** 2 + ref[..., half:] ** 2)
    scale = np.concatenate([pn, pn], axis=-1)
    err = np.abs(got - ref)
    bound = np.maximum(1e-5 * scale, 1.2e-38)
    if dt == torch.float16:
        bound = bound + F16_ULPS * ulp_f16(ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outside 1e-5 of the pair norm, max {err.max()}"


def check_rope(q, k, v, positions, cache0, slots, theta, q_gpu, cache_gpu, dt, what):
    """q_out within tolerance; cache: V rows and untouched bytes bit-exact,
    K rows within tolerance."""
    cache_ref = np_bits(cache0).copy()
    q_rot, k_rot = oracle.rope_kvstore(np_bits(q), np_bits(k), np_bits(v), positions.numpy(), theta,
                                       cache_ref, slots.numpy(), block_size=cache0.shape[2])
    assert_rope_close(q_gpu.double().numpy(), q_rot, dt, f"{what}: q_out")
    got = np_bits(cache_gpu)
    nb, bs, hkv, d = cache0.shape[1:]
    live = slots.numpy()
    live = live[(live >= 0) & (live < nb * bs)]
    g_flat, r_flat = got.reshape(2, nb * bs, hkv, d), cache_ref.reshape(2, nb * bs, hkv, d)
    # everything except the K rows of live slots: bit-exact (V rows, untouched sentinel)
    mask = np.ones((nb * bs,), dtype=bool)
    mask[live] = False
    assert np.array_equal(g_flat[1].view(np.uint8), r_flat[1].view(np.uint8)), f"{what}: V half"
    assert np.array_equal(g_flat[0][mask].view(np.uint8), r_flat[0][mask].view(np.uint8)), \
        f"{what}: untouched K slots"
    # K rows of live slots against the fp64 rotation
    tok = {int(s): t for t, s in enumerate(slots.numpy()) if 0 <= s < nb * bs}
    order = np.array([tok[int(s)] for s in live], dtype=np.int64)
    kg = torch.from_numpy(g_flat[0][live].view(np.int16 if dt.itemsize == 2 else np.int32).copy())
    kg = kg.view(dt).double().numpy()
    assert_rope_close(kg, k_rot[order], dt, f"{what}: K rows")



"""Test-side helpers: bit views between torch and numpy, and the comparison
rules shared by the parity tests.

Comparison rules (bf16 and fp32 outputs against the fp64 oracle):
  * bf16: |gpu - ref| <= 2 * ulp_bf16(ref)  or  |gpu - ref| <= 1e-2, with
    ulp_bf16(y) = 2^(floor(log2|y|) - 7) (2^-133 at the bottom of the range);
  * fp32: |gpu - ref| <= 1e-5 * |ref|, with an absolute floor at the fp32
    normal minimum (1.2e-38) for results that underflow;
  * integer, index and copied data: bit-exact;
  * +0 and -0 compare equal.
Pure relative error is never used on its own: it explodes near zero.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_ATOL = 1e-2
BF16_ULPS = 2.0
F32_RTOL = 1e-5
F32_FLOOR = 1.1754943508222875e-38


def np_bits(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy view in the oracle's storage convention (bf16 as
    uint16 bit patterns, fp32 as float32); strides are kept."""
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.exp2(e - 7.0), 2.0 ** -133)


def tol_violations(got: np.ndarray, ref: np.ndarray, dtype) -> np.ndarray:
    """Boolean mask of elements outside the tolerance for ``dtype``."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    if dtype in (torch.bfloat16, "bf16"):
        ok = (err <= BF16_ULPS * ulp_bf16(ref)) | (err <= BF16_ATOL)
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

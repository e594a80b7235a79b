"""Pins for the CPU oracle: each check ties one oracle function to something
other than itself -- a hand-worked case from tests/golden (each with its
citation), a closed form, an invariant, or an independent library routine
(torch's float64 rms_norm and silu, numpy complex rotation, numpy advanced
indexing, torch's fp32 -> bf16 rounding).

Every check takes the oracle library handle, so the same checks run against
the real build (test_oracle_pins.py) and against deliberately broken copies
(test_oracle_mutants.py), which shows that a plausible mistake anywhere in
the oracle fails at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads
from helpers import np_bits

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BF16, F32, F16 = oracle.BF16, oracle.F32, oracle.F16
TORCH_DT = {BF16: torch.bfloat16, F32: torch.float32, F16: torch.float16}
DTS = (F32, BF16, F16)


def golden(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def enc(values, dt) -> np.ndarray:
    """Inputs are encoded with torch (independent of the oracle's codec)."""
    return np_bits(torch.tensor(np.asarray(values, dtype=np.float64)).to(TORCH_DT[dt]))


def dec(bits: np.ndarray) -> np.ndarray:
    """Decode with torch (independent of the oracle's codec)."""
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    return bits.astype(np.float64)


def rand_rows(rows, d, dt, seed, scale=1.0):
    g = workloads.gen(seed)
    return np_bits((workloads.randn([rows, d], g) * scale).to(TORCH_DT[dt]))


# ------------------------------------------------------------- codec pins
def pin_encode_golden(L):
    for c in golden("bf16_rounding.json")["cases"]:
        v = float.fromhex(c["value"])
        got = int(oracle.encode(np.array([v]), BF16, L=L)[0])
        assert got == int(c["bits"], 16), (c["value"], hex(got), c["bits"])


def pin_encode_vs_torch(L):
    # Random float32 values, subnormals and exact ties included: torch's
    # float32 -> bf16 cast rounds to nearest even in one step.
    g = torch.Generator().manual_seed(1)
    bits = torch.randint(-2**31, 2**31 - 1, (200000,), generator=g, dtype=torch.int64).to(torch.int32)
    f = bits.view(torch.float32)
    f = f[torch.isfinite(f)]
    ties = (torch.randint(0, 2**15, (5000,), generator=g, dtype=torch.int32) << 16 | 0x8000).view(torch.float32)
    f = torch.cat([f, ties[torch.isfinite(ties)], torch.tensor([1e-40, -3e-39, 0.0, -0.0])])
    want = np_bits(f.to(torch.bfloat16))
    got = oracle.encode(f.double().numpy(), BF16, L=L)
    assert np.array_equal(got, want), int((got != want).sum())


def pin_encode_f32_vs_numpy(L):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-140, 120, 100000))
    got = oracle.encode(x, F32, L=L)
    assert np.array_equal(got.view(np.uint32), x.astype(np.float32).view(np.uint32))


def pin_decode_known(L):
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, math.inf, -0.0, 3.140625]
    got = oracle.decode(bits, L=L)
    assert list(got) == want and math.copysign(1, got[4]) == -1


def pin_f16_decode_every_pattern(L):
    # All 65536 binary16 patterns against numpy's float16 widening.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    got = oracle.decode(h, L=L)
    want = h.astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), want[~nan].view(np.uint64))


def pin_f16_encode_vs_numpy(L):
    # numpy rounds float64 -> float16 to nearest even in one step; the values
    # span the subnormals, the normals and the overflow threshold.
    rng = np.random.default_rng(21)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-30, 18, 200000))
    x = np.concatenate([x, [65519.99, 65520.0, -65520.0, 2.0 ** -25, 2.0 ** -26, 1e-9, -0.0]])
    got = oracle.encode(x, F16, L=L)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def pin_f16_ties_closed_form(L):
    # Exact midpoints between neighbouring finite binary16 values go to the
    # one with an even last bit; a nudge of one part in 2^30 either way goes
    # to the nearer neighbour. Built from the bit patterns alone.
    pos = np.arange(0, 0x7C00, dtype=np.uint32)
    lo = pos[:-1].astype(np.uint16).view(np.float16).astype(np.float64)
    hi = pos[1:].astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2                      # exact in float64
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:]).astype(np.uint16)
    assert np.array_equal(oracle.encode(mid, F16, L=L).view(np.uint16), even)
    assert np.array_equal(oracle.encode(-mid, F16, L=L).view(np.uint16), even | 0x8000)
    gap = hi - lo
    assert np.array_equal(oracle.encode(mid - gap * 2.0 ** -30, F16, L=L).view(np.uint16),
                          pos[:-1].astype(np.uint16))
    assert np.array_equal(oracle.encode(mid + gap * 2.0 ** -30, F16, L=L).view(np.uint16),
                          pos[1:].astype(np.uint16))
    # 65504 is the largest finite value; its midpoint to 2^16 rounds to inf
    top = oracle.encode(np.array([65504.0, 65519.0, 65520.0, math.inf, -math.inf]), F16, L=L)
    assert list(top.view(np.uint16)) == [0x7BFF, 0x7BFF, 0x7C00, 0x7C00, 0xFC00]
    assert np.isnan(oracle.encode(np.array([math.nan]), F16, L=L)[0])


# ----------------------------------------------------------- RMSNorm pins
def pin_rmsnorm_golden(L):
    for c in golden("rmsnorm_hand.json")["cases"]:
        for dt in DTS:
            y = oracle.rmsnorm(enc([c["x"]], dt), enc(c["w"], dt), c["eps"], L=L)
            assert np.allclose(y[0], c["y"], rtol=1e-14, atol=0), (c, y)


def pin_rmsnorm_meansq_closed_form(L):
    # Unit weight: y = x / sqrt(ms + eps), so mean(y^2) = ms / (ms + eps).
    for dt in DTS:
        x = rand_rows(16, 2176, dt, seed=3)
        xd = dec(x)
        for eps in (0.5, 1e-6):
            y = oracle.rmsnorm(x, enc(np.ones(2176), dt), eps, L=L)
            ms = np.mean(xd ** 2, axis=1)
            assert np.allclose(np.mean(y ** 2, axis=1), ms / (ms + eps), rtol=1e-12)


def pin_rmsnorm_constant_row(L):
    for dt in DTS:
        for c in (0.75, -3.0, 100.0):
            w = enc(np.linspace(0.5, 1.5, 37), dt)
            y = oracle.rmsnorm(enc(np.full((1, 37), c), dt), w, 0.25, L=L)
            assert np.allclose(y[0], c / math.sqrt(c * c + 0.25) * dec(w), rtol=1e-14)


def pin_rmsnorm_scale_invariance(L):
    x = rand_rows(8, 1000, F32, seed=4)
    w = enc(np.linspace(-1, 2, 1000), F32)
    y1 = oracle.rmsnorm(x, w, 1e-3, L=L)
    y2 = oracle.rmsnorm((x * np.float32(4)).astype(np.float32), w, 16e-3, L=L)
    assert np.allclose(y1, y2, rtol=1e-13, atol=0)


def pin_rmsnorm_vs_torch(L):
    for dt in DTS:
        for d in (1, 7, 1536, 2176):
            x = rand_rows(9, d, dt, seed=5 + d, scale=3.0)
            w = enc(1 + 0.1 * np.random.default_rng(d).standard_normal(d), dt)
            y = oracle.rmsnorm(x, w, 1e-6, L=L)
            ref = F.rms_norm(torch.from_numpy(dec(x)), (d,), torch.from_numpy(dec(w)), eps=1e-6)
            assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-300)


def pin_rmsnorm_row_stride(L):
    big = rand_rows(6, 300, BF16, seed=6)
    view = big[:, :257]
    w = enc(np.ones(257), BF16)
    assert np.array_equal(oracle.rmsnorm(view, w, 1e-6, L=L),
                          oracle.rmsnorm(np.ascontiguousarray(view), w, 1e-6, L=L))


# ------------------------------------------------------ add + RMSNorm pins
def pin_add_rmsnorm_zero_delta(L):
    for dt in DTS:
        x = rand_rows(5, 1536, dt, seed=7)
        w = enc(1 + 0.1 * np.random.default_rng(7).standard_normal(1536), dt)
        zero = enc(np.zeros((5, 1536)), dt)
        xn, y = oracle.add_rmsnorm(x, zero, w, 1e-6, L=L)
        assert np.array_equal(xn.view(np.uint8), x.view(np.uint8))
        ref = F.rms_norm(torch.from_numpy(dec(x)), (1536,), torch.from_numpy(dec(w)), eps=1e-6)
        assert np.allclose(y, ref.numpy(), rtol=1e-12)


def pin_add_rmsnorm_sum_rounding(L):
    # x_new = round(x + delta): for two bf16 (or fp32) inputs torch's float32
    # add is exact or rounds far from a bf16 tie, so the fp32 add followed by
    # torch's bf16 cast is an independent route to the same bits.
    for dt in DTS:
        x = rand_rows(7, 2048, dt, seed=8)
        dl = rand_rows(7, 2048, dt, seed=9, scale=0.01)
        xn, _ = oracle.add_rmsnorm(x, dl, enc(np.ones(2048), dt), 1e-6, L=L)
        want = (torch.from_numpy(dec(x)).float() + torch.from_numpy(dec(dl)).float()).to(TORCH_DT[dt])
        assert np.array_equal(xn, np_bits(want))


def pin_add_rmsnorm_norms_rounded_sum(L):
    # y is the norm of the stored (rounded) sum, not of the exact sum.
    x = rand_rows(4, 1536, BF16, seed=10)
    dl = rand_rows(4, 1536, BF16, seed=11, scale=0.3)
    w = enc(1 + 0.1 * np.random.default_rng(11).standard_normal(1536), BF16)
    xn, y = oracle.add_rmsnorm(x, dl, w, 1e-6, L=L)
    ref = F.rms_norm(torch.from_numpy(dec(xn)), (1536,), torch.from_numpy(dec(w)), eps=1e-6)
    assert np.allclose(y, ref.numpy(), rtol=1e-12)


def pin_add_rmsnorm_commutes(L):
    x = rand_rows(3, 999, BF16, seed=12)
    dl = rand_rows(3, 999, BF16, seed=13)
    w = enc(np.linspace(0.5, 1.5, 999), BF16)
    a = oracle.add_rmsnorm(x, dl, w, 1e-6, L=L)
    b = oracle.add_rmsnorm(dl, x, w, 1e-6, L=L)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------- RoPE pins
def _one_head(x, dt, pos, theta, L):
    d = len(x)
    q = enc(np.array(x).reshape(1, 1, d), dt)
    k = enc(np.array(x).reshape(1, 1, d), dt)
    q_rot, k_rot = oracle.rope_kvstore(q, k, k, np.array([pos]), theta, None, None, L=L)
    return q_rot[0, 0], k_rot[0, 0]


def pin_rope_golden(L):
    for c in golden("rope_hand.json")["cases"]:
        for dt in DTS:
            qr, kr = _one_head(c["x"], dt, c["pos"], c["theta"], L)
            assert np.allclose(qr, c["out"], rtol=1e-13, atol=1e-15), (c, qr)
            assert np.array_equal(qr, kr)


def _heads(T, H, d, dt, seed):
    g = workloads.gen(seed)
    return np_bits(workloads.randn([T, H, d], g).to(TORCH_DT[dt]))


def pin_rope_position_zero_identity(L):
    for dt in DTS:
        q, k = _heads(3, 12, 128, dt, 14), _heads(3, 2, 128, dt, 15)
        qr, kr = oracle.rope_kvstore(q, k, k, np.zeros(3, np.int64), 1e6, None, None, L=L)
        assert np.array_equal(qr, dec(q)) and np.array_equal(kr, dec(k))


def pin_rope_pair_norm(L):
    q, k = _heads(4, 12, 128, BF16, 16), _heads(4, 2, 128, BF16, 17)
    pos = np.array([1, 37, 4096, 131071])
    qr, _ = oracle.rope_kvstore(q, k, k, pos, 1e6, None, None, L=L)
    x = dec(q)
    n_in = x[..., :64] ** 2 + x[..., 64:] ** 2
    n_out = qr[..., :64] ** 2 + qr[..., 64:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12, atol=1e-300)


def pin_rope_vs_complex(L):
    # (x_i + i x_{i+d/2}) * exp(i p base^(-2i/d)), evaluated by numpy complex128.
    for d, theta in ((128, 1e6), (64, 1e4), (2, 10.0)):
        q, k = _heads(5, 3, d, F32, 18 + d), _heads(5, 1, d, F32, 19 + d)
        pos = np.array([0, 1, 17, 999, 65536])
        qr, _ = oracle.rope_kvstore(q, k, k, pos, theta, None, None, L=L)
        x = dec(q)
        z = x[..., : d // 2] + 1j * x[..., d // 2:]
        ang = pos[:, None, None] * theta ** (-np.arange(d // 2) * 2.0 / d)[None, None, :]
        zr = z * np.exp(1j * ang)
        want = np.concatenate([zr.real, zr.imag], axis=-1)
        assert np.allclose(qr, want, rtol=1e-10, atol=1e-12)


def pin_rope_relative_position(L):
    # <R(m) q, R(n) k> depends only on m - n.
    q, k = _heads(1, 1, 128, F32, 20), _heads(1, 1, 128, F32, 21)
    dots = []
    for m, n in ((10, 3), (110, 103), (5007, 5000)):
        qm, _ = oracle.rope_kvstore(q, k, k, np.array([m]), 1e6, None, None, L=L)
        kn, _ = oracle.rope_kvstore(k, k, k, np.array([n]), 1e6, None, None, L=L)
        dots.append(float(np.dot(qm.ravel(), kn.ravel())))
    assert np.allclose(dots, dots[0], rtol=1e-9)


def pin_rope_angle_additivity(L):
    # cos/sin tables: angle(p1 + p2) = angle(p1) + angle(p2).
    c, s = oracle.rope_angles(300, 128, 1e6, L=L)
    p1, p2 = 123, 171
    assert np.allclose(c[p1 + p2], c[p1] * c[p2] - s[p1] * s[p2], atol=1e-12)
    assert np.allclose(s[p1 + p2], s[p1] * c[p2] + c[p1] * s[p2], atol=1e-12)
    assert np.array_equal(c[0], np.ones(64)) and np.array_equal(s[0], np.zeros(64))


def pin_rope_table_matches_rotation(L):
    # Rotating the unit vector e_i yields (cos, sin) of frequency i at i and i + d/2.
    d, pos = 16, 29
    c, s = oracle.rope_angles(pos + 1, d, 1e6, L=L)
    for i in range(d // 2):
        e = np.zeros(d)
        e[i] = 1.0
        qr, _ = _one_head(e, F32, pos, 1e6, L)
        assert math.isclose(qr[i], c[pos, i], rel_tol=1e-15) and math.isclose(qr[i + d // 2], s[pos, i], rel_tol=1e-15, abs_tol=1e-300)


def pin_rope_strided_views(L):
    T, hq, hkv, d = 6, 12, 2, 128
    g = workloads.gen(22)
    qkv = workloads.randn([T, (hq + 2 * hkv) * d], g).to(torch.bfloat16)
    q, k, v = workloads.qkv_views(qkv, hq, hkv, d)
    pos = np.arange(T) * 7
    a = oracle.rope_kvstore(np_bits(q), np_bits(k), np_bits(v), pos, 1e6, None, None, L=L)
    b = oracle.rope_kvstore(np_bits(q.contiguous()), np_bits(k.contiguous()),
                            np_bits(v.contiguous()), pos, 1e6, None, None, L=L)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------ qk-norm + RoPE pins
def pin_qknorm_rope_golden(L):
    for c in golden("qknorm_rope_hand.json")["cases"]:
        for dt in DTS:
            d = len(c["x"])
            x = enc(np.array(c["x"]).reshape(1, 1, d), dt)
            w = enc(c["w"], dt)
            qr, kr = oracle.qknorm_rope_kvstore(x, x, x, w, w, c["eps"], np.array([c["pos"]]),
                                                c["theta"], None, None, L=L)
            assert np.allclose(qr[0, 0], c["out"], rtol=1e-13, atol=1e-15), (c, qr)
            assert np.array_equal(qr, kr)


def pin_qknorm_rope_energy(L):
    # Unit weight: the norm scales each head to mean square ms/(ms+eps) and the
    # rotation keeps every pair's norm, so sum(out^2) = d * ms / (ms + eps).
    q, k = _heads(3, 12, 128, BF16, 31), _heads(3, 2, 128, BF16, 32)
    ones = enc(np.ones(128), BF16)
    for eps in (0.0, 0.7):
        qr, kr = oracle.qknorm_rope_kvstore(q, k, k, ones, ones, eps, np.array([5, 900, 4096]), 1e6,
                                            None, None, L=L)
        for got, x in ((qr, dec(q)), (kr, dec(k))):
            ms = np.mean(x ** 2, axis=-1)
            assert np.allclose(np.sum(got ** 2, axis=-1), 128 * ms / (ms + eps), rtol=1e-12)


def pin_qknorm_rope_is_rope_of_rms_norm(L):
    # Position by position, the result is the complex rotation of torch's
    # float64 rms_norm of each head, with separate Q and K weights.
    T, d = 4, 64
    q, k = _heads(T, 3, d, F32, 33), _heads(T, 1, d, F32, 34)
    rng = np.random.default_rng(35)
    wq, wk = enc(1 + 0.1 * rng.standard_normal(d), F32), enc(0.5 + rng.random(d), F32)
    pos = np.array([0, 3, 77, 2048])
    qr, kr = oracle.qknorm_rope_kvstore(q, k, k, wq, wk, 1e-6, pos, 1e4, None, None, L=L)
    ang = pos[:, None, None] * 1e4 ** (-np.arange(d // 2) * 2.0 / d)[None, None, :]
    for got, x, w in ((qr, dec(q), dec(wq)), (kr, dec(k), dec(wk))):
        n = F.rms_norm(torch.from_numpy(x), (d,), torch.from_numpy(w), eps=1e-6).numpy()
        z = (n[..., : d // 2] + 1j * n[..., d // 2:]) * np.exp(1j * ang)
        assert np.allclose(got, np.concatenate([z.real, z.imag], axis=-1), rtol=1e-10, atol=1e-12)


def pin_qknorm_rope_store(L):
    # The cache holds round(normed, rotated K) at the named slots and V as is;
    # q_out and the cache image agree with the plain store for identical K.
    wl = workloads.prefill(n_seqs=2, len_lo=3, len_hi=20, seed=36)
    q, k, v = (np_bits(t) for t in (wl["q"], wl["k"], wl["v"]))
    ones = enc(np.ones(128), BF16)
    cache = np_bits(wl["cache"]).copy()
    _, k_rot = oracle.qknorm_rope_kvstore(q, k, v, ones, ones, 0.0, wl["positions"].numpy(),
                                          wl["theta"], cache, wl["slot_mapping"].numpy(), L=L)
    flat = cache.reshape(2, -1, 2, 128)
    slots = wl["slot_mapping"].numpy()
    assert np.array_equal(flat[1][slots], np.ascontiguousarray(v))
    got = dec(flat[0][slots])
    assert np.all(np.abs(got - k_rot) <= np.abs(k_rot) * 2.0 ** -8 + 1e-300)
    assert int((flat == 0xFFFF).sum()) == flat.size - 2 * len(slots) * 2 * 128


# ----------------------------------------------------- cache scatter pins
def _sentinel(shape, dt):
    return np_bits(workloads.sentinel_cache(shape, TORCH_DT[dt]))


def pin_scatter_golden(L):
    for c in golden("scatter_hand.json")["cases"]:
        for dt in DTS:
            bs, nb, hkv, d = c["block_size"], c["num_blocks"], c["hkv"], c["d"]
            k, v = enc(c["k"], dt), enc(c["v"], dt)
            cache = _sentinel([2, nb, bs, hkv, d], dt)
            want = cache.copy()
            for w in c["written"]:
                want[w["kv"], w["block"], w["offset"], w["head"]] = enc(w["values"], dt)
            oracle.rope_kvstore(k, k, v, np.array(c["positions"]), 1e6, cache,
                                np.array(c["slots"]), block_size=bs, L=L)
            assert np.array_equal(cache.view(np.uint8), want.view(np.uint8)), c["derivation"]


def pin_scatter_bijection_vs_numpy(L):
    wl = workloads.prefill(n_seqs=3, len_lo=5, len_hi=40, seed=23)
    q, k, v = (np_bits(t) for t in (wl["q"], wl["k"], wl["v"]))
    slots = wl["slot_mapping"].numpy().copy()
    slots[::7] = -1  # padding tokens
    cache = np_bits(wl["cache"]).copy()
    _, k_rot = oracle.rope_kvstore(q, k, v, wl["positions"].numpy(), wl["theta"], cache, slots,
                                   block_size=wl["block_size"], L=L)
    nb, bs, hkv, d = cache.shape[1:]
    flat = cache.reshape(2, nb * bs, hkv, d)
    live = slots >= 0
    # V: numpy advanced-index assignment into a sentinel image gives the same bits.
    want_v = np_bits(wl["cache"]).reshape(2, nb * bs, hkv, d)[1].copy()
    want_v[slots[live]] = np.ascontiguousarray(v)[live]
    assert np.array_equal(flat[1], want_v)
    # K: the written slots are exactly the live slots; each holds k_rot rounded
    # to nearest (error at most half a bf16 ulp, 2^-8 relative).
    written = np.nonzero((flat[0] != 0xFFFF).any(axis=(1, 2)))[0]
    assert np.array_equal(np.sort(written), np.sort(slots[live]))
    assert int((flat[0] == 0xFFFF).sum()) == (nb * bs - live.sum()) * hkv * d
    got = dec(flat[0][slots[live]])
    ref = k_rot[live]
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-300)


def pin_scatter_round_trip(L):
    # Gathering through the block table (slot = block * bs + offset) returns
    # the stored V rows of each sequence in order.
    wl = workloads.prefill(n_seqs=2, len_lo=17, len_hi=50, seed=24)
    q, k, v = (np_bits(t) for t in (wl["q"], wl["k"], wl["v"]))
    cache = np_bits(wl["cache"]).copy()
    oracle.rope_kvstore(q, k, v, wl["positions"].numpy(), wl["theta"], cache,
                        wl["slot_mapping"].numpy(), block_size=wl["block_size"], L=L)
    off = 0
    for L_seq, bt in zip(wl["layout"].lens, wl["layout"].block_tables):
        got = oracle.paged_gather(cache, 1, bt.numpy(), L_seq, L=L)
        assert np.array_equal(got, np.ascontiguousarray(v[off:off + L_seq]))
        off += L_seq


def pin_gather_golden(L):
    # Reading back the golden scatter image through a hand block table: the
    # sequence that owns block 2 then block 0 (block size 2) sees the rows
    # written at slots 5 and 0 at its positions 1 and 2, and the sentinel at
    # its never-written positions 0 and 3.
    c = golden("scatter_hand.json")["cases"][0]
    for dt in DTS:
        cache = _sentinel([2, c["num_blocks"], c["block_size"], c["hkv"], c["d"]], dt)
        oracle.rope_kvstore(enc(c["k"], dt), enc(c["k"], dt), enc(c["v"], dt),
                            np.array(c["positions"]), 1e6, cache, np.array(c["slots"]),
                            block_size=c["block_size"], L=L)
        def same(a, b):  # bit patterns: the sentinel is a NaN
            return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))
        sentinel = _sentinel([1, 1, c["d"]], dt)[0]
        k = oracle.paged_gather(cache, 0, np.array([2, 0]), 4, L=L)
        v = oracle.paged_gather(cache, 1, np.array([2, 0]), 4, L=L)
        assert same(k[0], sentinel) and same(k[3], sentinel) and same(v[0], sentinel)
        assert same(k[1], enc(c["k"][0], dt)) and same(k[2], enc(c["k"][1], dt))
        assert same(v[1], enc(c["v"][0], dt)) and same(v[2], enc(c["v"][1], dt))


def pin_gqa_map(L):
    for c in golden("gqa_map.json")["cases"]:
        got = [oracle.gqa_kv_head(h, c["hq"], c["hkv"], L=L) for h in range(c["hq"])]
        assert got == c["map"], (c, got)


# ------------------------------------------------------------- SwiGLU pins
def pin_swiglu_golden(L):
    gd = golden("swiglu_hand.json")
    for c in gd["cases"]:
        out = oracle.swiglu(enc([[c["g"]]], F32), enc([[c["u"]]], F32), L=L)[0, 0]
        assert math.isclose(out, c["out"], rel_tol=gd["rel_tol"], abs_tol=1e-300), (c, out)


def pin_swiglu_odd_identity(L):
    # silu(-g) = silu(g) - g.
    g = rand_rows(4, 333, F32, seed=25, scale=4.0)
    one = enc(np.ones((4, 333)), F32)
    a = oracle.swiglu(g, one, L=L)
    b = oracle.swiglu((-g).astype(np.float32), one, L=L)
    assert np.allclose(b, a - dec(g), rtol=1e-13, atol=1e-13)


def pin_swiglu_limits(L):
    g = enc([[40.0, -40.0, 0.0]], F32)
    u = enc([[3.0, 3.0, 3.0]], F32)
    out = oracle.swiglu(g, u, L=L)[0]
    assert math.isclose(out[0], 120.0, rel_tol=1e-15)
    assert abs(out[1]) < 1e-14 and out[1] <= 0
    assert out[2] == 0.0


def pin_swiglu_vs_torch(L):
    for dt in DTS:
        g, u = rand_rows(7, 1000, dt, 26, scale=2.0), rand_rows(7, 1000, dt, 27)
        out = oracle.swiglu(g, u, L=L)
        ref = F.silu(torch.from_numpy(dec(g))) * torch.from_numpy(dec(u))
        assert np.allclose(out, ref.numpy(), rtol=1e-14, atol=1e-300)


def pin_swiglu_fused_halves(L):
    wl = workloads.swiglu_fused(rows=5, inter=96, seed=28)
    a = oracle.swiglu(np_bits(wl["gate"]), np_bits(wl["up"]), L=L)
    b = oracle.swiglu(np_bits(wl["gate"].contiguous()), np_bits(wl["up"].contiguous()), L=L)
    assert np.array_equal(a, b)


# ------------------------------------------------- ReGLU and clip-norm pins
def pin_reglu_golden(L):
    c = golden("reglu_clip_norm_hand.json")["reglu"][0]
    for dt in DTS:
        out = oracle.reglu(enc([c["g"]], dt), enc([c["u"]], dt), L=L)[0]
        assert np.array_equal(out, c["out"]), out


def pin_reglu_vs_torch(L):
    for dt in DTS:
        g, u = rand_rows(6, 1001, dt, 61, scale=2.0), rand_rows(6, 1001, dt, 62)
        ref = F.relu(torch.from_numpy(dec(g))) * torch.from_numpy(dec(u))
        assert np.allclose(oracle.reglu(g, u, L=L), ref.numpy(), rtol=0, atol=0)


def pin_clip_norm_golden(L):
    for c in golden("reglu_clip_norm_hand.json")["clip_norm"]:
        for dt in DTS:
            d = len(c["x"])
            y = oracle.clip_norm(enc(np.array(c["x"]).reshape(1, 1, d), dt), enc(c["alpha"], dt),
                                 enc(c["gamma"], dt), c["lo"], c["hi"], L=L)
            assert np.array_equal(y[0, 0], c["out"]), (c, y)


def pin_clip_norm_vs_numpy_and_bounds(L):
    # numpy's clip on the exact products; |y| <= max(|lo|, |hi|) * |gamma|;
    # strided [N, H, D] views give the same result as contiguous copies.
    g = workloads.gen(63)
    qkv = (workloads.randn([5, 16 * 64], g) * 3).to(torch.bfloat16)
    q = qkv[:, : 12 * 64].unflatten(1, (12, 64))
    rng = np.random.default_rng(64)
    a = enc(rng.standard_normal(64), BF16)
    gm = enc(1 + 0.2 * rng.standard_normal(64), BF16)
    y = oracle.clip_norm(np_bits(q), a, gm, -1.0, 1.0, L=L)
    x = dec(np.ascontiguousarray(np_bits(q)))
    ref = np.clip(dec(a) * x, -1.0, 1.0) * dec(gm)
    assert np.array_equal(y, ref)
    assert np.all(np.abs(y) <= np.abs(dec(gm)))
    y2 = oracle.clip_norm(np.ascontiguousarray(np_bits(q)), a, gm, -1.0, 1.0, L=L)
    assert np.array_equal(y, y2)


PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}

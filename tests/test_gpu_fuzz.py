"""Seeded randomized GPU parity against the CPU oracle: every case draws its
own sizes, strides, buffer offsets, dtype and variant, so the launch-shape
tiers (small calls, measured per-width shapes, unaligned rows, the
two-pass wide kernel), the strided views and the padding / permuted-block
cache layouts are crossed in combinations the hand-picked tests do not
list. Each case prints its parameters before it runs; the comparison rules
are the same as everywhere else (helpers.py). KCR_FUZZ_SCALE=k runs k times
as many cases of each kind (the first ones are the default cases)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_close, check_rope, assert_rope_close, np_bits

pytestmark = pytest.mark.gpu

DTS = [torch.bfloat16, torch.float16, torch.float32]
SCALE = max(1, int(os.environ.get("KCR_FUZZ_SCALE", "1")))


@pytest.fixture(scope="module")
def kcr():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import kv_cache_rmsnorm_amd as k
    return k


def say(*a):
    print(*a, flush=True)


def strided(data: torch.Tensor, stride: int, offset: int) -> torch.Tensor:
    """A device [rows, d] view with row stride `stride`, starting `offset`
    elements into a larger buffer, holding `data`."""
    rows, d = data.shape
    buf = torch.full((offset + rows * stride + 8,), float("nan"), dtype=data.dtype, device="cuda")
    view = buf[offset:offset + rows * stride].view(rows, stride)[:, :d]
    view.copy_(data)
    return view


TUNED_WIDTHS = [1536, 2048, 2176, 4096, 5120, 1024]
TIERS = ["tuned", "small", "unaligned", "wide", "rule", "any"]


def norm_case(case: int):
    """Each case targets one launch tier of the row-norm engine, and each tier
    meets every dtype: measured per-width shapes (>= 4096 plain rows at a
    listed width), small calls (<= 32 MB), rows at odd 2-byte offsets,
    rows beyond register residency, large calls under the shape rule, and
    unconstrained draws."""
    rng = np.random.default_rng(1000 + case)
    tier = TIERS[case % 6]
    dt = DTS[(case // 6) % 3]
    es = dt.itemsize
    add = bool(rng.integers(0, 2))
    x_pad, y_pad = int(rng.choice([0, 8, 64])), int(rng.choice([0, 16]))
    x_off = y_off = 0
    if tier == "tuned":
        add = False
        d = int(rng.choice(TUNED_WIDTHS))
        rows = int(rng.integers(4096, 4700))
    elif tier == "small":
        d = int(rng.integers(1, 9000))
        rows = int(rng.integers(1, 200))
    elif tier == "unaligned":
        d = int(rng.integers(1, 20000)) | 1
        rows = int(rng.integers(2, 150))
        x_pad, x_off, y_off = int(rng.choice([1, 3])), int(rng.integers(0, 4)), 1
    elif tier == "wide":
        d = int(rng.integers(4097, 9000)) * (16 // es)
        rows = int(rng.integers(1, 12))
    elif tier == "rule":
        d = int(rng.choice([1000, 3001, 2304, 6000])) * (2 if es == 2 else 1)
        rows = (40 << 20) // ((4 if add else 2) * d * es) + int(rng.integers(0, 64))
    else:
        d = int(rng.integers(1, 30000 if es == 2 else 15000))
        rows = int(rng.integers(1, 100))
        x_off, y_off = int(rng.integers(0, 4)), int(rng.integers(0, 4))
        x_pad = int(rng.choice([0, 1, 3, 8]))
    return tier, dt, d, rows, add, d + x_pad, d + y_pad, x_off, y_off, rng


@pytest.mark.parametrize("case", range(72 * SCALE))
def test_fuzz_norms(kcr, case):
    tier, dt, d, rows, add, x_stride, y_stride, x_off, y_off, rng = norm_case(case)
    say(f"norm case {case} ({tier}): dt={dt} d={d} rows={rows} add={add} strides x={x_stride} "
        f"y={y_stride} offsets {x_off},{y_off}")
    g = workloads.gen(2000 + case)
    x0 = (workloads.randn([rows, d], g) * float(rng.choice([1.0, 30.0]))).to(dt)
    w0 = (0.5 + torch.rand([d], generator=g)).to(dt)
    eps = float(np.float32(1e-6))
    x = strided(x0, x_stride, x_off)
    y = strided(torch.zeros_like(x0), y_stride, y_off)
    w = w0.cuda()
    if add:
        d0 = workloads.randn([rows, d], g).to(dt)
        dl = strided(d0, d + int(rng.choice([0, 5])), x_off)
        kcr.add_rmsnorm(x, dl, w, eps, out=y)
        x_ref, y_ref = oracle.add_rmsnorm(np_bits(x0), np_bits(d0), np_bits(w0), eps)
        assert np.array_equal(np_bits(x.cpu()).view(np.uint8), x_ref.view(np.uint8)), "residual"
    else:
        kcr.rmsnorm(x, w, eps, out=y)
        y_ref = oracle.rmsnorm(np_bits(x0), np_bits(w0), eps)
    assert_close(y.cpu().double().numpy(), y_ref, dt, f"norm case {case}")


@pytest.mark.parametrize("case", range(48 * SCALE))
def test_fuzz_norm_wave_rows(kcr, case):
    """Small calls whose rows are exactly 64 * VPT 16-byte vectors (VPT 1..8)
    take the one-wave-per-row kernel: every VPT in every dtype, plain and
    add (48 cases, one per combination), with row strides, buffer offsets
    and in-place output."""
    rng = np.random.default_rng(12000 + case)
    dt = DTS[case % 3]
    add = bool((case // 3) % 2)
    vpt = 1 + case // 6
    vec = 16 // dt.itemsize
    d = 64 * vpt * vec
    rows = int(rng.choice([1, int(rng.integers(2, 64)), int(rng.integers(200, 400))]))
    pad = int(rng.choice([0, 8, 32])) * (2 if dt.itemsize == 2 else 1)
    off = int(rng.choice([0, 8])) * (2 if dt.itemsize == 2 else 1)
    in_place = (not add) and bool(rng.integers(0, 2))
    say(f"wave-row case {case}: dt={dt} d={d} rows={rows} add={add} pad={pad} off={off} in_place={in_place}")
    g = workloads.gen(13000 + case)
    x0 = (workloads.randn([rows, d], g) * float(rng.choice([1.0, 30.0]))).to(dt)
    w0 = (0.5 + torch.rand([d], generator=g)).to(dt)
    eps = float(np.float32(1e-6))
    x = strided(x0, d + pad, off)
    y = x if in_place else strided(torch.zeros_like(x0), d + pad, off)
    w = w0.cuda()
    if add:
        d0 = workloads.randn([rows, d], g).to(dt)
        dl = strided(d0, d + pad, off)
        kcr.add_rmsnorm(x, dl, w, eps, out=y)
        x_ref, y_ref = oracle.add_rmsnorm(np_bits(x0), np_bits(d0), np_bits(w0), eps)
        assert np.array_equal(np_bits(x.cpu()).view(np.uint8), x_ref.view(np.uint8)), "residual"
    else:
        kcr.rmsnorm(x, w, eps, out=y)
        y_ref = oracle.rmsnorm(np_bits(x0), np_bits(w0), eps)
    assert_close(y.cpu().double().numpy(), y_ref, dt, f"wave-row case {case}")


@pytest.mark.parametrize("case", range(36 * SCALE))
def test_fuzz_gated(kcr, case):
    rng = np.random.default_rng(3000 + case)
    dt = DTS[case % 3]
    rows = int(rng.integers(1, 400))
    cols = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 20000)), 8960]))
    relu = bool(rng.integers(0, 2))
    fused = bool(rng.integers(0, 2))
    say(f"gated case {case}: dt={dt} rows={rows} cols={cols} relu={relu} fused={fused}")
    g = workloads.gen(4000 + case)
    gu0 = (workloads.randn([rows, 2 * cols], g) * 2).to(dt)
    if fused:
        gu = gu0.cuda()
        gate, up = gu[:, :cols], gu[:, cols:]
    else:
        gate = strided(gu0[:, :cols].contiguous(), cols + int(rng.choice([0, 3])), int(rng.integers(0, 4)))
        up = strided(gu0[:, cols:].contiguous(), cols + int(rng.choice([0, 7])), int(rng.integers(0, 4)))
    out = strided(torch.zeros((rows, cols), dtype=dt), cols + int(rng.choice([0, 1])), int(rng.integers(0, 4)))
    (kcr.reglu if relu else kcr.swiglu)(gate, up, out=out)
    ref = (oracle.reglu if relu else oracle.swiglu)(np_bits(gu0[:, :cols]), np_bits(gu0[:, cols:]))
    assert_close(out.cpu().double().numpy(), ref, dt, f"gated case {case}")


@pytest.mark.parametrize("case", range(36 * SCALE))
def test_fuzz_rope(kcr, case):
    rng = np.random.default_rng(5000 + case)
    dt = DTS[case % 3]
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 3, 6]))
    step = 16 if dt != torch.float32 else 8
    dh = int(rng.choice([d for d in (16, 32, 64, 96, 128, 256) if d % step == 0]))
    bs = int(rng.choice([1, 3, 16, 32]))
    n_seqs = int(rng.integers(1, 6))
    qknorm = bool(rng.integers(0, 2))
    say(f"rope case {case}: dt={dt} hq={hq} hkv={hkv} dh={dh} block_size={bs} seqs={n_seqs} qknorm={qknorm}")
    wl = workloads.prefill(n_seqs=n_seqs, len_lo=1, len_hi=300, dtype=dt, seed=6000 + case, hq=hq,
                           hkv=hkv, dh=dh, block_size=bs, theta=float(rng.choice([1e4, 1e6])))
    T = wl["qkv"].shape[0]
    slots = wl["slot_mapping"].clone()
    pad = torch.from_numpy(rng.random(T) < 0.1)                  # ~10% padding tokens
    slots[pad] = -1
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], dh, wl["theta"])
    cache = wl["cache"].cuda()
    q, k, v = workloads.qkv_views(wl["qkv"].cuda(), hq, hkv, dh)
    if not qknorm:
        qo = kcr.rope_kvstore(q, k, v, wl["positions"].cuda(), cos, sin, cache, slots.cuda())
        check_rope(wl["q"], wl["k"], wl["v"], wl["positions"], wl["cache"], slots, wl["theta"], qo.cpu(),
                   cache.cpu(), dt, f"rope case {case}")
        return
    g = workloads.gen(7000 + case)
    wq, wk = (1 + 0.2 * workloads.randn([dh], g)).to(dt), (0.5 + torch.rand([dh], generator=g)).to(dt)
    eps = float(np.float32(1e-6))
    qo = kcr.qknorm_rope_kvstore(q, k, v, wq.cuda(), wk.cuda(), eps, wl["positions"].cuda(), cos, sin,
                                 cache, slots.cuda())
    cache_ref = np_bits(wl["cache"]).copy()
    q_rot, k_rot = oracle.qknorm_rope_kvstore(np_bits(wl["q"]), np_bits(wl["k"]), np_bits(wl["v"]),
                                              np_bits(wq), np_bits(wk), eps, wl["positions"].numpy(),
                                              wl["theta"], cache_ref, slots.numpy(), block_size=bs)
    assert_rope_close(qo.cpu().double().numpy(), q_rot, dt, f"rope case {case}: q_out")
    n_slots = wl["cache"].shape[1] * bs
    got = np_bits(cache.cpu()).reshape(2, n_slots, hkv, dh)
    ref = cache_ref.reshape(2, n_slots, hkv, dh)
    assert np.array_equal(got[1].view(np.uint8), ref[1].view(np.uint8)), "V half and untouched V slots"
    live = slots.numpy()
    tok = np.nonzero(live >= 0)[0]
    mask = np.ones(n_slots, dtype=bool)
    mask[live[tok]] = False
    assert np.array_equal(got[0][mask].view(np.uint8), ref[0][mask].view(np.uint8)), "untouched K slots"
    kg = torch.from_numpy(got[0][live[tok]].view(np.int16 if dt.itemsize == 2 else np.int32).copy())
    assert_rope_close(kg.view(dt).double().numpy(), k_rot[tok], dt, f"rope case {case}: K rows")


@pytest.mark.parametrize("case", range(16 * SCALE))
def test_fuzz_gather(kcr, case):
    rng = np.random.default_rng(8000 + case)
    dt = DTS[case % 3]
    hkv = int(rng.choice([1, 2, 8]))
    dh = int(rng.choice([64, 128]))
    bs = int(rng.choice([1, 5, 16]))
    n_seqs = int(rng.integers(1, 7))
    say(f"gather case {case}: dt={dt} hkv={hkv} dh={dh} block_size={bs} seqs={n_seqs}")
    g = workloads.gen(9000 + case)
    lens = torch.randint(1, 200, (n_seqs,), generator=g)
    max_len = int(lens.max()) + int(rng.integers(0, 5))
    nbps = -(-max_len // bs)
    nb = n_seqs * nbps + 3
    bt = torch.randperm(nb, generator=g)[:n_seqs * nbps].view(n_seqs, nbps)
    cache = workloads.randn([2, nb, bs, hkv, dh], g).to(dt)
    k, v = kcr.paged_kv_gather(cache.cuda(), bt.cuda(), lens.cuda(), max_len,
                               k_out=torch.zeros((n_seqs, max_len, hkv, dh), dtype=dt, device="cuda"),
                               v_out=torch.zeros((n_seqs, max_len, hkv, dh), dtype=dt, device="cuda"))
    c = np_bits(cache)
    for b in range(n_seqs):
        L = int(lens[b])
        for half, out in ((0, k), (1, v)):
            ref = oracle.paged_gather(c, half, bt[b].numpy(), L)
            got = np_bits(out[b].cpu())
            assert np.array_equal(got[:L].view(np.uint8), ref.view(np.uint8)), f"seq {b} half {half}"
            assert not got[L:].any(), f"seq {b}: rows past the length were written"


@pytest.mark.parametrize("case", range(12 * SCALE))
def test_fuzz_chain_one_launch(kcr, case):
    """The one-launch decode chain (kcr_decode_chain_batch) at random
    batches, layer counts, widths, head layouts and block sizes in every
    dtype, with padding tokens and random positions, against the oracle run
    layer by layer (the same check as the benchmark's chain)."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    from test_gpu_configs import check_chain
    rng = np.random.default_rng(10000 + case)
    dt = DTS[case % 3]
    vec = 16 // dt.itemsize
    hidden = vec * int(rng.integers(1, 1025))
    inter = vec * int(rng.choice([int(rng.integers(1, 1025)), int(rng.integers(1025, 4097))]))
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 6]))
    dh = int(rng.choice([d for d in (16, 32, 64, 128, 256) if (d // 2) % vec == 0]))
    batch = int(rng.choice([1, int(rng.integers(2, 40)), int(rng.integers(200, 300))]))
    layers = int(rng.integers(1, 5))
    bs = int(rng.choice([1, 8, 16]))
    say(f"chain case {case}: dt={dt} batch={batch} layers={layers} hidden={hidden} inter={inter} "
        f"hq={hq} hkv={hkv} dh={dh} block_size={bs}")
    wl = workloads.decode_chain(layers=layers, batch=batch, ctx=int(rng.integers(1, 60)), dtype=dt,
                                seed=11000 + case, hidden=hidden, inter=inter, hq=hq, hkv=hkv, dh=dh,
                                block_size=bs)
    wl["positions"] = torch.from_numpy(rng.integers(0, wl["max_pos"], batch))
    pad = rng.random(batch) < 0.1
    wl["slot_mapping"][torch.from_numpy(pad)] = -1
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    chain.step_one_launch()
    torch.cuda.synchronize()
    check_chain(wl, chain)

"""GPU parity of each op against the CPU fp64 oracle, element by element, on
seeded inputs sized to span several workgroups and ragged tails, plus the
edge cases: widths 1..32768 including primes and 16-byte-misaligned tails,
strided views, in-place forms, padding slots, out-of-range indices, empty
calls and non-default streams.

Tolerances (written out in helpers.py): bf16 within 2 ulp or 1e-2, fp16
within 2 ulp, fp32 within 1e-5 relative; the updated residual, V and every untouched cache byte
bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (assert_bits_equal, assert_close, assert_rope_close, check_rope, gpu_qkv, np_bits,
                     tol_violations)

pytestmark = pytest.mark.gpu

DTS = [torch.bfloat16, torch.float32, torch.float16]
DT_ID = {torch.bfloat16: "bf16", torch.float32: "f32", torch.float16: "f16"}


@pytest.fixture(scope="module")
def kcr():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import kv_cache_rmsnorm_amd as k
    return k


from helpers import dev


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ RMSNorm
# 1538, 2180 and 8196 put 2-byte rows 4 or 8 bytes past a 16-byte boundary
# (dword-aligned vectors); odd widths alternate with 2-byte offsets (element
# access).
NORM_WIDTHS = [1, 7, 8, 9, 63, 64, 65, 127, 511, 512, 513, 1000, 1536, 1538, 2048, 2176, 2180, 3001,
               4095, 4096, 4097, 8191, 8192, 8193, 8196, 12289, 16384]


@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
@pytest.mark.parametrize("d", NORM_WIDTHS)
def test_rmsnorm_widths(kcr, dt, d):
    rows = 37
    say(f"rmsnorm dt={dt} d={d} rows={rows}")
    wl = workloads.rmsnorm_rows(rows=rows, d=d, dtype=dt, seed=d)
    y = kcr.rmsnorm(dev(wl["x"]), dev(wl["w"]), wl["eps"])
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    assert_close(y.cpu().double().numpy(), ref, dt, f"rmsnorm d={d}")


# 20000..32768: 8 waves of up to 8 vectors in registers; just past the
# register limit (32776), odd widths at 2-byte row offsets (40001, 49999) and
# whole 112 KB / 128 KB rows (57344, 65536) take the LDS-staged two-pass
# kernel.
@pytest.mark.parametrize("d", [20000, 24577, 32768, 32776, 40001, 49999, 57344, 65536])
def test_rmsnorm_widest_bf16(kcr, d):
    say(f"rmsnorm bf16 wide d={d}")
    wl = workloads.rmsnorm_rows(rows=9, d=d, dtype="bf16", seed=d)
    y = kcr.rmsnorm(dev(wl["x"]), dev(wl["w"]), wl["eps"])
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    assert_close(y.cpu().double().numpy(), ref, torch.bfloat16, f"rmsnorm d={d}")


# Rows wider than the register-resident engine (4096 vectors): the two-pass
# kernel, LDS-staged while a row fits in 160 KB, else reading the part beyond
# LDS twice.
WIDE = [(torch.bfloat16, 32769), (torch.bfloat16, 40000), (torch.bfloat16, 65536),
        (torch.bfloat16, 81000), (torch.bfloat16, 100003), (torch.float16, 50001),
        (torch.float16, 131072), (torch.float32, 16385), (torch.float32, 40000),
        (torch.float32, 50001)]


@pytest.mark.parametrize("dt,d", WIDE, ids=lambda v: DT_ID.get(v, str(v)))
def test_rmsnorm_wide_two_pass(kcr, dt, d):
    say(f"rmsnorm two-pass dt={dt} d={d}")
    wl = workloads.rmsnorm_rows(rows=7, d=d, dtype=dt, seed=d)
    y = kcr.rmsnorm(dev(wl["x"]), dev(wl["w"]), wl["eps"])
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    assert_close(y.cpu().double().numpy(), ref, dt, f"rmsnorm d={d}")


@pytest.mark.parametrize("dt,d", [(torch.bfloat16, 40000), (torch.bfloat16, 100003),
                                  (torch.float32, 20000), (torch.float32, 50001),
                                  (torch.float16, 65543)], ids=lambda v: DT_ID.get(v, str(v)))
def test_add_rmsnorm_wide_two_pass(kcr, dt, d):
    say(f"add_rmsnorm two-pass dt={dt} d={d}")
    wl = workloads.add_rmsnorm_rows(6, d, dtype=dt, seed=d)
    x = dev(wl["x"])
    y = kcr.add_rmsnorm(x, dev(wl["delta"]), dev(wl["w"]), wl["eps"])
    xn, ref = oracle.add_rmsnorm(np_bits(wl["x"]), np_bits(wl["delta"]), np_bits(wl["w"]),
                                 float(np.float32(wl["eps"])))
    assert np.array_equal(np_bits(x).view(np.uint8), xn.view(np.uint8)), "residual not bit-exact"
    assert_close(y.cpu().double().numpy(), ref, dt, f"add_rmsnorm d={d}")


def test_rmsnorm_wide_in_place_strided(kcr):
    say("rmsnorm two-pass, strided rows, in place")
    wl = workloads.rmsnorm_rows(rows=5, d=90001, dtype="bf16", seed=5)
    buf = torch.zeros((5, 90017), dtype=torch.bfloat16)
    buf[:, :90001] = wl["x"]
    xd = dev(buf)[:, :90001]
    kcr.rmsnorm(xd, dev(wl["w"]), wl["eps"], out=xd)
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    assert_close(xd.cpu().double().numpy(), ref, torch.bfloat16, "in place")
    assert bool((dev(buf)[:, 90001:] == 0).all())


def test_rmsnorm_wide_row_loop(kcr):
    # more rows than the two-pass grid (65536 workgroups): the row loop; the
    # oracle checks sampled rows on both sides of the wrap
    rows, d = 65536 + 37, 32776
    say(f"rmsnorm two-pass row loop rows={rows} d={d}")
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    x = torch.randn((rows, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn((d,), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = kcr.rmsnorm(x, w, 1e-6)
    pick = torch.tensor([0, 1, 65535, 65536, 65537, rows - 1], device="cuda")
    ref = oracle.rmsnorm(np_bits(x[pick].cpu()), np_bits(w.cpu()), float(np.float32(1e-6)))
    assert_close(y[pick].cpu().double().numpy(), ref, torch.bfloat16, "sampled rows")


# Widths with a measured launch shape of their own when a call has at least
# 4096 rows (some read two rows per row group before writing either); 4099
# rows leave the last group half empty.
TUNED = [(torch.bfloat16, 1536), (torch.bfloat16, 2048), (torch.bfloat16, 2176),
         (torch.bfloat16, 4096), (torch.bfloat16, 5120), (torch.float16, 1536),
         (torch.float16, 2048), (torch.float16, 2176), (torch.float16, 4096), (torch.float16, 5120),
         (torch.float32, 1024), (torch.float32, 2176)]


@pytest.mark.parametrize("dt,d", TUNED, ids=lambda v: DT_ID.get(v, str(v)))
def test_rmsnorm_tuned_widths(kcr, dt, d):
    rows = 4099
    say(f"rmsnorm tuned shape dt={dt} d={d} rows={rows}")
    wl = workloads.rmsnorm_rows(rows=rows, d=d, dtype=dt, seed=d + 1)
    y = kcr.rmsnorm(dev(wl["x"]), dev(wl["w"]), wl["eps"])
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    assert_close(y.cpu().double().numpy(), ref, dt, f"rmsnorm d={d}")


def test_rmsnorm_tuned_in_place_strided(kcr):
    rows, d = 4097, 2176
    say(f"rmsnorm tuned shape, strided rows in place, rows={rows}")
    wl = workloads.rmsnorm_rows(rows=rows, d=d, dtype="bf16", seed=3)
    buf = torch.zeros((rows, d + 24), dtype=torch.bfloat16)
    buf[:, :d] = wl["x"]
    xd = dev(buf)[:, :d]
    kcr.rmsnorm(xd, dev(wl["w"]), wl["eps"], out=xd)
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    assert_close(xd.cpu().double().numpy(), ref, torch.bfloat16, "in place")


@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_rmsnorm_many_rows(kcr, dt):
    # tens of thousands of one-pass workgroups; bf16 and fp16 stay in the
    # small-call tier (32 MB streamed), fp32 takes the shape rule
    rows, d = 40000, 200
    say(f"rmsnorm many rows rows={rows} dt={dt}")
    wl = workloads.rmsnorm_rows(rows=rows, d=d, dtype=dt, seed=5)
    y = kcr.rmsnorm(dev(wl["x"]), dev(wl["w"]), wl["eps"])
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    assert_close(y.cpu().double().numpy(), ref, dt, "rmsnorm many rows")


@pytest.mark.parametrize("add", [False, True], ids=["plain", "add"])
def test_norm_launch_split(kcr, add):
    # A grid holds at most 2^32 - 1 work-items, so a call with more rows than
    # one launch covers is split into launches over consecutive row ranges.
    # At one 16-byte vector per row that happens near 2^26 rows; the window
    # checked here covers every row within 6000 of 2^26, the last rows, and a
    # random sample.
    rows, d = (1 << 26) + 6000, 8
    say(f"norm launch split add={add} rows={rows} d={d}")
    g = torch.Generator(device="cuda")
    g.manual_seed(31)
    x = torch.randn((rows, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn((d,), generator=g, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
    pick = torch.cat([torch.arange((1 << 26) - 6000, rows, device="cuda"),
                      torch.randint(0, rows, (4000,), generator=g, device="cuda")])
    x0 = x[pick].cpu()
    eps = float(np.float32(1e-6))
    if add:
        dl = torch.randn((rows, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        y = kcr.add_rmsnorm(x, dl, w, eps)
        x_ref, y_ref = oracle.add_rmsnorm(np_bits(x0), np_bits(dl[pick].cpu()), np_bits(w.cpu()), eps)
        del dl
        assert np.array_equal(np_bits(x[pick].cpu()).view(np.uint8), x_ref.view(np.uint8)), "residual"
    else:
        y = kcr.rmsnorm(x, w, eps)
        y_ref = oracle.rmsnorm(np_bits(x0), np_bits(w.cpu()), eps)
    assert_close(y[pick].cpu().double().numpy(), y_ref, torch.bfloat16, "rows around the split")
    del x, y
    torch.cuda.empty_cache()


def test_rmsnorm_strided_and_in_place(kcr):
    say("rmsnorm strided + in place")
    wl = workloads.rmsnorm_rows(rows=50, d=1536 + 64, dtype="bf16", seed=7)
    big = dev(wl["x"])
    x = big[:, :1528]  # row stride 1600, width 1528 (ragged: 1528 = 191 vectors)
    w = dev(wl["w"][:1528].contiguous())
    ref = oracle.rmsnorm(np_bits(wl["x"][:, :1528]), np_bits(wl["w"][:1528].contiguous()), 1e-6)
    y = kcr.rmsnorm(x, w, 1e-6)
    assert_close(y.cpu().double().numpy(), ref, torch.bfloat16, "strided")
    before = big[:, 1528:].clone()
    kcr.rmsnorm(x, w, 1e-6, out=x)  # in place
    assert_close(x.cpu().double().numpy(), ref, torch.bfloat16, "in place")
    assert_bits_equal(big[:, 1528:], before, "columns past the view")


def test_rmsnorm_outlier_rows_fp32(kcr):
    # the 1% x100 outlier rows keep full fp32 accuracy
    wl = workloads.rmsnorm_rows(rows=512, d=2176, dtype="f32", seed=0)
    y = kcr.rmsnorm(dev(wl["x"]), dev(wl["w"]), wl["eps"]).cpu().double().numpy()
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), float(np.float32(wl["eps"])))
    rows = wl["outlier_rows"].numpy()
    assert len(rows) == 5
    assert_close(y[rows], ref[rows], torch.float32, "outlier rows")


# fp32 accumulation (the pages' norm computes in fp32) bounds the rows a norm can
# take: once a row's sum of squares overflows fp32 (|x| around 2e19 and
# up, which bf16 and fp32 hold), the sum is inf, the scale 1/sqrt(inf) = 0
# and y is a signed zero, where the fp64 oracle stays finite. The other rows
# of the same call are unaffected, and the add variant's residual stays
# bit-exact. No other test feeds such rows.
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=DT_ID.get)
@pytest.mark.parametrize("rows,d", [(8, 1536), (300, 2176), (4, 40000)])
@pytest.mark.parametrize("add", [False, True], ids=["plain", "add"])
def test_norm_fp32_sum_overflow(kcr, dt, rows, d, add):
    say(f"norm overflow dt={dt} rows={rows} d={d} add={add}")
    g = torch.Generator().manual_seed(rows + d)
    x = torch.randn((rows, d), generator=g).to(dt)
    delta = torch.randn((rows, d), generator=g).to(dt)
    w = (torch.rand(d, generator=g) + 0.5).to(dt)
    huge = [1, rows - 1]
    sign = torch.where(torch.rand((2, d), generator=g) < 0.5, -1.0, 1.0)
    x[huge] = (3e19 * sign).to(dt)
    eps = 1e-6
    xd = dev(x)
    if add:
        delta[huge] = 0
        y = kcr.add_rmsnorm(xd, dev(delta), dev(w), eps).cpu()
        x_ref, ref = oracle.add_rmsnorm(np_bits(x), np_bits(delta), np_bits(w), float(np.float32(eps)))
        assert np.array_equal(np_bits(xd.cpu()).view(np.uint8), x_ref.view(np.uint8)), "residual"
    else:
        y = kcr.rmsnorm(xd, dev(w), eps).cpu()
        ref = oracle.rmsnorm(np_bits(x), np_bits(w), float(np.float32(eps)))
    yd = y.double().numpy()
    assert np.all(np.isfinite(ref[huge])) and np.all(ref[huge] != 0), "the oracle stays finite"
    assert np.all(yd[huge] == 0), "rows whose fp32 sum of squares overflows give zeros"
    want_sign = np.signbit(x[huge].double().numpy()) ^ np.signbit(w.double().numpy())[None, :]
    assert np.array_equal(np.signbit(yd[huge]), want_sign), "the zeros carry the sign of x * w"
    keep = [r for r in range(rows) if r not in huge]
    assert_close(yd[keep], ref[keep], dt, "the other rows")


# The method's degenerate rows, among ordinary ones, against the oracle: a
# zero row (y exactly zero), a constant row (y = c / sqrt(c^2 + eps) * w), a
# row with one nonzero element, and a row so small that its squares
# underflow in fp32 (the sum is 0, so y = x * eps^(-1/2) * w, which is also
# the fp64 result to within the tolerance since eps dominates).
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
@pytest.mark.parametrize("rows,d", [(8, 1536), (300, 2176), (4, 40000)])
def test_norm_degenerate_rows(kcr, dt, rows, d):
    say(f"norm degenerate rows dt={dt} rows={rows} d={d}")
    g = torch.Generator().manual_seed(7 * rows + d)
    x = torch.randn((rows, d), generator=g).to(dt)
    w = (torch.rand(d, generator=g) + 0.5).to(dt)
    tiny = 1e-4 if dt == torch.float16 else 1e-30
    x[0] = 0
    x[1] = 0.75
    x[2] = 0
    x[2, d // 3] = -2.5
    x[rows - 1] = (tiny * torch.randn(d, generator=g)).to(dt)
    eps = 1e-6
    y = kcr.rmsnorm(dev(x), dev(w), eps).cpu().double().numpy()
    ref = oracle.rmsnorm(np_bits(x), np_bits(w), float(np.float32(eps)))
    assert np.all(y[0] == 0), "a zero row gives zeros"
    assert np.all(ref[0] == 0)
    assert_close(y, ref, dt, "degenerate rows")


def test_rmsnorm_empty_and_stream(kcr):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    assert kcr.rmsnorm(x, w).shape == (0, 64)
    wl = workloads.rmsnorm_rows(rows=300, d=1536, dtype="bf16", seed=9)
    s = torch.cuda.Stream()
    xs, ws = dev(wl["x"]), dev(wl["w"])
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = kcr.rmsnorm(xs, ws, 1e-6)
    s.synchronize()
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), 1e-6)
    assert_close(y.cpu().double().numpy(), ref, torch.bfloat16, "side stream")


# ------------------------------------------------------------- add + RMSNorm
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
@pytest.mark.parametrize("d", [1, 9, 1536, 2176, 4097, 8960, 16384])
def test_add_rmsnorm(kcr, dt, d):
    rows = 33
    say(f"add_rmsnorm dt={dt} d={d}")
    wl = workloads.add_rmsnorm_rows(rows, d, dtype=dt, seed=d)
    x = dev(wl["x"])
    y = kcr.add_rmsnorm(x, dev(wl["delta"]), dev(wl["w"]), wl["eps"])
    x_ref, y_ref = oracle.add_rmsnorm(np_bits(wl["x"]), np_bits(wl["delta"]), np_bits(wl["w"]),
                                      float(np.float32(wl["eps"])))
    got = np_bits(x.cpu())
    assert np.array_equal(got.view(np.uint8), x_ref.view(np.uint8)), "residual not bit-exact"
    assert_close(y.cpu().double().numpy(), y_ref, dt, f"add_rmsnorm y d={d}")


def test_add_rmsnorm_strided_delta(kcr):
    wl = workloads.add_rmsnorm_rows(300, 2048, dtype="bf16", seed=11)
    x = dev(wl["x"][:, :1536].contiguous())
    delta = dev(wl["delta"])[:, 256:1792]  # strided view, stride 2048
    w = dev(wl["w"][:1536].contiguous())
    y = kcr.add_rmsnorm(x, delta, w, 1e-6)
    x_ref, y_ref = oracle.add_rmsnorm(np_bits(wl["x"][:, :1536].contiguous()),
                                      np_bits(wl["delta"][:, 256:1792]),
                                      np_bits(wl["w"][:1536].contiguous()), 1e-6)
    assert np.array_equal(np_bits(x.cpu()), x_ref)
    assert_close(y.cpu().double().numpy(), y_ref, torch.bfloat16, "strided delta")


# ---------------------------------------------------------- RoPE + KV store
def rope_case(kcr, q, k, v, positions, cache, slots, theta, max_pos, q_out=None):
    """q, k, v on the device; runs the op and returns (q_out, cache) on the CPU."""
    cos, sin = kcr.rope_cos_sin(max_pos, q.shape[-1], theta)
    c = dev(cache)
    qo = kcr.rope_kvstore(q, k, v, dev(positions), cos, sin, c, dev(slots), q_out=q_out)
    return qo.cpu(), c.cpu()


@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_rope_decode_token(kcr, dt):
    say(f"rope decode token dt={dt}")
    wl = workloads.decode_token(dtype=dt)
    qg, cg = rope_case(kcr, *gpu_qkv(wl), wl["positions"], wl["cache"], wl["slot_mapping"],
                       wl["theta"], wl["max_pos"])
    check_rope(wl["q"], wl["k"], wl["v"], wl["positions"], wl["cache"], wl["slot_mapping"],
               wl["theta"], qg, cg, dt, "decode token")
    # the written slot is 597 = block 37, offset 5, and nothing else changed
    changed = (cg.view(torch.int16 if dt == torch.bfloat16 else torch.int32) != -1)
    assert changed.any(dim=(3, 4)).nonzero().tolist() == [[0, 37, 5], [1, 37, 5]]


@pytest.mark.parametrize("hq,hkv,dh", [(12, 2, 128), (8, 8, 64), (32, 8, 128), (16, 1, 256),
                                       (4, 2, 16), (2, 1, 512)])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_rope_shapes(kcr, hq, hkv, dh, dt):
    say(f"rope shapes hq={hq} hkv={hkv} dh={dh} dt={dt}")
    wl = workloads.prefill(n_seqs=3, len_lo=1, len_hi=70, dtype=dt, seed=hq * dh, hq=hq, hkv=hkv,
                           dh=dh, block_size=16)
    slots = wl["slot_mapping"].clone()
    slots[::5] = -1  # padding tokens
    qg, cg = rope_case(kcr, *gpu_qkv(wl), wl["positions"], wl["cache"], slots, wl["theta"],
                       wl["max_pos"])
    check_rope(wl["q"], wl["k"], wl["v"], wl["positions"], wl["cache"], slots, wl["theta"], qg, cg,
               dt, f"hq={hq} hkv={hkv} dh={dh}")


@pytest.mark.parametrize("hq,hkv,dh", [(12, 2, 128), (16, 8, 128), (8, 1, 96), (4, 4, 256),
                                       (2, 2, 512), (6, 3, 16)])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_qknorm_rope_kvstore(kcr, hq, hkv, dh, dt):
    say(f"qknorm rope hq={hq} hkv={hkv} dh={dh} dt={dt}")
    wl = workloads.prefill(n_seqs=3, len_lo=1, len_hi=60, dtype=dt, seed=hq + dh, hq=hq, hkv=hkv,
                           dh=dh, block_size=16)
    g = workloads.gen(dh)
    wq = (1 + 0.1 * workloads.randn([dh], g)).to(dt)
    wk = (0.5 + torch.rand([dh], generator=g)).to(dt)
    slots = wl["slot_mapping"].clone()
    slots[::4] = -1
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], dh, wl["theta"])
    cache = dev(wl["cache"])
    qo = kcr.qknorm_rope_kvstore(*gpu_qkv(wl), dev(wq), dev(wk), 1e-6, dev(wl["positions"]), cos,
                                 sin, cache, dev(slots))
    cache_ref = np_bits(wl["cache"]).copy()
    q_rot, k_rot = oracle.qknorm_rope_kvstore(np_bits(wl["q"]), np_bits(wl["k"]), np_bits(wl["v"]),
                                              np_bits(wq), np_bits(wk), float(np.float32(1e-6)),
                                              wl["positions"].numpy(), wl["theta"], cache_ref,
                                              slots.numpy())
    assert_rope_close(qo.cpu().double().numpy(), q_rot, dt, "q_out")
    got = np_bits(cache.cpu())
    nb, bs = wl["cache"].shape[1:3]
    g_flat, r_flat = got.reshape(2, nb * bs, hkv, dh), cache_ref.reshape(2, nb * bs, hkv, dh)
    live = slots.numpy()[slots.numpy() >= 0]
    assert np.array_equal(g_flat[1].view(np.uint8), r_flat[1].view(np.uint8)), "V half"
    mask = np.ones(nb * bs, dtype=bool)
    mask[live] = False
    assert np.array_equal(g_flat[0][mask].view(np.uint8), r_flat[0][mask].view(np.uint8))
    kg = torch.from_numpy(g_flat[0][live].view(np.int16 if dt == torch.bfloat16 else np.int32).copy())
    order = np.nonzero(slots.numpy() >= 0)[0]
    assert_rope_close(kg.view(dt).double().numpy(), k_rot[order], dt, "K rows")


def test_rope_prefill_block_size_and_in_place(kcr):
    say("rope block_size 7, contiguous q rotated in place")
    wl = workloads.prefill(n_seqs=4, len_lo=3, len_hi=300, dtype="bf16", seed=3, block_size=7)
    _, k, v = gpu_qkv(wl)
    q = dev(wl["q"].contiguous())
    qg, cg = rope_case(kcr, q, k, v, wl["positions"], wl["cache"], wl["slot_mapping"],
                       wl["theta"], wl["max_pos"], q_out=q)
    check_rope(wl["q"], wl["k"], wl["v"], wl["positions"], wl["cache"], wl["slot_mapping"],
               wl["theta"], qg, cg, torch.bfloat16, "in place, block size 7")


def test_rope_position_zero_and_out_of_range(kcr):
    say("rope position 0 identity; out-of-range positions and slots skipped")
    g = workloads.gen(17)
    T, hq, hkv, dh = 6, 12, 2, 128
    q = workloads.randn([T, hq, dh], g).to(torch.bfloat16)
    k = workloads.randn([T, hkv, dh], g).to(torch.bfloat16)
    v = workloads.randn([T, hkv, dh], g).to(torch.bfloat16)
    cache = workloads.sentinel_cache([2, 4, 16, hkv, dh], torch.bfloat16)
    positions = torch.tensor([0, 0, 5, 99, -1, 3], dtype=torch.int64)   # max_pos 64: 99, -1 invalid
    slots = torch.tensor([1, 63, 64, 2, 3, -7], dtype=torch.int64)      # 64 slots: 64 invalid
    q_out = torch.full((T, hq, dh), 7.0, dtype=torch.bfloat16, device="cuda")
    qg, cg = rope_case(kcr, dev(q), dev(k), dev(v), positions, cache, slots, 1e6, 64, q_out=q_out)
    # position 0 is the identity (values; +0 and -0 compare equal)
    assert torch.equal(qg[:2].float(), q[:2].float())
    # tokens with invalid positions copy their query heads unrotated (bit for
    # bit) and write nothing to the cache
    assert torch.equal(qg[3:5].view(torch.int16), q[3:5].view(torch.int16))
    cb = cg.view(torch.int16)
    written = sorted({(b * 16 + o) for _, b, o in (cb != -1).any(dim=(3, 4)).nonzero().tolist()})
    assert written == [1, 63]  # token 2's slot 64 is out of range, tokens 3/4 invalid, 5 padding
    assert torch.equal(cg[0, 0, 1].float(), k[0].float()) and torch.equal(cg[1, 3, 15], v[1])


def test_rope_table(kcr):
    say("rope cos/sin table")
    for max_pos, dh, theta in ((4097, 128, 1e6), (70000, 64, 1e4), (3, 2, 10.0)):
        cos, sin = kcr.rope_cos_sin(max_pos, dh, theta)
        c_ref, s_ref = oracle.rope_angles(max_pos, dh, theta)
        for got, ref in ((cos, c_ref), (sin, s_ref)):
            err = np.abs(got.cpu().double().numpy() - ref)
            # one fp32 rounding of an fp64 value (2^-24 relative) plus fp64 angle error
            assert np.all(err <= np.abs(ref) * 2.0 ** -24 + 1e-10), float(err.max())
        # the host-built tables meet the same bound (their fp64 pow/cos/sin are
        # the host's, which may differ from the device's in the last fp64 bit:
        # an absolute error of up to ~1e-11 at position 70000, hence the floor)
        ch, sh = kcr.rope_cos_sin_host(max_pos, dh, theta)
        for got, ref in ((ch, c_ref), (sh, s_ref)):
            err = np.abs(got.double().numpy() - ref)
            assert np.all(err <= np.abs(ref) * 2.0 ** -24 + 1e-10), float(err.max())


# ---------------------------------------------------------- paged KV gather
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
@pytest.mark.parametrize("bs", [16, 7])
def test_paged_kv_gather(kcr, dt, bs):
    say(f"paged gather dt={dt} block_size={bs}")
    wl = workloads.prefill(n_seqs=5, len_lo=1, len_hi=90, dtype=dt, seed=41 + bs, block_size=bs)
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], wl["dh"], wl["theta"])
    cache = dev(wl["cache"])
    kcr.rope_kvstore(*gpu_qkv(wl), dev(wl["positions"]), cos, sin, cache, dev(wl["slot_mapping"]))
    lay = wl["layout"]
    n, max_len = len(lay.lens), max(lay.lens) + 3
    mb = (max_len + bs - 1) // bs
    bt = torch.full((n, mb), -1, dtype=torch.int64)
    for i, t in enumerate(lay.block_tables):
        bt[i, :len(t)] = t
    lens = torch.tensor(lay.lens, dtype=torch.int64)
    fill = workloads.sentinel_cache([2, n, max_len, wl["hkv"], wl["dh"]], dt).to("cuda")
    k, v = kcr.paged_kv_gather(cache, dev(bt), dev(lens), max_len, k_out=fill[0], v_out=fill[1])
    c = np_bits(cache.cpu())
    for i, L in enumerate(lay.lens):
        for which, got in ((0, k), (1, v)):
            ref = oracle.paged_gather(c, which, bt[i, :len(lay.block_tables[i])].numpy(), L)
            g = np_bits(got[i].cpu())
            assert np.array_equal(g[:L].view(np.uint8), ref.view(np.uint8)), (i, which)
            assert (g[L:].view(np.uint8) == 0xFF).all(), "rows past the length must stay untouched"


def test_paged_kv_gather_bad_block_skipped(kcr):
    hkv, dh, bs, nb = 2, 128, 16, 4
    cache = torch.randn((2, nb, bs, hkv, dh), generator=workloads.gen(5)).to(torch.bfloat16).cuda()
    bt = torch.tensor([[1, 99], [-3, 2]], dtype=torch.int64).cuda()   # 99 and -3 are invalid
    lens = torch.tensor([32, 32], dtype=torch.int64).cuda()
    k = torch.zeros((2, 32, hkv, dh), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    kcr.paged_kv_gather(cache, bt, lens, 32, k_out=k, v_out=v)
    assert torch.equal(k[0, :16], cache[0, 1]) and torch.equal(v[1, 16:], cache[1, 2])
    assert bool((k[0, 16:] == 0).all()) and bool((v[1, :16] == 0).all())


# ------------------------------------------------------------------ SwiGLU
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 7), (1, 8960), (5, 8961), (300, 100),
                                       (64, 1023), (257, 4096), (1000, 17)])
def test_swiglu(kcr, dt, rows, cols):
    say(f"swiglu dt={dt} rows={rows} cols={cols}")
    wl = workloads.swiglu_fused(rows=rows, inter=cols, dtype=dt, seed=rows + cols)
    out = kcr.swiglu(dev(wl["gate"].contiguous()), dev(wl["up"].contiguous()))
    ref = oracle.swiglu(np_bits(wl["gate"]), np_bits(wl["up"]))
    assert_close(out.cpu().double().numpy(), ref, dt, f"swiglu {rows}x{cols}")


@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_swiglu_fused_halves_and_in_place(kcr, dt):
    wl = workloads.swiglu_fused(rows=123, inter=8960, dtype=dt, seed=4)
    gu = dev(wl["gate_up"])
    ref = oracle.swiglu(np_bits(wl["gate"]), np_bits(wl["up"]))
    out = kcr.swiglu_fused(gu)
    assert_close(out.cpu().double().numpy(), ref, dt, "fused halves")
    up_before = gu[:, 8960:].clone()
    kcr.swiglu(gu[:, :8960], gu[:, 8960:], out=gu[:, :8960])  # into the gate half
    assert_close(gu[:, :8960].cpu().double().numpy(), ref, dt, "in place")
    assert_bits_equal(gu[:, 8960:], up_before, "up half untouched")


def test_swiglu_extremes(kcr):
    # Inside |g| <= 87 every fp32 intermediate stays normal and the relative
    # bound holds; past the overflow of exp(-g) the result is +-0 or g * u.
    g = torch.tensor([[-200.0, -87.0, -20.0, -1.0, -1e-30, 0.0, 1e-30, 1.0, 20.0, 87.0, 200.0,
                       3e38, -3e38]], dtype=torch.float32)
    u = torch.full_like(g, 0.5)
    out = kcr.swiglu(dev(g), dev(u)).cpu().double().numpy()
    ref = oracle.swiglu(np_bits(g), np_bits(u))
    assert not tol_violations(out, ref, torch.float32).any(), (out, ref)
    # between -104 and -88 the exact result is below 2e-36 and may flush to zero
    g2 = torch.linspace(-104, -88, 64, dtype=torch.float32).reshape(1, -1)
    out2 = kcr.swiglu(dev(g2), dev(torch.ones_like(g2))).cpu().double().numpy()
    assert np.all(np.abs(out2) <= 2e-36) and np.all(out2 <= 0)


# ------------------------------------------------------------------ ReGLU
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
@pytest.mark.parametrize("rows,cols", [(1, 8960), (7, 13), (300, 1000)])
def test_reglu(kcr, dt, rows, cols):
    say(f"reglu dt={dt} {rows}x{cols}")
    wl = workloads.swiglu_fused(rows=rows, inter=cols, dtype=dt, seed=rows * cols)
    gu = dev(wl["gate_up"])
    out = kcr.reglu(gu[:, :cols], gu[:, cols:])
    ref = oracle.reglu(np_bits(wl["gate"]), np_bits(wl["up"]))
    assert_close(out.cpu().double().numpy(), ref, dt, "reglu")


# ------------------------------------------------------------- clip norm
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
@pytest.mark.parametrize("apc,gpc", [(True, True), (False, True), (True, False), (False, False)])
def test_clip_norm_qk_views(kcr, dt, apc, gpc):
    say(f"clip norm dt={dt} alpha per channel={apc} gamma per channel={gpc}")
    g = workloads.gen(70)
    qkv = (workloads.randn([123, 16 * 128], g) * 2).to(dt)
    q = qkv[:, : 12 * 128].unflatten(1, (12, 128))          # token stride 2048, head stride 128
    a = (workloads.randn([128 if apc else 1], g)).to(dt)
    gm = (1 + 0.3 * workloads.randn([128 if gpc else 1], g)).to(dt)
    qd = dev(qkv)[:, : 12 * 128].unflatten(1, (12, 128))
    y = kcr.clip_norm(qd, dev(a), dev(gm))
    ref = oracle.clip_norm(np_bits(q), np_bits(a), np_bits(gm))
    assert_close(y.cpu().double().numpy(), ref, dt, "clip norm")


def test_clip_norm_in_place_and_ragged(kcr):
    say("clip norm in place, ragged rows")
    g = workloads.gen(71)
    x = (workloads.randn([57, 3, 75], g) * 3).to(torch.bfloat16)  # 75 bf16: rows not 16-byte aligned
    a = torch.tensor([0.7], dtype=torch.bfloat16)
    gm = (workloads.randn([75], g)).to(torch.bfloat16)
    ref = oracle.clip_norm(np_bits(x), np_bits(a), np_bits(gm), -0.5, 2.0)
    xd = dev(x)
    kcr.clip_norm(xd, dev(a), dev(gm), -0.5, 2.0, out=xd)
    assert_close(xd.cpu().double().numpy(), ref, torch.bfloat16, "clip norm in place")


# ------------------------------------------------------------------ copy
def test_copy(kcr):
    src = torch.randint(-2**31, 2**31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    kcr.copy_(dst, src)
    assert torch.equal(dst, src)


def test_concurrent_host_threads(kcr):
    """Two host threads call the library at once (ctypes releases the GIL),
    each on its own stream, with row widths that take the LDS-staged
    two-pass kernel at different staging sizes, plus a register-resident
    width. Every result must equal the same call made alone."""
    import threading
    say("concurrent calls from two host threads")
    cases = []
    for d in (40000, 65536, 2176):
        wl = workloads.rmsnorm_rows(rows=6, d=d, dtype="bf16", seed=d)
        x, w = dev(wl["x"]), dev(wl["w"])
        cases.append((x, w, kcr.rmsnorm(x, w, wl["eps"]).clone(), wl["eps"]))
    torch.cuda.synchronize()
    errors = []

    def worker(order):
        s = torch.cuda.Stream()
        try:
            with torch.cuda.stream(s):
                for _ in range(25):
                    for i in order:
                        x, w, ref, eps = cases[i]
                        y = kcr.rmsnorm(x, w, eps)
                        s.synchronize()
                        if not torch.equal(y.view(torch.int16), ref.view(torch.int16)):
                            errors.append(f"case {i} differs")
        except Exception as e:  # reported below, in the test's own thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(o,)) for o in ((0, 1, 2), (1, 0, 2))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors[:3]


def test_errors_launch_nothing(kcr):
    """A refused call enqueues nothing: after each entry point below returns
    its error code, the output (and, for the aliasing call, the input it
    would have overwritten) keeps every byte."""
    lib, s = kcr._lib, torch.cuda.current_stream().cuda_stream
    g = torch.Generator().manual_seed(3)
    xb = torch.randn((9, 64), generator=g).to(torch.bfloat16).cuda()  # one spare row
    x = xb[:8]
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    y = torch.full((8, 64), -1, dtype=torch.int16, device="cuda")
    x0, y0 = xb.clone(), y.clone()
    assert lib.kcr_rmsnorm(x.data_ptr(), 64, w.data_ptr(), y.data_ptr(), 64, 8, 64, 1e-6, 9, s) == -3
    assert lib.kcr_rmsnorm(x.data_ptr(), 64, w.data_ptr(), x.data_ptr() + 128, 64, 8, 64, 1e-6, 0, s) == -6
    assert lib.kcr_swiglu(x.data_ptr(), 64, x.data_ptr(), 64, y.data_ptr(), 16, 8, 32, 0, s) == -2
    q = torch.randn((2, 3, 128), generator=g).to(torch.bfloat16).cuda()
    kv = torch.randn((2, 2, 128), generator=g).to(torch.bfloat16).cuda()
    pos = torch.zeros(2, dtype=torch.int64, device="cuda")
    cos = torch.ones((4, 64), device="cuda")
    cache = torch.full((2, 4, 4, 2, 128), -1, dtype=torch.int16, device="cuda")
    cache0 = cache.clone()
    qo = torch.full((2, 3, 128), -1, dtype=torch.int16, device="cuda")
    assert lib.kcr_rope_kvstore(q.data_ptr(), 384, 128, kv.data_ptr(), 256, 128, kv.data_ptr(), 256, 128,
                                qo.data_ptr(), pos.data_ptr(), cos.data_ptr(), cos.data_ptr(), 4,
                                cache.data_ptr(), pos.data_ptr(), 2, 3, 2, 128, 4, 4, 0, s) == -5
    torch.cuda.synchronize()
    assert torch.equal(xb, x0) and torch.equal(y, y0) and torch.equal(cache, cache0)
    assert bool((qo == -1).all())


def test_debug_mode(kcr):
    """KCR_DEBUG=1: every call synchronizes and checks its kernel, and a
    captured graph still records and replays; the results are the same bits
    as without it."""
    import hashlib
    import os
    import subprocess
    import sys
    code = (
        "import hashlib, torch\n"
        "import kv_cache_rmsnorm_amd as k\n"
        "g = torch.Generator().manual_seed(5)\n"
        "x = torch.randn((300, 2176), generator=g).to(torch.bfloat16).cuda()\n"
        "w = (0.5 + torch.rand(2176, generator=g)).to(torch.bfloat16).cuda()\n"
        "y = k.rmsnorm(x, w)\n"
        "s = torch.cuda.Stream()\n"
        "s.wait_stream(torch.cuda.current_stream())\n"
        "with torch.cuda.stream(s):\n"
        "    k.rmsnorm(x, w, out=y)\n"
        "torch.cuda.current_stream().wait_stream(s)\n"
        "torch.cuda.synchronize()\n"
        "graph = torch.cuda.CUDAGraph()\n"
        "with torch.cuda.graph(graph):\n"
        "    k.rmsnorm(x, w, out=y)\n"
        "y.zero_()\n"
        "graph.replay()\n"
        "torch.cuda.synchronize()\n"
        "print(hashlib.sha256(y.cpu().view(torch.int16).numpy().tobytes()).hexdigest(), flush=True)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("debug mode in a child process")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=dict(os.environ, KCR_DEBUG="1"),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    g = torch.Generator().manual_seed(5)
    x = torch.randn((300, 2176), generator=g).to(torch.bfloat16).cuda()
    w = (0.5 + torch.rand(2176, generator=g)).to(torch.bfloat16).cuda()
    y = kcr.rmsnorm(x, w)
    torch.cuda.synchronize()
    want = hashlib.sha256(y.cpu().view(torch.int16).numpy().tobytes()).hexdigest()
    assert r.stdout.strip().splitlines()[-1] == want

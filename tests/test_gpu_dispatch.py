"""GPU parity for the launch shapes the host-side dispatch chooses.

Each entry point picks a kernel variant from the call's width, row count,
dtype, row alignment, size and head layout: the row-norm engine's shape
rule, its small-call, unaligned-row and wide-row tiers; the RoPE unit
kernel (half a head that is not a power-of-two number of 16-byte chunks, or
more than 1024 lanes of heads per token) and the token kernel at every
chunk count, with and without the Q/K norm and with fused or separate
q/k/v; the clip norm and gated activations at unaligned rows; the
one-launch chain at every SwiGLU depth and workgroup size. These cases are
chosen so that every such variant runs at least once, and each is compared
with the oracle under the rules of helpers.py. Large calls (more than
32 MB, where the shape rule differs from small calls) are checked on
sampled rows: their rows repeat a small seeded pool, and the oracle computes
the sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_close, assert_rope_close, check_rope, np_bits

pytestmark = pytest.mark.gpu

DTS = [torch.bfloat16, torch.float16, torch.float32]
DT_ID = {torch.bfloat16: "bf16", torch.float32: "f32", torch.float16: "f16"}
EPS = float(np.float32(1e-6))
SMALL_CALL_BYTES = 32 << 20


@pytest.fixture(scope="module")
def kcr():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import kv_cache_rmsnorm_amd as k
    return k


def say(*a):
    print(*a, flush=True)


def vec_of(dt) -> int:
    return 16 // dt.itemsize


# Row widths in 16-byte vectors: every count up to 9, and 64k - 1, 64k,
# 64k + 1 up to the register engine's limit of 4096 vectors, so that each
# (vectors per lane, waves per row, workgroup) choice and both sides of
# every boundary between them occur.
NVEC = sorted({n for n in range(1, 10)} |
              {n for k in range(1, 65) for n in (64 * k - 1, 64 * k, 64 * k + 1) if n <= 4096})


def norm_width(nvec: int, vec: int, rng, even: bool) -> int:
    """A width of exactly `nvec` vectors: a whole number of vectors at each
    multiple of 64, otherwise a ragged last vector (an even number of
    elements short for 2-byte types, so rows stay dword aligned)."""
    if nvec % 64 == 0 or vec == 1:
        return nvec * vec
    short = int(rng.integers(1, vec))
    if even:
        short -= short % 2
    return max(1, nvec * vec - short)


def run_norm(kcr, x0, d0, w0, add, what):
    dt = x0.dtype
    x = x0.cuda()
    if add:
        dl = d0.cuda()
        y = kcr.add_rmsnorm(x, dl, w0.cuda(), EPS)
        x_ref, y_ref = oracle.add_rmsnorm(np_bits(x0), np_bits(d0), np_bits(w0), EPS)
        assert np.array_equal(np_bits(x.cpu()).view(np.uint8), x_ref.view(np.uint8)), f"{what}: residual"
    else:
        y = kcr.rmsnorm(x, w0.cuda(), EPS)
        y_ref = oracle.rmsnorm(np_bits(x0), np_bits(w0), EPS)
    assert_close(y.cpu().double().numpy(), y_ref, dt, what)


@pytest.mark.parametrize("add", [False, True], ids=["plain", "add"])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_norm_small_call_shapes(kcr, dt, add):
    """Small calls (the decode-size tier) at every width class: rows of
    whole vectors (the one-wave kernel, exact or ragged, where it applies)
    and rows whose last vector is cut short (the rule's shapes)."""
    rng = np.random.default_rng(21000 + 2 * DTS.index(dt) + add)
    vec = vec_of(dt)
    g = workloads.gen(21100 + 2 * DTS.index(dt) + add)
    for nvec in NVEC:
        # whole vectors (one-wave kernels up to their limits) and a last
        # vector cut short (the rule's shapes with their element tail)
        short = int(rng.integers(1, vec // 2)) * 2 if dt.itemsize == 2 else int(rng.integers(1, vec))
        for d in (nvec * vec, nvec * vec - short):
            rows = int(rng.integers(1, 6))
            say(f"small-call norm dt={DT_ID[dt]} add={add} d={d} ({nvec} vectors) rows={rows}")
            x0 = (workloads.randn([rows, d], g) * 3).to(dt)
            d0 = workloads.randn([rows, d], g).to(dt) if add else None
            w0 = (0.5 + torch.rand([d], generator=g)).to(dt)
            run_norm(kcr, x0, d0, w0, add, f"d={d} rows={rows}")


# Large calls: the shape rule's regions (one wave of 1-5 vectors per lane,
# 2-3 vectors over 2-8 waves, 8 waves of 4-8 vectors; the add variant's
# 1-2 vectors) and their boundaries; widths off the measured per-width table.
LARGE_NVEC = [1, 2, 64, 65, 128, 129, 192, 256, 300, 320, 321, 384, 385, 512, 513, 700, 768, 769, 1024,
              1025, 1200, 1536, 1537, 2000, 2048, 2049, 2560, 3000, 3072, 3073, 3584, 4000, 4096]


@pytest.mark.parametrize("add", [False, True], ids=["plain", "add"])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_norm_large_call_shapes(kcr, dt, add):
    """Calls above the small-call size take the shape rule with several row
    groups per workgroup; rows repeat seeded pools of 61 (x) and 59 (delta)
    rows, and 40 sampled rows are checked, the first, middle and last among
    them."""
    rng = np.random.default_rng(22000 + 2 * DTS.index(dt) + add)
    vec, es = vec_of(dt), dt.itemsize
    g = workloads.gen(22100 + 2 * DTS.index(dt) + add)
    for nvec in LARGE_NVEC:
        d = norm_width(nvec, vec, rng, even=es == 2)
        if nvec % 64 == 0 and vec > 1:
            d -= 2 if es == 2 else 1      # keep the widths off the per-width table
        rows = SMALL_CALL_BYTES // ((4 if add else 2) * d * es) + 1 + int(rng.integers(0, 50))
        say(f"large-call norm dt={DT_ID[dt]} add={add} d={d} ({nvec} vectors) rows={rows}")
        px = (workloads.randn([61, d], g) * 3).to(dt)
        pd = workloads.randn([59, d], g).to(dt)
        w0 = (0.5 + torch.rand([d], generator=g)).to(dt)
        idx = torch.arange(rows, device="cuda")
        x = px.cuda()[idx % 61]
        w = w0.cuda()
        sample = np.unique(np.concatenate([[0, 1, rows // 2, rows - 2, rows - 1],
                                           rng.integers(0, rows, 35)]))
        xs0 = px[torch.from_numpy(sample % 61)]
        if add:
            dl = pd.cuda()[idx % 59]
            y = kcr.add_rmsnorm(x, dl, w, EPS)
            ds0 = pd[torch.from_numpy(sample % 59)]
            x_ref, y_ref = oracle.add_rmsnorm(np_bits(xs0), np_bits(ds0), np_bits(w0), EPS)
            got_x = np_bits(x[torch.from_numpy(sample).cuda()].cpu())
            assert np.array_equal(got_x.view(np.uint8), x_ref.view(np.uint8)), f"d={d}: residual"
        else:
            y = kcr.rmsnorm(x, w, EPS)
            y_ref = oracle.rmsnorm(np_bits(xs0), np_bits(w0), EPS)
        got = y[torch.from_numpy(sample).cuda()].cpu().double().numpy()
        assert_close(got, y_ref, dt, f"large call d={d} rows={rows}")
        del x, y, idx


@pytest.mark.parametrize("add", [False, True], ids=["plain", "add"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=DT_ID.get)
def test_norm_unaligned_row_shapes(kcr, dt, add):
    """Odd widths put every other row at an odd 2-byte offset: the
    unaligned tier's one-wave shapes (1-8 vectors per lane) and eight-wave
    shapes (2-8 vectors per lane)."""
    rng = np.random.default_rng(23000 + 2 * DTS.index(dt) + add)
    g = workloads.gen(23100 + 2 * DTS.index(dt) + add)
    widths = [1, 3, 7, 9] + [64 * v * 8 - 1 for v in range(1, 9)] + [512 * v * 8 - 1 for v in range(2, 9)]
    for d in widths:
        rows = int(rng.integers(2, 7))
        say(f"unaligned norm dt={DT_ID[dt]} add={add} d={d} rows={rows}")
        x0 = (workloads.randn([rows, d], g) * 3).to(dt)
        d0 = workloads.randn([rows, d], g).to(dt) if add else None
        w0 = (0.5 + torch.rand([d], generator=g)).to(dt)
        run_norm(kcr, x0, d0, w0, add, f"unaligned d={d} rows={rows}")


@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_add_norm_beyond_lds(kcr, dt):
    """Residual-add rows wider than LDS: the part that fits stays in LDS, the
    rest is read again."""
    d = {2: 90002, 4: 45001}[dt.itemsize]
    say(f"add norm beyond LDS dt={DT_ID[dt]} d={d}")
    g = workloads.gen(23500 + DTS.index(dt))
    x0 = (workloads.randn([3, d], g) * 3).to(dt)
    d0 = workloads.randn([3, d], g).to(dt)
    w0 = (0.5 + torch.rand([d], generator=g)).to(dt)
    run_norm(kcr, x0, d0, w0, True, f"add beyond LDS d={d}")


# ---------------------------------------------------------------- RoPE
def rope_case(kcr, dt, hq, hkv, dh, n_seqs, len_lo, len_hi, qknorm, fused, seed, what):
    wl = workloads.prefill(n_seqs=n_seqs, len_lo=len_lo, len_hi=len_hi, dtype=dt, seed=seed, hq=hq,
                           hkv=hkv, dh=dh, block_size=16)
    T = wl["qkv"].shape[0]
    say(f"{what}: dt={DT_ID[dt]} hq={hq} hkv={hkv} dh={dh} tokens={T} qknorm={qknorm} fused={fused}")
    slots = wl["slot_mapping"].clone()
    slots[::7] = -1                                              # padding tokens
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], dh, wl["theta"])
    cache = wl["cache"].cuda()
    if fused:
        q, k, v = workloads.qkv_views(wl["qkv"].cuda(), hq, hkv, dh)
    else:
        q, k, v = (t.contiguous().cuda() for t in (wl["q"], wl["k"], wl["v"]))
    pos = wl["positions"].cuda()
    if not qknorm:
        qo = kcr.rope_kvstore(q, k, v, pos, cos, sin, cache, slots.cuda())
        check_rope(wl["q"], wl["k"], wl["v"], wl["positions"], wl["cache"], slots, wl["theta"], qo.cpu(),
                   cache.cpu(), dt, what)
        return
    g = workloads.gen(seed + 1)
    wq, wk = (1 + 0.2 * workloads.randn([dh], g)).to(dt), (0.5 + torch.rand([dh], generator=g)).to(dt)
    qo = kcr.qknorm_rope_kvstore(q, k, v, wq.cuda(), wk.cuda(), EPS, pos, cos, sin, cache, slots.cuda())
    cache_ref = np_bits(wl["cache"]).copy()
    q_rot, k_rot = oracle.qknorm_rope_kvstore(np_bits(wl["q"]), np_bits(wl["k"]), np_bits(wl["v"]),
                                              np_bits(wq), np_bits(wk), EPS, wl["positions"].numpy(),
                                              wl["theta"], cache_ref, slots.numpy(), block_size=16)
    assert_rope_close(qo.cpu().double().numpy(), q_rot, dt, f"{what}: q_out")
    n_slots = wl["cache"].shape[1] * 16
    got = np_bits(cache.cpu()).reshape(2, n_slots, hkv, dh)
    ref = cache_ref.reshape(2, n_slots, hkv, dh)
    assert np.array_equal(got[1].view(np.uint8), ref[1].view(np.uint8)), f"{what}: V half"
    live = slots.numpy()
    tok = np.nonzero(live >= 0)[0]
    mask = np.ones(n_slots, dtype=bool)
    mask[live[tok]] = False
    assert np.array_equal(got[0][mask].view(np.uint8), ref[0][mask].view(np.uint8)), f"{what}: untouched K"
    kg = torch.from_numpy(got[0][live[tok]].view(np.int16 if dt.itemsize == 2 else np.int32).copy())
    assert_rope_close(kg.view(dt).double().numpy(), k_rot[tok], dt, f"{what}: K rows")


@pytest.mark.parametrize("prefill", [False, True], ids=["decode", "prefill"])
@pytest.mark.parametrize("qknorm", [False, True], ids=["rope", "qknorm"])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_rope_unit_kernel_head_dims(kcr, dt, qknorm, prefill):
    """Half a head of 3, 5, 10 or 20 chunks (not a power of two) takes the
    unit kernel with 4, 8, 16 or 32 lanes per head, and fp32 at 40 chunks
    with 64 (head_dim is at most 512); up to 4096 tokens one head per unit,
    beyond that two."""
    vec = vec_of(dt)
    for i, chunks in enumerate((3, 5, 10, 20, 40)):
        if 2 * chunks * vec > 512:
            continue
        dh = 2 * chunks * vec
        if prefill:
            rope_case(kcr, dt, 4, 2, dh, 3, 1400, 1500, qknorm, True, 24000 + 10 * i + qknorm,
                      f"unit kernel, {chunks} chunks, prefill")
        else:
            rope_case(kcr, dt, 4, 2, dh, 3, 5, 40, qknorm, True, 24100 + 10 * i + qknorm,
                      f"unit kernel, {chunks} chunks, decode")


@pytest.mark.parametrize("prefill", [False, True], ids=["decode", "prefill"])
@pytest.mark.parametrize("qknorm", [False, True], ids=["rope", "qknorm"])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_rope_unit_kernel_many_heads(kcr, dt, qknorm, prefill):
    """More than 1024 lanes of heads per token at 1 and 2 chunks per half
    head: the unit kernel with 1 and 2 lanes per head, one or (beyond 4096
    tokens) two heads per unit."""
    vec = vec_of(dt)
    for chunks, hq, hkv in ((1, 1023, 1), (2, 511, 1)):
        n, lo, hi = (1, 4097, 4120) if prefill else (2, 2, 4)
        rope_case(kcr, dt, hq, hkv, 2 * chunks * vec, n, lo, hi, qknorm, True,
                  24500 + chunks + 2 * qknorm + 4 * prefill, f"unit kernel, {chunks} chunk(s), {hq}/{hkv} heads")


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("qknorm", [False, True], ids=["rope", "qknorm"])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_rope_token_kernel_head_dims(kcr, dt, qknorm, fused):
    """The token kernel at every power-of-two chunk count of half a head up
    to head_dim 512 (1..32 lanes per head, 64 for fp32; head_dim 128 through
    its fixed-size form), with q/k/v as views of one fused projection or as
    separate tensors."""
    vec = vec_of(dt)
    for i, chunks in enumerate((1, 2, 4, 8, 16, 32, 64)):
        dh = 2 * chunks * vec
        if dh > 512:
            continue
        hq, hkv = (4, 2) if chunks >= 32 else (6, 2)
        rope_case(kcr, dt, hq, hkv, dh, 2, 3, 30, qknorm, fused, 25000 + 10 * i + 2 * qknorm + fused,
                  f"token kernel, {chunks} chunks")


# --------------------------------------------------- clip norm, gated ops
def at_odd_offset(data: torch.Tensor) -> torch.Tensor:
    """A device copy of `data` starting one element past a 16-byte boundary."""
    buf = torch.zeros(data.numel() + 8, dtype=data.dtype, device="cuda")
    view = buf[1:1 + data.numel()].view(data.shape)
    view.copy_(data)
    return view


@pytest.mark.parametrize("gpc", [False, True], ids=["gamma1", "gammaC"])
@pytest.mark.parametrize("apc", [False, True], ids=["alpha1", "alphaC"])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=DT_ID.get)
def test_clip_norm_unaligned_rows(kcr, dt, apc, gpc):
    """Head rows at odd 2-byte offsets take the element-access form."""
    say(f"clip norm unaligned dt={DT_ID[dt]} alpha per channel={apc} gamma per channel={gpc}")
    g = workloads.gen(26000 + 4 * apc + 2 * gpc + DTS.index(dt))
    x0 = (workloads.randn([37, 3, 64], g) * 2).to(dt)
    a = workloads.randn([64 if apc else 1], g).to(dt)
    gm = (1 + 0.3 * workloads.randn([64 if gpc else 1], g)).to(dt)
    y = kcr.clip_norm(at_odd_offset(x0), a.cuda(), gm.cuda())
    ref = oracle.clip_norm(np_bits(x0), np_bits(a), np_bits(gm))
    assert_close(y.cpu().double().numpy(), ref, dt, "clip norm, unaligned rows")


@pytest.mark.parametrize("relu", [False, True], ids=["swiglu", "reglu"])
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_gated_launch_forms(kcr, dt, relu):
    """Small calls whose width is not a whole number of vectors (128-lane
    flat form), and for 2-byte types rows at odd offsets, small and large
    (element access)."""
    fn, ref_fn = (kcr.reglu, oracle.reglu) if relu else (kcr.swiglu, oracle.swiglu)
    vec = vec_of(dt)
    g = workloads.gen(27000 + 2 * DTS.index(dt) + relu)
    cases = [("small, ragged width", 37, 8 * vec + 2, False),
             ("large, aligned", (SMALL_CALL_BYTES // (3 * 4000 * dt.itemsize)) + 3, 4000, False)]
    if dt.itemsize == 2:
        cases += [("small, odd offsets", 29, 1001, True),
                  ("large, odd offsets", (SMALL_CALL_BYTES // (3 * 4001 * dt.itemsize)) + 3, 4001, True)]
    for what, rows, cols, odd in cases:
        say(f"gated {'reglu' if relu else 'swiglu'} dt={DT_ID[dt]} {what}: rows={rows} cols={cols}")
        gate0 = (workloads.randn([rows, cols], g) * 2).to(dt)
        up0 = (workloads.randn([rows, cols], g) * 2).to(dt)
        if odd:
            gate, up = at_odd_offset(gate0), at_odd_offset(up0)
            out = at_odd_offset(torch.zeros_like(gate0))
        else:
            gate, up, out = gate0.cuda(), up0.cuda(), torch.zeros_like(gate0, device="cuda")
        fn(gate, up, out=out)
        assert_close(out.cpu().double().numpy(), ref_fn(np_bits(gate0), np_bits(up0)), dt, what)


# ------------------------------------------------------ one-launch chain
@pytest.mark.parametrize("dt", DTS, ids=DT_ID.get)
def test_chain_launch_forms(kcr, dt):
    """The one-launch chain's kernel forms: the residual rows at 1 to 4
    vectors per lane (200, 300, 700 and 1000-1024 vectors), each in the
    deeply pipelined form (batches up to 64) and the lean one (larger
    batches), with layer counts below, at and past a whole number of
    pipeline groups (1 to 9 layers where the deep form pairs them); RoPE
    over two workgroups of query heads, and over two of key/value heads."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    from test_gpu_configs import check_chain
    vec = vec_of(dt)
    # (row vectors, SwiGLU vectors, layers, batch, query heads, KV heads, head_dim)
    forms = [(200, 300, 5, 3, 4, 2, 64), (300, 700, 2, 3, 4, 2, 64), (700, 1000, 5, 3, 4, 2, 64),
             (1024, 1500, 3, 3, 4, 2, 64),
             (200, 300, 3, 65, 80, 4, 64), (300, 700, 3, 65, 4, 2, 64), (700, 1000, 3, 65, 4, 2, 64),
             (1000, 257, 2, 65, 4, 2, 64)]
    # key/value heads over two workgroups (LPU lanes per head, 256 lanes each)
    kv = 16 if vec == 8 else 8
    forms.append((64, 256, 3, 2, kv, kv, 256))
    # the deep form at one vector per lane runs pairs of layers, the last
    # n % 4 layers one at a time: every remainder, with and without pairs
    forms += [(100, 200, n, 2, 4, 2, 64) for n in (1, 2, 3, 4, 6, 7, 9)]
    for i, (hv, iv, layers, batch, hq, hkv, dh) in enumerate(forms):
        hidden, inter = hv * vec, iv * vec
        say(f"chain dt={DT_ID[dt]} hidden={hidden} inter={inter} layers={layers} batch={batch} heads={hq}/{hkv}x{dh}")
        wl = workloads.decode_chain(layers=layers, batch=batch, ctx=20, dtype=dt,
                                    seed=28000 + 10 * i + DTS.index(dt), hidden=hidden, inter=inter,
                                    hq=hq, hkv=hkv, dh=dh, block_size=16)
        chain = DecodeChain(wl, "cuda", sentinel_cache=True)
        chain.step_one_launch()
        torch.cuda.synchronize()
        check_chain(wl, chain)

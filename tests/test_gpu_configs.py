"""GPU parity on the five workloads at their full sizes, and at the large
per-kernel shapes the benchmark times (same entry points, same launch
configuration), against the CPU fp64 oracle:

  1 batch-1 Qwen2.5-1.5B decode token (rmsnorm, rope_kvstore, swiglu)
  2 RMSNorm 512 x 2176, fp32 and bf16, 1% outlier rows x100
  3 prefill RoPE + paged store, 8 sequences of 128..2048 tokens
  4 SwiGLU of a fused gate_up [8192, 2 x 8960]
  5 the 28-layer batch-256 decode chain, replayed from a captured HIP graph

At the large shapes (including those of the NEXT rows the benchmark times:
the per-head Q/K norm, the clip norm, ReGLU and the wide-row kernel) the
oracle checks sampled rows/tokens one by one and whole-tensor properties
cover the rest (residual and V bit-exact, untouched cache slots still hold
the sentinel)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_close, assert_rope_close, check_rope, gpu_qkv, np_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kcr():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import kv_cache_rmsnorm_amd as k
    return k


def say(*a):
    print(*a, flush=True)


def f32eps(e):
    return float(np.float32(e))


def test_config1_decode_token(kcr):
    say("config 1: batch-1 decode token")
    wl = workloads.decode_token(seed=0)
    dev = torch.device("cuda")
    y = kcr.rmsnorm(wl["x"].to(dev), wl["w"].to(dev), wl["eps"])
    assert_close(y.cpu().double().numpy(),
                 oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), f32eps(wl["eps"])),
                 torch.bfloat16, "rmsnorm [1,1536]")
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], 128, wl["theta"])
    cache = wl["cache"].to(dev)
    qo = kcr.rope_kvstore(*gpu_qkv(wl), wl["positions"].to(dev), cos, sin, cache,
                          wl["slot_mapping"].to(dev))
    check_rope(wl["q"], wl["k"], wl["v"], wl["positions"], wl["cache"], wl["slot_mapping"],
               wl["theta"], qo.cpu(), cache.cpu(), torch.bfloat16, "config 1 rope")
    act = kcr.swiglu(wl["gate"].to(dev), wl["up"].to(dev))
    assert_close(act.cpu().double().numpy(), oracle.swiglu(np_bits(wl["gate"]), np_bits(wl["up"])),
                 torch.bfloat16, "swiglu [1,8960]")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_config2_rmsnorm(kcr, dt):
    say(f"config 2: rmsnorm 512x2176 {dt}")
    wl = workloads.rmsnorm_rows(rows=512, d=2176, dtype=dt, seed=0)
    y = kcr.rmsnorm(wl["x"].cuda(), wl["w"].cuda(), wl["eps"])
    ref = oracle.rmsnorm(np_bits(wl["x"]), np_bits(wl["w"]), f32eps(wl["eps"]))
    assert_close(y.cpu().double().numpy(), ref, workloads.as_dtype(dt), "config 2")


def test_config3_prefill(kcr):
    say("config 3: prefill rope + paged store, 8 seqs")
    wl = workloads.prefill(n_seqs=8, dtype="bf16", seed=0)
    assert 8 * 128 <= wl["qkv"].shape[0] <= 8 * 2048
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], wl["dh"], wl["theta"])
    cache = wl["cache"].cuda()
    qo = kcr.rope_kvstore(*gpu_qkv(wl), wl["positions"].cuda(), cos, sin, cache,
                          wl["slot_mapping"].cuda())
    check_rope(wl["q"], wl["k"], wl["v"], wl["positions"], wl["cache"], wl["slot_mapping"],
               wl["theta"], qo.cpu(), cache.cpu(), torch.bfloat16, "config 3")
    # round trip: gathering each sequence through its block table returns V
    c = cache.cpu()
    off = 0
    for L, bt in zip(wl["layout"].lens, wl["layout"].block_tables):
        got = oracle.paged_gather(np_bits(c), 1, bt.numpy(), L)
        assert np.array_equal(got, np.ascontiguousarray(np_bits(wl["v"][off:off + L])))
        off += L


def test_config4_swiglu(kcr):
    say("config 4: swiglu gate_up [8192, 17920]")
    wl = workloads.swiglu_fused(rows=8192, inter=8960, dtype="bf16", seed=0)
    out = kcr.swiglu_fused(wl["gate_up"].cuda())
    ref = oracle.swiglu(np_bits(wl["gate"]), np_bits(wl["up"]))
    assert_close(out.cpu().double().numpy(), ref, torch.bfloat16, "config 4")
    # ReGLU on the same fused buffer (the benchmark times both at this shape)
    gu = wl["gate_up"].cuda()
    out = kcr.reglu(gu[:, :8960], gu[:, 8960:])
    ref = oracle.reglu(np_bits(wl["gate"]), np_bits(wl["up"]))
    assert_close(out.cpu().double().numpy(), ref, torch.bfloat16, "config 4 reglu")


def test_config5_decode_chain_graph(kcr):
    """The benchmark's own step (DecodeChain, HIP graph replay), all 28
    layers at batch 256, against the oracle run layer by layer."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say("config 5: 28-layer decode chain, graph replay")
    wl = workloads.decode_chain(seed=0)
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    chain.capture()           # runs one eager warm-up step, then captures
    for L in chain.layers:    # reset the state the warm-up step changed
        L["cache"].view(torch.int16).fill_(-1)
    chain.reset_residual()
    torch.cuda.synchronize()
    chain.step_graph()
    torch.cuda.synchronize()
    check_chain(wl, chain)


def _chain_outputs(chain):
    """Bit views of everything one step writes: each layer's y_attn, q_out,
    y_mlp and act, the K/V cache rows at the step's slots, and h."""
    slots = chain.slot_mapping
    out = []
    for L in chain.layers:
        cache = L["cache"]
        rows = cache.view(2, -1, *cache.shape[3:])[:, slots]
        for t in (L["y_attn"], L["q_out"], L["y_mlp"], L["act"], rows):
            out.append(t.clone())
    out.append(chain.h.clone())
    return out


def _reset_chain(chain):
    for L in chain.layers:
        L["cache"].view(torch.int16 if L["cache"].element_size() == 2 else torch.int32).fill_(-1)
    chain.reset_residual()
    torch.cuda.synchronize()


@pytest.mark.parametrize("batch,form", [(256, "graph"), (1, "b1"), (256, "one")],
                         ids=["b256_graph_of_112", "b1_one_launch", "b256_one_launch"])
def test_graph_replays_match_eager(kcr, batch, form):
    """A captured step replayed three times, with eager work (cache and
    residual resets) and synchronizations between the replays: every replay
    writes the same bits as the eager step."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say(f"graph replays against the eager step, batch {batch}, {form}")
    wl = workloads.decode_chain(batch=batch, seed=7)
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    eager = {"graph": chain.step_eager, "b1": chain.step_b1, "one": chain.step_one_launch}[form]
    capture = {"graph": chain.capture, "b1": chain.capture_b1, "one": chain.capture_one_launch}[form]
    replay = capture().replay
    _reset_chain(chain)
    eager()
    torch.cuda.synchronize()
    ref = _chain_outputs(chain)
    for rep in range(3):
        _reset_chain(chain)
        replay()
        torch.cuda.synchronize()
        got = _chain_outputs(chain)
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i} differs"


def test_decode_chain_batch_one_launch(kcr):
    """The benchmark's decode step (28 layers, batch 256) in one launch of
    kcr_decode_chain_batch (its lean form, past 64 tokens), against the
    oracle run layer by layer."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say("batch-256 decode chain, one launch")
    wl = workloads.decode_chain(seed=0)
    assert wl["h"].shape[0] == 256
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    chain.step_one_launch()
    torch.cuda.synchronize()
    check_chain(wl, chain)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_decode_chain_batch_ragged(kcr, dt):
    """The one-launch chain at an odd batch (37 tokens) with two padding
    tokens (slot -1) and two positions outside the tables (-1 and max_pos),
    at other shapes (5 layers, hidden 512, intermediate 1408, 8 query / 2 KV
    heads of 64, block size 8), two steps in a row (the residual carries
    over)."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say(f"batch-37 decode chain with padding tokens, one launch, {dt}")
    wl = workloads.decode_chain(layers=5, batch=37, ctx=100, dtype=dt, seed=5, hidden=512, inter=1408,
                                hq=8, hkv=2, dh=64, block_size=8)
    wl["slot_mapping"][[3, 36]] = -1
    wl["positions"] = torch.randint(0, wl["max_pos"], (37,), generator=workloads.gen(6))
    wl["positions"][[10, 20]] = torch.tensor([-1, wl["max_pos"]])
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    chain.step_one_launch()
    torch.cuda.synchronize()
    h_after = check_chain(wl, chain)
    _reset_cache(chain)
    chain.step_one_launch()
    torch.cuda.synchronize()
    check_chain(dict(wl, h=bits_to_tensor(h_after, workloads.as_dtype(dt))), chain)


def test_decode_chain_batch_matches_b1(kcr):
    """Token b of a batched one-launch step writes the same bits as a
    batch-1 one-launch step of token b alone (no token's result depends on
    another's)."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say("batched one-launch chain against per-token batch-1 launches")
    wl = workloads.decode_chain(layers=3, batch=6, ctx=64, seed=11)
    wl["positions"] = torch.randint(0, wl["max_pos"], (6,), generator=workloads.gen(12))
    full = DecodeChain(wl, "cuda", sentinel_cache=True)
    full.step_one_launch()
    torch.cuda.synchronize()
    for b in (0, 5):
        one = dict(wl, h=wl["h"][b:b + 1], positions=wl["positions"][b:b + 1],
                   slot_mapping=wl["slot_mapping"][b:b + 1],
                   layers=[{k: (t[b:b + 1] if k in ("d_attn", "d_mlp", "qkv", "gate_up") else t)
                            for k, t in lw.items()} for lw in wl["layers"]])
        single = DecodeChain(one, "cuda", sentinel_cache=True)
        single.step_b1()
        torch.cuda.synchronize()
        assert torch.equal(single.h.view(torch.int16), full.h[b:b + 1].view(torch.int16)), f"token {b} h"
        s = int(wl["slot_mapping"][b])
        for i, (Lf, Ls) in enumerate(zip(full.layers, single.layers)):
            for name in ("y_attn", "q_out", "y_mlp", "act"):
                assert torch.equal(Ls[name].view(torch.int16), Lf[name][b:b + 1].view(torch.int16)), \
                    f"token {b} layer {i} {name}"
            cf, cs = (L["cache"].view(2, -1, *L["cache"].shape[3:]) for L in (Lf, Ls))
            assert torch.equal(cf[:, s].view(torch.int16), cs[:, s].view(torch.int16)), f"token {b} layer {i} cache"


@pytest.mark.parametrize("batch", [3, 70], ids=["deep", "lean"])
def test_decode_chain_shared_cache(kcr, batch):
    """Layers that all name one cache range: the last layer's K/V rows
    remain, as with the separate calls in order. The shared cache must equal,
    bit for bit, the last layer's own cache of a run with one cache per
    layer, every other output must match that run, and the V rows must equal
    those the separate calls leave."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say(f"one-launch chain, 5 layers sharing one cache, batch {batch}")
    wl = workloads.decode_chain(layers=5, batch=batch, ctx=40, seed=21 + batch, hidden=512, inter=1408,
                                hq=8, hkv=2, dh=64, block_size=8)
    wl["slot_mapping"][1] = -1  # a padding token stores nothing in any layer
    per_layer = DecodeChain(wl, "cuda", sentinel_cache=True)
    per_layer.step_one_launch()
    shared = DecodeChain(wl, "cuda", sentinel_cache=True)
    one = shared.layers[0]["cache"]
    for L in shared.layers:
        L["cache"] = one
    shared.step_one_launch()
    eager = DecodeChain(wl, "cuda", sentinel_cache=True)
    for L in eager.layers:
        L["cache"] = eager.layers[0]["cache"]
    eager.step_eager()
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)
    assert torch.equal(bits(one), bits(per_layer.layers[-1]["cache"])), "shared cache"
    assert torch.equal(bits(shared.h), bits(per_layer.h)), "residual"
    for i, (Ls, Lp) in enumerate(zip(shared.layers, per_layer.layers)):
        for name in ("y_attn", "q_out", "y_mlp", "act"):
            assert torch.equal(bits(Ls[name]), bits(Lp[name])), f"layer {i} {name}"
    assert torch.equal(bits(one[1]), bits(eager.layers[0]["cache"][1])), "V rows against the separate calls"


def _reset_cache(chain):
    for L in chain.layers:
        L["cache"].view(torch.int16 if L["cache"].element_size() == 2 else torch.int32).fill_(-1)


def test_decode_chain_b1_one_launch(kcr):
    """The batch-1 decode step's 28-layer chain in one launch
    (kcr_decode_chain_b1) against the oracle run layer by layer, twice in a
    row (the residual carries over)."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say("batch-1 decode chain, one launch")
    wl = workloads.decode_chain(batch=1, seed=3)
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    chain.step_b1()
    torch.cuda.synchronize()
    h_after = check_chain(wl, chain)
    # a second step continues from the updated residual
    for L in chain.layers:
        L["cache"].view(torch.int16).fill_(-1)
    wl2 = dict(wl, h=bits_to_tensor(h_after, torch.bfloat16))
    chain.step_b1()
    torch.cuda.synchronize()
    check_chain(wl2, chain)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_decode_chain_b1_dtypes_and_shapes(kcr, dt):
    """The one-launch batch-1 chain in every dtype at other shapes: 5 layers,
    hidden 512, intermediate 1408, 8 query / 2 KV heads of 64, block size 8."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say(f"batch-1 decode chain, one launch, {dt}")
    wl = workloads.decode_chain(layers=5, batch=1, ctx=100, dtype=dt, seed=4, hidden=512, inter=1408,
                                hq=8, hkv=2, dh=64, block_size=8)
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    chain.step_b1()
    torch.cuda.synchronize()
    check_chain(wl, chain)


@pytest.mark.parametrize("batch", [1, 3, 70])
def test_decode_chain_max_layers(kcr, batch):
    """The one-launch chain at the most layers its argument block holds (32):
    at batch 1 (b1 entry point), 3 (four-deep rings, pairs of layers per
    exchange) and 70 (two-deep rings, one exchange per layer); 32 layers are
    whole groups of either ring. Small shapes, bf16, every output against the
    oracle."""
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    say(f"decode chain, 32 layers, batch {batch}")
    wl = workloads.decode_chain(layers=32, batch=batch, ctx=40, seed=90 + batch, hidden=256, inter=512,
                                hq=4, hkv=2, dh=64, block_size=16)
    chain = DecodeChain(wl, "cuda", sentinel_cache=True)
    chain.step_b1() if batch == 1 else chain.step_one_launch()
    torch.cuda.synchronize()
    check_chain(wl, chain)


def bits_to_tensor(bits: np.ndarray, dt) -> torch.Tensor:
    """Inverse of np_bits: storage-convention numpy array -> CPU tensor."""
    if dt == torch.bfloat16:
        return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(bits.copy())


def check_chain(wl, chain):
    """Every layer's outputs of one step of `chain` against the oracle run
    layer by layer from wl["h"]; returns the oracle's final residual."""
    dt = wl["dtype"]
    ib = torch.int16 if dt.itemsize == 2 else torch.int32  # bit view; the sentinel is all ones
    eps = f32eps(wl["eps"])
    hq, hkv, dh, inter = wl["hq"], wl["hkv"], wl["dh"], wl["inter"]
    h = np_bits(wl["h"]).copy()
    pos, slots = wl["positions"].numpy(), wl["slot_mapping"].numpy()
    n_slots = wl["num_blocks"] * wl["block_size"]
    # a position outside the tables copies the token's query heads unrotated
    # and stores nothing; a negative slot (padding) stores nothing
    in_range = (pos >= 0) & (pos < wl["max_pos"])
    live = (slots >= 0) & in_range
    for i, (lw, L) in enumerate(zip(wl["layers"], chain.layers)):
        h, y_attn = oracle.add_rmsnorm(h, np_bits(lw["d_attn"]), np_bits(lw["w_attn"]), eps)
        q, k, v = workloads.qkv_views(lw["qkv"], hq, hkv, dh)
        q_rot, k_rot = oracle.rope_kvstore(np_bits(q), np_bits(k), np_bits(v), pos, wl["theta"],
                                           None, None)
        q_rot[~in_range] = q[torch.from_numpy(~in_range)].double().numpy()
        h, y_mlp = oracle.add_rmsnorm(h, np_bits(lw["d_mlp"]), np_bits(lw["w_mlp"]), eps)
        act = oracle.swiglu(np_bits(lw["gate_up"][:, :inter]), np_bits(lw["gate_up"][:, inter:]))
        assert_close(L["y_attn"].cpu().double().numpy(), y_attn, dt, f"layer {i} y_attn")
        assert_close(L["y_mlp"].cpu().double().numpy(), y_mlp, dt, f"layer {i} y_mlp")
        assert_rope_close(L["q_out"].cpu().double().numpy(), q_rot, dt, f"layer {i} q_out")
        assert_close(L["act"].cpu().double().numpy(), act, dt, f"layer {i} act")
        # cache: the named slots hold K_rot and V (padding tokens, slot < 0,
        # store nothing); every other slot keeps the sentinel
        flat = L["cache"].view(2, n_slots, hkv, dh)
        s_dev = chain.slot_mapping[torch.from_numpy(live).to(chain.slot_mapping.device)]
        k_got = flat[0][s_dev].cpu().double().numpy()
        assert_rope_close(k_got, k_rot[live], dt, f"layer {i} K slots")
        assert torch.equal(flat[1][s_dev].view(ib).cpu(), v[torch.from_numpy(live)].contiguous().view(ib))
        untouched = int((L["cache"].view(ib) == -1).sum())
        assert untouched == L["cache"].numel() - 2 * int(live.sum()) * hkv * dh, f"layer {i} stray writes"
    # the residual after 56 fused adds is bit-exact
    assert np.array_equal(np_bits(chain.h.cpu()), h), "residual stream after the step"
    return h


def test_large_rmsnorm_sampled(kcr):
    R, d = 131072, 2176
    for dt in ("bf16", "f32", "f16"):
        say(f"large rmsnorm [{R}, {d}] {dt}, sampled rows")
        wl = workloads.rmsnorm_rows(rows=R, d=d, dtype=dt, seed=0)
        y = kcr.rmsnorm(wl["x"].cuda(), wl["w"].cuda(), wl["eps"]).cpu()
        rng = np.random.default_rng(1)
        rows = np.unique(np.concatenate([[0, 1, R - 1], wl["outlier_rows"].numpy()[:50],
                                         rng.choice(R, 400, replace=False)]))
        ref = oracle.rmsnorm(np_bits(wl["x"][rows]), np_bits(wl["w"]), f32eps(wl["eps"]))
        assert_close(y[rows].double().numpy(), ref, workloads.as_dtype(dt), f"rows of {dt}")
        assert bool(torch.isfinite(y).all())


def test_large_add_rmsnorm_sampled(kcr):
    R, d = 131072, 1536
    say(f"large add_rmsnorm [{R}, {d}] bf16")
    wl = workloads.add_rmsnorm_rows(R, d, dtype="bf16", seed=0)
    x = wl["x"].cuda()
    delta = wl["delta"].cuda()
    y = kcr.add_rmsnorm(x, delta, wl["w"].cuda(), wl["eps"]).cpu()
    # every row's residual: bit-exact against torch's fp32 add rounded to bf16
    want = (wl["x"].cuda().float() + delta.float()).to(torch.bfloat16)
    assert torch.equal(x.view(torch.int16), want.view(torch.int16))
    rows = np.unique(np.concatenate([[0, R - 1], np.random.default_rng(2).choice(R, 400, replace=False)]))
    x_ref, y_ref = oracle.add_rmsnorm(np_bits(wl["x"][rows]), np_bits(wl["delta"][rows]),
                                      np_bits(wl["w"]), f32eps(wl["eps"]))
    assert np.array_equal(np_bits(x[rows].cpu()), x_ref)
    assert_close(y[rows].double().numpy(), y_ref, torch.bfloat16, "sampled rows")


def test_large_rope_sampled(kcr):
    say("large prefill rope + store, 64 seqs, sampled tokens")
    wl = workloads.prefill(n_seqs=64, dtype="bf16", seed=0)
    T = wl["qkv"].shape[0]
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], wl["dh"], wl["theta"])
    cache = wl["cache"].cuda()
    q, k, v = gpu_qkv(wl)
    slots = wl["slot_mapping"].cuda()
    qo = kcr.rope_kvstore(q, k, v, wl["positions"].cuda(), cos, sin, cache, slots)
    hkv, dh = wl["hkv"], wl["dh"]
    flat = cache.view(2, -1, hkv, dh)
    # V of every token bit-exact at its slot; all other slots untouched
    assert torch.equal(flat[1][slots].view(torch.int16), v.view(torch.int16))
    assert int((cache.view(torch.int16) == -1).sum()) == cache.numel() - 2 * T * hkv * dh
    toks = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(3).choice(T, 500, replace=False)]))
    q_rot, k_rot = oracle.rope_kvstore(np_bits(wl["q"][toks]), np_bits(wl["k"][toks]),
                                       np_bits(wl["v"][toks]), wl["positions"].numpy()[toks],
                                       wl["theta"], None, None)
    assert_rope_close(qo.cpu()[toks].double().numpy(), q_rot, torch.bfloat16, "sampled q_out")
    k_got = flat[0][slots[torch.from_numpy(toks).cuda()]].cpu().double().numpy()
    assert_rope_close(k_got, k_rot, torch.bfloat16, "sampled K slots")


def test_large_paged_gather_sampled(kcr):
    """The benchmark's gather shape: 256 sequences x 4096 cached positions of
    one decode-chain layer cache, every K/V row checked bit for bit against a
    torch index gather on the device, sampled rows against the oracle."""
    say("large paged gather 256 x 4096")
    wl = workloads.decode_chain(layers=1, seed=0)
    lay = wl["layout"]
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    cache = torch.randn(wl["cache_shape"], generator=g, device="cuda").to(torch.bfloat16)
    bt = torch.stack(lay.block_tables).cuda()
    lens = torch.full((len(lay.block_tables),), 4096, dtype=torch.int64, device="cuda")
    k, v = kcr.paged_kv_gather(cache, bt, lens, 4096)
    bs = wl["block_size"]
    pos = torch.arange(4096, device="cuda")
    slots = bt[:, pos // bs] * bs + pos % bs                      # [256, 4096]
    flat = cache.view(2, -1, wl["hkv"], wl["dh"])
    assert torch.equal(k.view(torch.int16), flat[0][slots].view(torch.int16))
    assert torch.equal(v.view(torch.int16), flat[1][slots].view(torch.int16))
    c = np_bits(cache.cpu())
    for b in (0, 131, 255):
        ref = oracle.paged_gather(c, 0, lay.block_tables[b].numpy(), 4096)
        assert np.array_equal(np_bits(k[b].cpu()), ref)


def test_large_qknorm_rope_sampled(kcr):
    """Per-head Q/K RMSNorm + RoPE + paged store at the benchmark's prefill
    shape (64 sequences), with non-unit norm weights."""
    say("large prefill qknorm + rope + store, 64 seqs, sampled tokens")
    wl = workloads.prefill(n_seqs=64, dtype="bf16", seed=0)
    T, hkv, dh = wl["qkv"].shape[0], wl["hkv"], wl["dh"]
    g = workloads.gen(11)
    wq = (1 + 0.2 * workloads.randn([dh], g)).to(torch.bfloat16)
    wk = (0.5 + torch.rand([dh], generator=g)).to(torch.bfloat16)
    eps = 1e-6
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], dh, wl["theta"])
    cache = wl["cache"].cuda()
    q, k, v = gpu_qkv(wl)
    slots = wl["slot_mapping"].cuda()
    qo = kcr.qknorm_rope_kvstore(q, k, v, wq.cuda(), wk.cuda(), eps, wl["positions"].cuda(), cos, sin,
                                 cache, slots)
    flat = cache.view(2, -1, hkv, dh)
    assert torch.equal(flat[1][slots].view(torch.int16), v.view(torch.int16))
    assert int((cache.view(torch.int16) == -1).sum()) == cache.numel() - 2 * T * hkv * dh
    toks = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(4).choice(T, 500, replace=False)]))
    q_rot, k_rot = oracle.qknorm_rope_kvstore(np_bits(wl["q"][toks]), np_bits(wl["k"][toks]),
                                              np_bits(wl["v"][toks]), np_bits(wq), np_bits(wk),
                                              f32eps(eps), wl["positions"].numpy()[toks], wl["theta"],
                                              None, None)
    assert_rope_close(qo.cpu()[toks].double().numpy(), q_rot, torch.bfloat16, "sampled q_out")
    k_got = flat[0][slots[torch.from_numpy(toks).cuda()]].cpu().double().numpy()
    assert_rope_close(k_got, k_rot, torch.bfloat16, "sampled K slots")


def test_large_clip_norm_sampled(kcr):
    """The DyHT clip norm at the benchmark's shape: [131072, 2176] bf16 with
    per-channel alpha and gamma."""
    R, d = 131072, 2176
    say(f"large clip norm [{R}, {d}] bf16, sampled rows")
    wl = workloads.rmsnorm_rows(rows=R, d=d, dtype="bf16", seed=0)
    g = workloads.gen(12)
    alpha = (0.5 * workloads.randn([d], g)).to(torch.bfloat16)
    gamma = wl["w"]
    y = kcr.clip_norm(wl["x"].cuda(), alpha.cuda(), gamma.cuda()).cpu()
    rows = np.unique(np.concatenate([[0, R - 1], wl["outlier_rows"].numpy()[:50],
                                     np.random.default_rng(5).choice(R, 400, replace=False)]))
    ref = oracle.clip_norm(np_bits(wl["x"][rows]).reshape(len(rows), 1, d), np_bits(alpha), np_bits(gamma))
    assert_close(y[rows].double().numpy(), ref.reshape(len(rows), d), torch.bfloat16, "sampled rows")
    assert bool((y.abs() <= gamma.abs().float().max() + 1e-6).all())


@pytest.mark.parametrize("rows,d", [(2048, 65536), (512, 262144)])
def test_large_wide_rmsnorm_sampled(kcr, rows, d):
    """The two-pass wide-row kernel at the benchmark's shapes: LDS-staged rows
    of 128 KB, and rows of 512 KB that are read twice."""
    say(f"large wide rmsnorm [{rows}, {d}] bf16, sampled rows")
    wl = workloads.rmsnorm_rows(rows=rows, d=d, dtype="bf16", seed=0)
    y = kcr.rmsnorm(wl["x"].cuda(), wl["w"].cuda(), wl["eps"]).cpu()
    pick = np.unique(np.concatenate([[0, rows - 1], wl["outlier_rows"].numpy()[:4],
                                     np.random.default_rng(6).choice(rows, 24, replace=False)]))
    ref = oracle.rmsnorm(np_bits(wl["x"][pick]), np_bits(wl["w"]), f32eps(wl["eps"]))
    assert_close(y[pick].double().numpy(), ref, torch.bfloat16, "sampled wide rows")


def test_large_wide_add_rmsnorm_sampled(kcr):
    """The residual-add form of the LDS-staged wide-row kernel at the
    benchmark's shape, [2048, 65536] bf16: the updated residual bit-exact and
    the normalised rows within tolerance, on sampled rows."""
    rows, d = 2048, 65536
    say(f"large wide add_rmsnorm [{rows}, {d}] bf16, sampled rows")
    wl = workloads.add_rmsnorm_rows(rows=rows, d=d, dtype="bf16", seed=3)
    x = wl["x"].cuda()
    y = kcr.add_rmsnorm(x, wl["delta"].cuda(), wl["w"].cuda(), wl["eps"]).cpu()
    pick = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(7).choice(rows, 30, replace=False)]))
    x_ref, y_ref = oracle.add_rmsnorm(np_bits(wl["x"][pick]), np_bits(wl["delta"][pick]), np_bits(wl["w"]),
                                      f32eps(wl["eps"]))
    assert np.array_equal(np_bits(x[torch.from_numpy(pick).cuda()].cpu()).view(np.uint8), x_ref.view(np.uint8))
    assert_close(y[pick].double().numpy(), y_ref, torch.bfloat16, "sampled wide add rows")

"""The Python binding's shape checks. The C ABI receives only pointers and
sizes, so a tensor smaller than the sizes passed with it would be read or
written past its end; the binding must refuse every such mismatch before
it calls the library. Each case here passes one wrong tensor and expects
ValueError (TypeError for a wrong index dtype), with the good call next to
it showing that the same arguments are otherwise accepted."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kcr():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import kv_cache_rmsnorm_amd as k
    return k


def t(*shape, dt=torch.bfloat16):
    return torch.randn(shape, device="cuda").to(dt)


def test_norm_shapes(kcr):
    x, w = t(4, 64), t(64)
    kcr.rmsnorm(x, w)
    with pytest.raises(ValueError):
        kcr.rmsnorm(x, t(32))                       # short weight
    with pytest.raises(ValueError):
        kcr.rmsnorm(x, w, out=t(3, 64))             # out with fewer rows
    with pytest.raises(ValueError):
        kcr.rmsnorm(x, w, out=t(4, 64, dt=torch.float32))
    kcr.add_rmsnorm(x, t(4, 64), w)
    with pytest.raises(ValueError):
        kcr.add_rmsnorm(x, t(2, 64), w)             # delta with fewer rows
    with pytest.raises(ValueError):
        kcr.add_rmsnorm(x, t(4, 64), w, out=t(4, 32))
    torch.cuda.synchronize()


def test_gated_shapes(kcr):
    g, u = t(3, 40), t(3, 40)
    kcr.swiglu(g, u)
    kcr.reglu(g, u)
    for fn in (kcr.swiglu, kcr.reglu):
        with pytest.raises(ValueError):
            fn(g, t(2, 40))                         # up with fewer rows
        with pytest.raises(ValueError):
            fn(g, u, out=t(3, 32))                  # out too narrow
    torch.cuda.synchronize()


def test_clip_norm_shapes(kcr):
    x = t(5, 2, 16)
    kcr.clip_norm(x, t(16), t(1))
    with pytest.raises(ValueError):
        kcr.clip_norm(x, t(8), t(16))               # alpha neither [d] nor [1]
    with pytest.raises(ValueError):
        kcr.clip_norm(x, t(16), t(16), out=t(4, 2, 16))
    torch.cuda.synchronize()


def _rope_args(T=3, hq=4, hkv=2, hd=16, nb=4, bs=4, max_pos=8):
    q, k, v = t(T, hq, hd), t(T, hkv, hd), t(T, hkv, hd)
    pos = torch.arange(T, device="cuda", dtype=torch.int64)
    slots = torch.arange(T, device="cuda", dtype=torch.int64)
    cos = torch.ones((max_pos, hd // 2), device="cuda")
    sin = torch.zeros((max_pos, hd // 2), device="cuda")
    cache = t(2, nb, bs, hkv, hd)
    return q, k, v, pos, cos, sin, cache, slots


def test_rope_shapes(kcr):
    q, k, v, pos, cos, sin, cache, slots = _rope_args()
    kcr.rope_kvstore(q, k, v, pos, cos, sin, cache, slots)
    bad = [
        dict(k=t(2, 2, 16)),                               # k with fewer tokens
        dict(v=t(3, 2, 8)),                                # v with another head_dim
        dict(positions=pos[:2]),                           # positions shorter than T
        dict(slot_mapping=slots[:1]),                      # slot_mapping shorter than T
        dict(cos=torch.ones((8, 4), device="cuda")),       # table narrower than head_dim / 2
        dict(sin=torch.zeros((4, 8), device="cuda")),      # sin shaped unlike cos
        dict(q_out=t(3, 4, 8)),                            # q_out too small
        dict(q_out=t(3, 4, 32)[..., :16]),                 # q_out not contiguous
    ]
    names = ["q", "k", "v", "positions", "cos", "sin", "kv_cache", "slot_mapping"]
    for change in bad:
        args = dict(zip(names, (q, k, v, pos, cos, sin, cache, slots)))
        args.update(change)
        with pytest.raises(ValueError):
            kcr.rope_kvstore(**args)
    with pytest.raises(TypeError):
        kcr.rope_kvstore(q, k, v, pos.to(torch.int32), cos, sin, cache, slots)
    w = t(16)
    kcr.qknorm_rope_kvstore(q, k, v, w, w, 1e-6, pos, cos, sin, cache, slots)
    with pytest.raises(ValueError):
        kcr.qknorm_rope_kvstore(q, k, v, t(8), w, 1e-6, pos, cos, sin, cache, slots)
    torch.cuda.synchronize()


def test_gather_shapes(kcr):
    cache = t(2, 6, 4, 2, 16)
    bt = torch.tensor([[0, 1], [2, 3]], device="cuda", dtype=torch.int64)
    lens = torch.tensor([8, 5], device="cuda", dtype=torch.int64)
    kcr.paged_kv_gather(cache, bt, lens, 8)
    with pytest.raises(ValueError):
        kcr.paged_kv_gather(cache, bt, lens[:1], 8)        # fewer lengths than sequences
    with pytest.raises(ValueError):
        kcr.paged_kv_gather(cache, bt, lens, 8, k_out=t(2, 4, 2, 16))
    with pytest.raises(ValueError):
        kcr.paged_kv_gather(cache, bt, lens, 8, v_out=t(2, 8, 2, 32)[..., :16])
    torch.cuda.synchronize()


def test_decode_chain_b1_shapes(kcr):
    import workloads
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    wl = workloads.decode_chain(layers=2, batch=1, ctx=40, seed=1, hidden=256, inter=512, hq=4, hkv=2,
                                dh=32, block_size=8)
    chain = DecodeChain(wl, "cuda", sentinel_cache=False)
    chain.step_b1()
    args = (chain.h, chain.positions, chain.slot_mapping, chain.cos, chain.sin, chain.eps, chain.hq, chain.hkv)
    for name, bad in (("act", t(1, 256)), ("q_out", t(1, 4, 16)), ("w_mlp", t(128)), ("qkv", t(1, 64))):
        layers = [dict(L) for L in chain.layers]
        layers[1][name] = bad
        with pytest.raises(ValueError):
            kcr.DecodeChainB1(layers, *args)
    with pytest.raises(ValueError):
        kcr.DecodeChainB1(chain.layers, chain.h, chain.positions.repeat(2), *args[2:])
    torch.cuda.synchronize()


def test_decode_chain_batch_shapes(kcr):
    import workloads
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    wl = workloads.decode_chain(layers=2, batch=3, ctx=40, seed=1, hidden=256, inter=512, hq=4, hkv=2,
                                dh=32, block_size=8)
    chain = DecodeChain(wl, "cuda", sentinel_cache=False)
    chain.step_one_launch()
    args = (chain.h, chain.positions, chain.slot_mapping, chain.cos, chain.sin, chain.eps, chain.hq, chain.hkv)
    for name, bad in (("d_attn", t(2, 256)), ("q_out", t(3, 4, 16)), ("gate_up", t(3, 1000)),
                      ("y_mlp", t(6, 256)[::2])):
        layers = [dict(L) for L in chain.layers]
        layers[0][name] = bad
        with pytest.raises(ValueError):
            kcr.DecodeChainBatch(layers, *args)
    with pytest.raises(ValueError):                     # one position for three tokens
        kcr.DecodeChainBatch(chain.layers, chain.h, chain.positions[:1], *args[2:])
    with pytest.raises(ValueError):                     # a batch-1 entry given three tokens
        kcr.DecodeChainB1(chain.layers, *args)
    with pytest.raises(ValueError):
        kcr.DecodeChainBatch(chain.layers, t(6, 256)[::2], *args[1:])
    torch.cuda.synchronize()

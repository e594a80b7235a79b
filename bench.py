#!/usr/bin/env python3
"""Benchmark of the fused per-token decode ops on one MI355X.

Workload (one "step"): the batched decode chain of a Qwen2.5-1.5B-shaped
model -- 28 layers x [add_rmsnorm, rope_kvstore, add_rmsnorm, swiglu] at
batch 256, every sequence with 4096 tokens already cached and decoding
position 4096, random block tables, bf16, hidden 1536, intermediate 8960,
12 query / 2 KV heads of 128. Inputs are seeded synthetic data, resident in
HBM before timing starts. The timed step is a captured HIP graph replay.

Prints ONE JSON line:
  value        algorithmic bytes of a step / step time (GB/s), whole job
  ms_per_step  decode-step fused-op latency (graph replay)
  roofline     the step's dominant kernel: the chain op with the largest
               kernel time per step (its per-launch time inside a captured
               graph of that op's 28 launches on the chain's buffers, from
               HIP events on the launch stream around graph replays, times
               its launches per step); its algorithmic bytes per launch /
               that time, the counter-measured traffic, a graph of plain
               copies of the same size, and every chain op's share and
               fraction beside it
  cpu_baseline the CPU fp64 oracle on a bounded sample of the same workload;
               per_config: the oracle at each parity-shape config, with
               every oracle thread and with one
  kernels      each kernel at its large shape on cold, rotated buffers
  ceiling      1 GiB device copies: the library's copy kernel and hipMemcpy
  decode_token_b1  per-op latency of the batch-1 decode token (per launch in
               a graph, and event-stamped durations, which include the
               stamps' own cost)
  decode_chain_b1  the 28-layer chain at batch 1: graph of 112 launches vs one launch
  decode_chain_b256_one_launch  the timed step's chain (batch 256) as one launch
               (residual, RoPE and SwiGLU workgroups side by side), beside the
               graph of 112 launches; its
               rate over its own algorithmic bytes (h read once per token)
               and over the counter-measured HBM traffic
  source_sha256    hash of the library's sources the line was measured with
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "achieved HBM GB/s (% of peak) per kernel; decode-step fused-op latency"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def events(n):
    """n timing events, each recorded once so that it exists."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    return evs


def timed_launch(kcr, fn, ev0, ev1):
    """Run fn (one kcr op) with the kernel's own start/end stamped on ev0/ev1."""
    kcr.time_next_launch(ev0, ev1)
    fn()


def kernel_stats(ms):
    ms = sorted(ms)
    return dict(n=len(ms), median_us=1e3 * statistics.median(ms), min_us=1e3 * ms[0],
                mean_us=1e3 * statistics.fmean(ms),
                p20_us=1e3 * ms[int(0.2 * (len(ms) - 1))], p80_us=1e3 * ms[int(0.8 * (len(ms) - 1))])


# ------------------------------------------------------------------ chain
def chain_ops(kcr, chain, L):
    return [
        ("add_rmsnorm", lambda: kcr.add_rmsnorm(chain.h, L["d_attn"], L["w_attn"], chain.eps, out=L["y_attn"])),
        ("rope_kvstore", lambda: kcr.rope_kvstore(L["q"], L["k"], L["v"], chain.positions, chain.cos,
                                                  chain.sin, L["cache"], chain.slot_mapping, q_out=L["q_out"])),
        ("add_rmsnorm", lambda: kcr.add_rmsnorm(chain.h, L["d_mlp"], L["w_mlp"], chain.eps, out=L["y_mlp"])),
        ("swiglu", lambda: kcr.swiglu(L["gate"], L["up"], out=L["act"])),
    ]


def instrumented_steps(kcr, chain, n_steps, prelude: int = 10):
    """Whole eager steps with every launch's kernel duration stamped at the
    kernel's own start and end; returns {op: [ms, ...]} and the per-step
    kernel-time sums. Each step is enqueued behind `prelude` replays of the
    captured step, so the GPU is still busy with them while the host enqueues
    the step's launches, which then run back to back as in the timed graph
    replays rather than spaced out by host launch time."""
    import torch
    per_op, sums = {}, []
    n_launch = 4 * len(chain.layers)
    ev = events(2 * n_launch)
    for _ in range(n_steps):
        for _ in range(prelude):
            chain.step_graph()
        names = []
        i = 0
        for L in chain.layers:
            for name, fn in chain_ops(kcr, chain, L):
                timed_launch(kcr, fn, ev[2 * i], ev[2 * i + 1])
                names.append(name)
                i += 1
        torch.cuda.synchronize()
        tot = 0.0
        for j, name in enumerate(names):
            ms = ev[2 * j].elapsed_time(ev[2 * j + 1])
            per_op.setdefault(name, []).append(ms)
            tot += ms
        sums.append(tot)
    return per_op, sums


# ------------------------------------------------------- large shapes
def large_shapes(kcr, iters: int):
    """Each kernel at its large shape, three rotated buffer sets (more than
    the 256 MB Infinity Cache holds), kernel durations from start/end stamps."""
    import torch
    import workloads
    from kv_cache_rmsnorm_amd.chain import norm_bytes, rope_bytes, swiglu_bytes
    dev = torch.device("cuda")
    out = {}

    def run(name, nbytes, fns, shape_desc):
        ev = events(2 * iters)
        # warm-up: about 150 ms of the same launches, so clocks have settled
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < 0.15 or i < 4:
            fns[i % len(fns)]()
            i += 1
            if i % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        for i in range(iters):
            timed_launch(kcr, fns[i % len(fns)], ev[2 * i], ev[2 * i + 1])
        torch.cuda.synchronize()
        st = kernel_stats([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(iters)])
        gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
        out[name] = dict(shape=shape_desc, bytes=nbytes, **{k: round(v, 3) for k, v in st.items()},
                         gbs=round(gbs, 1), frac_of_peak=round(gbs / PEAK_GBS, 4))
        log(f"{name}: {st['median_us']:.1f} us median, {gbs:.0f} GB/s ({100 * gbs / PEAK_GBS:.1f}% of peak)")

    R = 131072
    for dt, tag in ((torch.bfloat16, "bf16"), (torch.float32, "f32"), (torch.float16, "f16")):
        wl = workloads.rmsnorm_rows(rows=R, d=2176, dtype=tag, seed=0)
        xs = [wl["x"].to(dev)]
        xs += [xs[0].clone() for _ in range(2)]
        ys = [torch.empty_like(xs[0]) for _ in range(3)]
        w = wl["w"].to(dev)
        fns = [lambda i=i: kcr.rmsnorm(xs[i], w, wl["eps"], out=ys[i]) for i in range(3)]
        run(f"rmsnorm_{tag}", norm_bytes(R, 2176, xs[0].element_size(), False), fns, f"[{R}, 2176] {tag}")
        del xs, ys, wl
    # rows wider than the register-resident engine: the two-pass kernel,
    # LDS-staged (65536 bf16 = 128 KB rows) and re-reading (262144 bf16)
    for rows, d, add, name in ((2048, 65536, False, "rmsnorm_bf16_wide_staged"),
                               (512, 262144, False, "rmsnorm_bf16_wide_reread"),
                               (2048, 65536, True, "add_rmsnorm_bf16_wide_staged")):
        if add:
            wl = workloads.add_rmsnorm_rows(rows, d, dtype="bf16", seed=0)
            xs = [wl["x"].to(dev) for _ in range(3)]
            ds = [wl["delta"].to(dev) for _ in range(3)]
        else:
            wl = workloads.rmsnorm_rows(rows=rows, d=d, dtype="bf16", seed=0)
            xs = [wl["x"].to(dev)]
            xs += [xs[0].clone() for _ in range(2)]
        ys = [torch.empty_like(xs[0]) for _ in range(3)]
        w = wl["w"].to(dev)
        if add:
            fns = [lambda i=i: kcr.add_rmsnorm(xs[i], ds[i], w, wl["eps"], out=ys[i]) for i in range(3)]
        else:
            fns = [lambda i=i: kcr.rmsnorm(xs[i], w, wl["eps"], out=ys[i]) for i in range(3)]
        run(name, norm_bytes(rows, d, 2, add), fns, f"[{rows}, {d}] bf16")
        del xs, ys, wl
        if add:
            del ds
    # DyHT clip norm on the same rows as RMSNorm bf16, per-channel alpha and gamma
    wl = workloads.rmsnorm_rows(rows=R, d=2176, dtype="bf16", seed=0)
    xs = [wl["x"].to(dev)]
    xs += [xs[0].clone() for _ in range(2)]
    ys = [torch.empty_like(xs[0]) for _ in range(3)]
    alpha = torch.full((2176,), 0.5, dtype=torch.bfloat16, device=dev)
    gamma = wl["w"].to(dev)
    fns = [lambda i=i: kcr.clip_norm(xs[i], alpha, gamma, out=ys[i]) for i in range(3)]
    run("clip_norm_bf16", 2 * R * 2176 * 2 + 2 * 2176 * 2, fns, f"[{R}, 2176] bf16, per-channel alpha, gamma")
    del xs, ys, wl
    wl = workloads.add_rmsnorm_rows(R, 1536, dtype="bf16", seed=0)
    xs = [wl["x"].to(dev) for _ in range(3)]
    ds = [wl["delta"].to(dev) for _ in range(3)]
    ys = [torch.empty_like(xs[0]) for _ in range(3)]
    w = wl["w"].to(dev)
    fns = [lambda i=i: kcr.add_rmsnorm(xs[i], ds[i], w, wl["eps"], out=ys[i]) for i in range(3)]
    run("add_rmsnorm_bf16", norm_bytes(R, 1536, 2, True), fns, f"[{R}, 1536] bf16")
    del xs, ds, ys, wl
    wl = workloads.prefill(n_seqs=64, dtype="bf16", seed=0)
    T = wl["qkv"].shape[0]
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], wl["dh"], wl["theta"])
    qkvs = [wl["qkv"].to(dev)]
    qkvs += [qkvs[0].clone() for _ in range(2)]
    views = [workloads.qkv_views(b, wl["hq"], wl["hkv"], wl["dh"]) for b in qkvs]
    cache = torch.empty(list(wl["cache"].shape), dtype=torch.bfloat16, device=dev)
    pos, slots = wl["positions"].to(dev), wl["slot_mapping"].to(dev)
    qo = [torch.empty((T, wl["hq"], wl["dh"]), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    fns = [lambda i=i: kcr.rope_kvstore(*views[i], pos, cos, sin, cache, slots, q_out=qo[i]) for i in range(3)]
    nb = rope_bytes(T, wl["hq"], wl["hkv"], wl["dh"], 2, int(torch.unique(wl["positions"]).numel()))
    run("rope_kvstore_bf16", nb, fns, f"64 seqs, T={T}, 12q/2kv x128, bf16")
    wq = torch.ones(wl["dh"], dtype=torch.bfloat16, device=dev)
    wk = torch.ones(wl["dh"], dtype=torch.bfloat16, device=dev)
    fns = [lambda i=i: kcr.qknorm_rope_kvstore(*views[i], wq, wk, 1e-6, pos, cos, sin, cache, slots,
                                               q_out=qo[i]) for i in range(3)]
    run("qknorm_rope_kvstore_bf16", nb + 2 * wl["dh"] * 2, fns,
        f"64 seqs, T={T}, 12q/2kv x128, per-head Q/K RMSNorm, bf16")
    del qkvs, views, cache, qo, wl
    # paged gather: one decode-chain layer cache read back for 256 sequences x 4096 positions
    B, L, bs, hkv, dh = 256, 4096, 16, 2, 128
    g = workloads.gen(0)
    nbps = L // bs
    N = B * (nbps + 1) + 64
    bt = torch.randperm(N, generator=g)[:B * nbps].view(B, nbps).to(dev)
    lens = torch.full((B,), L, dtype=torch.int64, device=dev)
    cache = torch.empty((2, N, bs, hkv, dh), dtype=torch.bfloat16, device=dev)
    outs = [(torch.empty((B, L, hkv, dh), dtype=torch.bfloat16, device=dev),
             torch.empty((B, L, hkv, dh), dtype=torch.bfloat16, device=dev)) for _ in range(3)]
    fns = [lambda i=i: kcr.paged_kv_gather(cache, bt, lens, L, k_out=outs[i][0], v_out=outs[i][1])
           for i in range(3)]
    run("paged_kv_gather_bf16", 2 * 2 * B * L * hkv * dh * 2 + B * nbps * 8 + B * 8, fns,
        f"{B} seqs x {L} positions, 2 kv heads x128, bf16")
    del cache, outs, bt, lens
    wl = workloads.swiglu_fused(rows=8192, inter=8960, dtype="bf16", seed=0)
    gus = [wl["gate_up"].to(dev)]
    gus += [gus[0].clone() for _ in range(2)]
    outs = [torch.empty((8192, 8960), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    fns = [lambda i=i: kcr.swiglu(gus[i][:, :8960], gus[i][:, 8960:], out=outs[i]) for i in range(3)]
    run("swiglu_bf16", swiglu_bytes(8192, 8960, 2), fns, "gate_up [8192, 17920] -> [8192, 8960] bf16")
    fns = [lambda i=i: kcr.reglu(gus[i][:, :8960], gus[i][:, 8960:], out=outs[i]) for i in range(3)]
    run("reglu_bf16", swiglu_bytes(8192, 8960, 2), fns, "gate_up [8192, 17920] -> [8192, 8960] bf16")
    del gus, outs, wl
    torch.cuda.empty_cache()
    return out


def chain_op_bytes(chain) -> dict:
    """Algorithmic bytes per launch of each chain op at the chain's shape."""
    from kv_cache_rmsnorm_amd.chain import norm_bytes, rope_bytes, swiglu_bytes
    import torch
    B, hid, inter = chain.h.shape[0], chain.hidden, chain.inter
    s = chain.h.element_size()
    distinct = int(torch.unique(chain.positions).numel())
    return dict(add_rmsnorm=norm_bytes(B, hid, s, True),
                rope_kvstore=rope_bytes(B, chain.hq, chain.hkv, chain.dh, s, distinct),
                swiglu=swiglu_bytes(B, inter, s))


def chain_roofline(chain, op_graph: dict, per_op: dict, n_steps: int, copy_us: dict) -> dict:
    """The roofline object for the step's dominant kernel: the chain op with
    the largest kernel time per step. A launch's time is its per-launch time
    inside a captured graph of that op's 28 launches on the chain's buffers
    (HIP events on the launch stream around graph replays), which matches
    the rocprofv3 trace of the timed replays; HIP events stamped at a single
    kernel's start and end have a floor near 4 us on this part, so those
    (per_op, from whole eager steps) are reported beside it only. Every
    chain op is listed with its launches, time share and fraction of peak."""
    B, hid, inter = chain.h.shape[0], chain.hidden, chain.inter
    nbytes = chain_op_bytes(chain)
    shapes = dict(add_rmsnorm=f"x, delta [{B}, {hid}] bf16 -> x, y",
                  rope_kvstore=f"{B} tokens, {chain.hq}q/{chain.hkv}kv heads x{chain.dh}, bf16, paged store",
                  swiglu=f"gate_up [{B}, {2 * inter}] -> [{B}, {inter}] bf16")
    in_graph = dict(add_rmsnorm=(op_graph["add_rmsnorm"] + op_graph["add_rmsnorm_2"]) / 2,
                    rope_kvstore=op_graph["rope_kvstore"], swiglu=op_graph["swiglu"])
    ops = {}
    for op, v in per_op.items():
        us = in_graph[op]
        n = len(v) / n_steps
        gbs = nbytes[op] / (us * 1e-6) / 1e9
        ops[op] = dict(shape=shapes[op], launches_per_step=n, bytes_per_launch=nbytes[op],
                       mean_us=round(us, 3), us_per_step=round(us * n, 2), achieved_gbs=round(gbs, 1),
                       frac=round(gbs / PEAK_GBS, 4),
                       size_matched_copy_us=round(copy_us[op], 3),
                       frac_of_size_matched_copy=round(copy_us[op] / us, 4),
                       event_stamped_mean_us=round(1e3 * statistics.fmean(v), 3))
    total = sum(o["us_per_step"] for o in ops.values())
    for o in ops.values():
        o["share_of_kernel_time"] = round(o["us_per_step"] / total, 4)
    dom = max(ops, key=lambda k: ops[k]["us_per_step"])
    d = ops[dom]
    traffic, note = counter_traffic(dom)
    roof = dict(bound="hbm", kernel=dom,
                selected_by="largest kernel time per step (per-launch time in a graph of the op's launches "
                            "x launches per step)",
                shape=d["shape"], bytes_per_launch=d["bytes_per_launch"], mean_us=d["mean_us"],
                mean_us_method="HIP events on the launch stream around replays of a captured graph of the op's "
                               "28 launches on the chain's buffers, per launch",
                launches_per_step=d["launches_per_step"], share_of_kernel_time=d["share_of_kernel_time"],
                achieved=d["achieved_gbs"], peak=PEAK_GBS, unit="GB/s", frac=d["frac"], traffic=traffic,
                size_matched_copy_us=d["size_matched_copy_us"],
                size_matched_copy_note="per-launch time of a graph of 28 plain copies moving the same bytes "
                                       "(half read, half written): what any kernel of this size attains in a graph",
                frac_of_size_matched_copy=d["frac_of_size_matched_copy"],
                traffic_source=f"{COUNTER_PROFILE} (rocprofv3 FETCH_SIZE + WRITE_SIZE of bench.py --pmc-pass, "
                               f"scaled by the copy kernel's counts)",
                chain_ops=ops)
    if note:
        roof["traffic_note"] = note
    return roof


def graph_copy_us(kcr, nbytes: int, n_launch: int, reps: int) -> float:
    """Per-launch time of a captured graph of n_launch copies that each move
    `nbytes` (nbytes / 2 read, nbytes / 2 written) on their own buffers: the
    attainable rate of a kernel of that size inside a graph."""
    import torch
    half = (nbytes // 2 + 15) // 16 * 16
    srcs = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(n_launch)]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(n_launch)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for a, b in zip(dsts, srcs):
            kcr.copy_(a, b)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for a, b in zip(dsts, srcs):
            kcr.copy_(a, b)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = events(2)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * n_launch)
    del g, srcs, dsts
    return us


def copy_equivalent_step_us(kcr, chain, reps: int) -> float:
    """Step time of a captured graph of 112 plain copies in the chain's
    order, each moving the bytes of the chain op at its place (half read,
    half written) on buffers of its own: what a graph of launches of these
    sizes attains on this device."""
    import torch
    nb = chain_op_bytes(chain)
    order = ["add_rmsnorm", "rope_kvstore", "add_rmsnorm", "swiglu"] * len(chain.layers)
    pairs = []
    for op in order:
        half = (nb[op] // 2 + 15) // 16 * 16
        pairs.append((torch.empty(half, dtype=torch.uint8, device="cuda"),
                      torch.empty(half, dtype=torch.uint8, device="cuda")))

    def step():
        for a, b in pairs:
            kcr.copy_(a, b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = events(2)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del g, pairs
    torch.cuda.empty_cache()
    return us


def graph_op_us(kcr, chain, reps: int):
    """Per-launch time of each op inside a captured graph of its 28 launches
    (one per layer, the chain's shapes and buffers), unprofiled."""
    import torch
    out = {}
    for k, name in enumerate(("add_rmsnorm", "rope_kvstore", "add_rmsnorm_2", "swiglu")):
        fns = [chain_ops(kcr, chain, L)[k][1] for L in chain.layers]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for f in fns:
                f()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = events(2)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / (reps * len(fns))
        del g
    return out


def rmsnorm_sweep(kcr, reps: int):
    """RMSNorm over [2 x 256, D] rows, the microbenchmark shape of the csdn
    page "Qwen3 from scratch (4-2): RMSNorm with Triton", section
    "performance comparison" (D = 128 ... 8196; FP32, FP16, BF16). Each point
    is the per-launch time inside a captured graph of 64 launches over 16
    rotated buffer sets, so it includes the graph's per-node launch cost;
    GB/s counts the algorithmic bytes (x read, y written, w once)."""
    import torch
    from kv_cache_rmsnorm_amd.chain import norm_bytes
    rows, sets, launches = 512, 16, 64
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    out = {}
    for dt, tag in ((torch.float32, "f32"), (torch.float16, "f16"), (torch.bfloat16, "bf16")):
        out[tag] = {}
        for d in (128, 256, 512, 1024, 1536, 2048, 2176, 4096, 8192, 8196):
            xs = [torch.randn((rows, d), generator=g, device="cuda").to(dt) for _ in range(sets)]
            ys = [torch.empty_like(x) for x in xs]
            w = torch.randn((d,), generator=g, device="cuda").to(dt)
            fns = [lambda i=i: kcr.rmsnorm(xs[i % sets], w, 1e-6, out=ys[i % sets]) for i in range(launches)]
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for f in fns:
                    f()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for f in fns:
                    f()
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            e0, e1 = events(2)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * launches)
            nb = norm_bytes(rows, d, xs[0].element_size(), False)
            out[tag][str(d)] = dict(us=round(us, 3), gbs=round(nb / (us * 1e-6) / 1e9, 1))
            del graph, xs, ys
        log(f"sweep [512, D] {tag}: " + ", ".join(f"{d}:{v['us']:.2f}us/{v['gbs']:.0f}GB/s"
                                                 for d, v in out[tag].items()))
    return out


def decode_token_latency(kcr, reps: int):
    """The batch-1 decode token (x[1,1536], Q[1,12,128] / K,V[1,2,128] at
    position 37 into slot 597, gate/up[1,8960]; bf16): each op's time per
    launch inside a captured graph of 64 back-to-back launches (which
    includes the graph's per-node cost), and its kernel duration stamped by
    HIP events at the kernel's own start and end (median of 200). At this
    size the data sits in cache, so latency, not GB/s, is the figure."""
    import torch
    import workloads
    dev = torch.device("cuda")
    wl = workloads.decode_token(seed=0)
    x, w = wl["x"].to(dev), wl["w"].to(dev)
    y = torch.empty_like(x)
    h = x.clone()
    delta = wl["gate"][:, :1536].contiguous().to(dev)
    q, k, v = wl["q"].to(dev), wl["k"].to(dev), wl["v"].to(dev)
    pos, slots = wl["positions"].to(dev), wl["slot_mapping"].to(dev)
    cos, sin = kcr.rope_cos_sin(wl["max_pos"], 128, wl["theta"], device=dev)
    cache = wl["cache"].to(dev)
    q_out = torch.empty_like(q)
    gate, up = wl["gate"].to(dev), wl["up"].to(dev)
    act = torch.empty_like(gate)
    ops = {
        "rmsnorm": lambda: kcr.rmsnorm(x, w, wl["eps"], out=y),
        "add_rmsnorm": lambda: kcr.add_rmsnorm(h, delta, w, wl["eps"], out=y),
        "rope_kvstore": lambda: kcr.rope_kvstore(q, k, v, pos, cos, sin, cache, slots, q_out=q_out),
        "swiglu": lambda: kcr.swiglu(gate, up, out=act),
    }
    out = {}
    for name, fn in ops.items():
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(64):
                fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = events(2)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        in_graph = e0.elapsed_time(e1) * 1e3 / (reps * 64)
        del g
        ev = events(400)
        for i in range(200):
            timed_launch(kcr, fn, ev[2 * i], ev[2 * i + 1])
        torch.cuda.synchronize()
        st = kernel_stats([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(200)])
        out[name] = dict(in_graph_us_per_launch=round(in_graph, 3),
                         event_stamped_median_us=round(st["median_us"], 3),
                         event_stamped_p20_us=round(st["p20_us"], 3), event_stamped_p80_us=round(st["p80_us"], 3))
    out["note"] = ("event_stamped_*: HIP events recorded at the kernel's own start and end of single "
                   "launches with the GPU otherwise idle; at this size the stamps' own cost dominates, "
                   "so the per-launch time inside a graph (in_graph_us_per_launch) is the latency figure")
    log("decode token (batch 1): " + ", ".join(f"{k} {v['in_graph_us_per_launch']:.2f} us/launch in graph, "
                                               f"{v['event_stamped_median_us']:.2f} us event-stamped"
                                               for k, v in out.items() if k != "note"))
    return out


def decode_chain_one_launch(kcr, chain, graph_us: float, reps: int):
    """The benchmark's step (batch 256) as one launch of
    kcr_decode_chain_batch: all 28 layers' ops, with the same results as the
    separate calls in order, on the same buffers as the graph of 112 launches. Step time
    from events over `reps` replays of a captured one-node graph; the
    kernel's own duration from events stamped at its start and end."""
    import torch
    by = chain.bytes_per_step()
    nb, nb_one = by["step"], by["one_launch_step"]
    chain.capture_one_launch()
    for _ in range(5):
        chain.graph_one.replay()
    torch.cuda.synchronize()
    e0, e1 = events(2)
    e0.record()
    for _ in range(reps):
        chain.graph_one.replay()
    e1.record()
    torch.cuda.synchronize()
    one_us = e0.elapsed_time(e1) * 1e3 / reps
    ev = events(2)
    samples = []
    for _ in range(20):
        kcr.time_next_launch(ev[0], ev[1])
        chain.step_one_launch()
        torch.cuda.synchronize()
        samples.append(ev[0].elapsed_time(ev[1]) * 1e3)
    traffic, note = counter_traffic("one_launch_b256")
    res = dict(graph_step_bytes=nb, one_launch_bytes=nb_one,
               one_launch_bytes_note="the graph step's algorithmic bytes less the residual's re-reads "
                                     "(h stays in registers: read once per token, not once per add) and "
                                     "less the per-layer re-reads of positions, slots and cos/sin rows",
               graph_112_launches_us=round(graph_us, 2), one_launch_us=round(one_us, 2),
               one_launch_event_stamped_median_us=round(statistics.median(samples), 2),
               one_launch_gbs=round(nb_one / (one_us * 1e-6) / 1e9, 1),
               one_launch_frac_of_peak=round(nb_one / (one_us * 1e-6) / 1e9 / PEAK_GBS, 4),
               counter_traffic_bytes=traffic,
               counter_traffic_gbs=round(traffic / (one_us * 1e-6) / 1e9, 1) if traffic else None,
               counter_traffic_frac_of_peak=round(traffic / (one_us * 1e-6) / 1e9 / PEAK_GBS, 4) if traffic else None,
               speedup=round(graph_us / one_us, 2))
    if note:
        res["counter_traffic_note"] = note
    log(f"batch-256 chain in one launch: {one_us:.1f} us/step ({res['one_launch_gbs']} GB/s of its own "
        f"algorithmic bytes), graph of 112 launches {graph_us:.1f} us/step")
    return res


def decode_chain_b1(kcr, reps: int):
    """The 28-layer chain at batch 1 (the decode token of a single sequence
    at position 4096): one step as a captured graph of the 112 separate
    launches, and as the single launch of kcr_decode_chain_b1 (same ops,
    same order, one workgroup), also replayed from a captured graph. Step
    time from events over `reps` replays; the single launch's kernel
    duration also from events stamped at its start and end."""
    import torch
    import workloads
    from kv_cache_rmsnorm_amd.chain import DecodeChain
    chain = DecodeChain(workloads.decode_chain(batch=1), "cuda", sentinel_cache=False)
    nb = chain.bytes_per_step()["step"]
    chain.capture()

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = events(2)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    graph_us = timed(chain.step_graph)
    chain.capture_b1()
    one_us = timed(chain.graph_b1.replay)
    ev = events(2)
    samples = []
    for _ in range(20):
        kcr.time_next_launch(ev[0], ev[1])
        chain.step_b1()
        torch.cuda.synchronize()
        samples.append(ev[0].elapsed_time(ev[1]) * 1e3)
    res = dict(step_bytes=nb, graph_112_launches_us=round(graph_us, 2), one_launch_us=round(one_us, 2),
               one_launch_kernel_median_us=round(statistics.median(samples), 2),
               one_launch_gbs=round(nb / (one_us * 1e-6) / 1e9, 1),
               speedup=round(graph_us / one_us, 2))
    log(f"batch-1 chain: graph of 112 launches {graph_us:.1f} us/step, one launch {one_us:.1f} us/step "
        f"({res['one_launch_gbs']} GB/s)")
    del chain
    torch.cuda.empty_cache()
    return res


def launch_floor(kcr, n_launch: int, reps: int):
    """Per-node time of a captured graph of n_launch minimal launches (a
    16-byte copy): what one graph node costs with (almost) no work."""
    import torch
    a = torch.zeros(4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kcr.copy_(b, a)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_launch):
            kcr.copy_(b, a)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = events(2)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n_launch)


def copy_ceiling(kcr, iters: int):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(generator=torch.Generator(device="cuda").manual_seed(0))
    dsts = [torch.empty_like(src) for _ in range(2)]
    ev = events(2 * iters)
    kcr.copy_(dsts[0], src)
    torch.cuda.synchronize()
    for i in range(iters):
        timed_launch(kcr, lambda i=i: kcr.copy_(dsts[i % 2], src), ev[2 * i], ev[2 * i + 1])
    torch.cuda.synchronize()
    st = kernel_stats([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(iters)])
    e0, e1 = events(2)
    e0.record()
    for i in range(iters):
        dsts[i % 2].copy_(src)
    e1.record()
    torch.cuda.synchronize()
    memcpy_ms = e0.elapsed_time(e1) / iters
    res = dict(bytes_moved=2 * n, copy_kernel_gbs=round(2 * n / (st["median_us"] * 1e-6) / 1e9, 1),
               copy_kernel_us=round(st["median_us"], 2),
               hip_memcpy_gbs=round(2 * n / (memcpy_ms * 1e-3) / 1e9, 1))
    log(f"copy ceiling: kernel {res['copy_kernel_gbs']} GB/s, hipMemcpy {res['hip_memcpy_gbs']} GB/s")
    del src, dsts
    return res


# --------------------------------------------------------- CPU baseline
def cpu_baseline_run(wl, bytes_per_step, budget_s: float):
    import numpy as np
    import torch
    import oracle

    def bits(t):
        t = t.contiguous() if t.dim() == 1 else t
        return t.view(torch.int16).numpy().view(np.uint16)

    threads = oracle.num_threads()
    eps = float(np.float32(wl["eps"]))
    hq, hkv, dh = wl["hq"], wl["hkv"], wl["dh"]
    layers = [dict(w_attn=bits(L["w_attn"]), w_mlp=bits(L["w_mlp"]), d_attn=bits(L["d_attn"]),
                   d_mlp=bits(L["d_mlp"]),
                   q=bits(L["qkv"][:, : hq * dh].unflatten(1, (hq, dh))),
                   k=bits(L["qkv"][:, hq * dh:(hq + hkv) * dh].unflatten(1, (hkv, dh))),
                   v=bits(L["qkv"][:, (hq + hkv) * dh:].unflatten(1, (hkv, dh))),
                   gate=bits(L["gate_up"][:, : wl["inter"]]), up=bits(L["gate_up"][:, wl["inter"]:]))
              for L in wl["layers"]]
    cache = np.zeros(wl["cache_shape"], dtype=np.uint16)  # one shared, lazily mapped cache
    pos, slots = wl["positions"].numpy(), wl["slot_mapping"].numpy()
    h = bits(wl["h"]).copy()
    steps, t0 = 0, time.perf_counter()
    while True:
        for L in layers:
            h, _ = oracle.add_rmsnorm(h, L["d_attn"], L["w_attn"], eps)
            oracle.rope_kvstore(L["q"], L["k"], L["v"], pos, wl["theta"], cache, slots,
                                block_size=wl["block_size"])
            h, _ = oracle.add_rmsnorm(h, L["d_mlp"], L["w_mlp"], eps)
            oracle.swiglu(L["gate"], L["up"])
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (steps + 1) / steps > 3 * budget_s:
            break
    gbs = steps * bytes_per_step / el / 1e9
    # the same oracle on one thread, over one layer-step slice (~1/16 of the time)
    oracle.set_num_threads(1)
    h1 = bits(wl["h"]).copy()
    t1 = time.perf_counter()
    n1 = 0
    while True:
        L = layers[n1 % len(layers)]
        h1, _ = oracle.add_rmsnorm(h1, L["d_attn"], L["w_attn"], eps)
        oracle.rope_kvstore(L["q"], L["k"], L["v"], pos, wl["theta"], cache, slots,
                            block_size=wl["block_size"])
        h1, _ = oracle.add_rmsnorm(h1, L["d_mlp"], L["w_mlp"], eps)
        oracle.swiglu(L["gate"], L["up"])
        n1 += 1
        if time.perf_counter() - t1 >= budget_s / 4:
            break
    el1 = time.perf_counter() - t1
    oracle.set_num_threads(threads)
    gbs1 = n1 * (bytes_per_step / len(layers)) / el1 / 1e9
    return dict(value=round(gbs, 3), unit="GB/s", cores=threads, kind="oracle",
                one_thread_value=round(gbs1, 3),
                one_thread_sample=f"{n1} layer(s) of the same chain on 1 thread ({el1:.1f} s)",
                cpu_model=cpu_model(),
                sample=f"{steps} full step(s) of the same 28-layer, batch-256 chain "
                       f"({steps * 112} op calls, {el:.1f} s); one shared cache array stands in "
                       f"for the 28 per-layer caches (only the 256 named slots are touched)",
                seconds=round(el, 2), ms_per_step=round(1e3 * el / steps, 1))


def cpu_configs_run():
    """The oracle at each parity-shape config (the batch-1 decode token's
    three ops; RMSNorm [512, 2176] in fp32 and bf16; the 8-sequence prefill
    RoPE + store; SwiGLU [8192, 2 x 8960]), timed once with every oracle
    thread and once with one thread."""
    import numpy as np
    import torch
    import oracle
    import workloads

    def npb(t):
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    tok = {k: (npb(v) if isinstance(v, torch.Tensor) else v)
           for k, v in workloads.decode_token(seed=0).items()}
    r32 = workloads.rmsnorm_rows(rows=512, d=2176, dtype="f32", seed=0)
    r16 = workloads.rmsnorm_rows(rows=512, d=2176, dtype="bf16", seed=0)
    x32, w32, x16, w16 = npb(r32["x"]), npb(r32["w"]), npb(r16["x"]), npb(r16["w"])
    pf = workloads.prefill(n_seqs=8, dtype="bf16", seed=0)
    qkv = [npb(t) for t in workloads.qkv_views(pf["qkv"], pf["hq"], pf["hkv"], pf["dh"])]
    cache, pos, slots = npb(pf["cache"]).copy(), pf["positions"].numpy(), pf["slot_mapping"].numpy()
    sw = workloads.swiglu_fused(rows=8192, inter=8960, dtype="bf16", seed=0)
    gate, up = npb(sw["gate_up"][:, :8960]), npb(sw["gate_up"][:, 8960:])
    eps = float(np.float32(1e-6))
    cases = {
        "decode_token_b1": lambda: (
            oracle.rmsnorm(tok["x"], tok["w"], eps),
            oracle.rope_kvstore(tok["q"], tok["k"], tok["v"], tok["positions"], tok["theta"],
                                tok["cache"], tok["slot_mapping"]),
            oracle.swiglu(tok["gate"], tok["up"])),
        "rmsnorm_512x2176_f32": lambda: oracle.rmsnorm(x32, w32, eps),
        "rmsnorm_512x2176_bf16": lambda: oracle.rmsnorm(x16, w16, eps),
        "prefill_rope_kvstore_8_seqs": lambda: oracle.rope_kvstore(
            *qkv, pos, pf["theta"], cache, slots, block_size=pf["block_size"]),
        "swiglu_8192x8960": lambda: oracle.swiglu(gate, up),
    }
    threads = oracle.num_threads()
    out = {}
    for name, fn in cases.items():
        row = {}
        for n in (threads, 1):
            oracle.set_num_threads(n)
            t0 = time.perf_counter()
            fn()
            row["seconds" if n == threads else "one_thread_seconds"] = round(time.perf_counter() - t0, 4)
        out[name] = row
    oracle.set_num_threads(threads)
    return dict(threads=threads, **out)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pmc_pass():
    """Eager launches only (no graphs), for hardware counter runs: the copy
    kernel on 1 GiB (the byte-counter reference), every op at the decode
    chain's shape over its 28 layers, the batch-256 and batch-1 chains' one
    launch, and
    each kernel at its large shape."""
    import torch
    import kv_cache_rmsnorm_amd as kcr
    import workloads
    from kv_cache_rmsnorm_amd.chain import DecodeChain

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(generator=torch.Generator(device="cuda").manual_seed(0))
    dst = torch.empty_like(src)
    for _ in range(3):
        kcr.copy_(dst, src)
    torch.cuda.synchronize()
    del src, dst
    chain = DecodeChain(workloads.decode_chain(), "cuda", sentinel_cache=False)
    for _ in range(2):
        chain.step_eager()
    torch.cuda.synchronize()
    log(f"pmc pass: copy x3, chain steps x2 ({2 * 4 * len(chain.layers)} launches)")
    for _ in range(3):
        chain.step_one_launch()
    torch.cuda.synchronize()
    log("pmc pass: batch-256 one-launch chain x3")
    del chain
    torch.cuda.empty_cache()
    b1 = DecodeChain(workloads.decode_chain(batch=1), "cuda", sentinel_cache=False)
    for _ in range(3):
        b1.step_b1()
    torch.cuda.synchronize()
    log("pmc pass: batch-1 one-launch chain x3")
    del b1
    large_shapes(kcr, 3)
    torch.cuda.synchronize()
    log("pmc pass done")


COUNTER_PROFILE = os.path.join("profiles", "hbm_bytes_counters.md")

# Sources each measured kernel is built from: a counter figure is used only
# while their hash matches the one recorded with it.
KERNEL_SOURCES = {
    "add_rmsnorm": ("norm_engine.h", "norm.h", "norm_inst.hip", "rmsnorm.hip", "kcr_device.h", "kcr_host.h"),
    "rope_kvstore": ("rope_kvstore.hip", "kcr_device.h", "kcr_host.h"),
    "swiglu": ("swiglu.hip", "kcr_device.h", "kcr_host.h"),
    "one_launch_b256": ("decode_chain.hip", "kcr_device.h", "kcr_host.h"),
    "one_launch_b1": ("decode_chain.hip", "kcr_device.h", "kcr_host.h"),
}


_C_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_only(text: str) -> str:
    """C/C++ source with its comments removed and its whitespace collapsed
    (string and character literals kept), so that an edit to comments or
    layout alone leaves the hash below unchanged."""
    text = _C_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_source_sha(op: str) -> str:
    """Hash of the code (comments and layout ignored) of the files that make
    up an op's kernels and their launch."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[op]:
        h.update(code_only(open(os.path.join(ROOT, "kv_cache_rmsnorm_amd", "csrc", f)).read()).encode())
    return h.hexdigest()


def counter_traffic(op: str):
    """HBM bytes per launch of a decode-chain kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE, WRITE_SIZE), if it was taken on
    the current kernel source; else (None, reason)."""
    path = os.path.join(ROOT, COUNTER_PROFILE)
    if not os.path.exists(path):
        return None, f"no {COUNTER_PROFILE}"
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None, f"no counter block in {COUNTER_PROFILE}"
    entry = json.loads(m.group(1)).get("decode_chain", {}).get(op)
    if not entry:
        return None, f"{op} not in {COUNTER_PROFILE}"
    if entry.get("source_sha256") != kernel_source_sha(op):
        return None, "kernel source changed since the counters were taken"
    return entry.get("traffic_bytes_per_launch"), None


def _dim(r: dict, key: str) -> int:
    """A launch dimension from a rocprofv3 CSV row: one column, or _X/_Y/_Z."""
    if key in r:
        return int(r[key])
    return int(r[key + "_X"]) * int(r[key + "_Y"]) * int(r[key + "_Z"])


def _pmc_dispatches(csv_dir: str, counter: str):
    """[(dispatch id, kernel name, grid, block, value)] of the library's
    kernels (the cos/sin table builds aside) in dispatch order."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {csv_dir}")
    out = []
    for r in csv.DictReader(open(files[0])):
        name = r["Kernel_Name"]
        if r["Counter_Name"] != counter or "kcr::" not in name or "rope_table_kernel" in name:
            continue
        out.append((int(r["Dispatch_Id"]), name, _dim(r, "Grid_Size"), _dim(r, "Workgroup_Size"),
                    float(r["Counter_Value"])))
    out.sort()
    return out


def counter_summary(fetch_dir: str, write_dir: str):
    """Markdown summary of two `rocprofv3 --pmc` runs of `bench.py
    --pmc-pass` (FETCH_SIZE, then WRITE_SIZE): HBM bytes per dispatch,
    scaled by the copy kernel's exactly known 1 GiB in and out; the decode
    chain's kernels (identified by their place in the pass's fixed launch
    order) with the hash of their sources; and every kernel grouped by
    name and grid."""
    import workloads
    from kv_cache_rmsnorm_amd.chain import chain_bytes
    fe, wr = _pmc_dispatches(fetch_dir, "FETCH_SIZE"), _pmc_dispatches(write_dir, "WRITE_SIZE")
    n = 1 << 30
    copies = [i for i, d in enumerate(fe) if "copy_kernel" in d[1]][:3]
    sf = n / (1024 * statistics.fmean(fe[i][4] for i in copies))
    sw = n / (1024 * statistics.fmean(wr[i][4] for i in copies))
    i0 = copies[-1] + 1
    # The fixed part of the pass (copies, chain steps, one-launch chains) must
    # have launched the same kernels in both runs; the large shapes' warm-up
    # is timed, so their counts may differ and they are grouped per run.
    fixed = i0 + 224 + 6
    assert [d[1:4] for d in fe[:fixed]] == [d[1:4] for d in wr[:fixed]], "the passes' fixed launches differ"
    wl = workloads.decode_chain(layers=1)
    B, hid, inter, hq, hkv, dh = 256, wl["hidden"], wl["inter"], wl["hq"], wl["hkv"], wl["dh"]
    per = chain_bytes(28, B, hid, inter, hq, hkv, dh, 2)
    alg = dict(add_rmsnorm=per["per_layer"]["add_rmsnorm"] // 2, rope_kvstore=per["per_layer"]["rope_kvstore"],
               swiglu=per["per_layer"]["swiglu"], one_launch_b256=per["one_launch_step"],
               one_launch_b1=chain_bytes(28, 1, hid, inter, hq, hkv, dh, 2)["one_launch_step"])
    order = ["add_rmsnorm", "rope_kvstore", "add_rmsnorm", "swiglu"]
    groups = {}
    for k in range(2 * 112):   # two eager steps of the 28-layer chain
        groups.setdefault(order[k % 4], []).append(i0 + k)
    groups["one_launch_b256"] = [i0 + 224 + k for k in range(3)]
    groups["one_launch_b1"] = [i0 + 227 + k for k in range(3)]
    chain = {}
    for op, idx in groups.items():
        names = {fe[i][1] for i in idx}
        assert len(names) == 1, f"{op}: mixed kernels {names}"
        f = statistics.fmean(fe[i][4] for i in idx)
        w = statistics.fmean(wr[i][4] for i in idx)
        traffic = int(round(1024 * (f * sf + w * sw)))
        chain[op] = dict(kernel=fe[idx[0]][1].replace("void kcr::", "").split("(")[0], grid=fe[idx[0]][2],
                         block=fe[idx[0]][3], dispatches=len(idx), fetch_kib=round(f, 1), write_kib=round(w, 1),
                         traffic_bytes_per_launch=traffic, algorithmic_bytes_per_launch=alg[op],
                         ratio=round(traffic / alg[op], 4), source_sha256=kernel_source_sha(op))
    table = {}
    for lst, j in ((fe, 0), (wr, 1)):
        for d in lst:
            key = (d[1].replace("void kcr::", "").split("(")[0], d[2], d[3])
            table.setdefault(key, ([], []))[j].append(d[4])
    print("# HBM byte counters per dispatch (FETCH_SIZE, WRITE_SIZE)\n")
    print("Commands (two passes, one counter each, then this summary; from the repository root on the "
          "MI355X machine, `REPO=$(pwd)`):\n")
    print("```")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        print(f"cd /tmp && timeout -s KILL 300 rocprofv3 --pmc {c} --output-format csv -d $REPO/gpurun_out/pmc_{c} "
              f"-o pmc -- python3 -u $REPO/bench.py --pmc-pass")
    print("cd $REPO && python3 bench.py --counter-summary gpurun_out/pmc_FETCH_SIZE gpurun_out/pmc_WRITE_SIZE")
    print("```\n")
    print(f"Scale: the library's copy kernel moves exactly 1 GiB in and 1 GiB out per dispatch; FETCH_SIZE is "
          f"scaled by {sf:.4f} and WRITE_SIZE by {sw:.4f} (KiB per dispatch to bytes).\n")
    print("## Decode chain (28 layers, batch 256, bf16) and its one-launch forms\n")
    print("| op | kernel | grid x block | dispatches | FETCH KiB | WRITE KiB | scaled HBM bytes | algorithmic bytes | ratio |")
    print("|---|---|---|---|---|---|---|---|---|")
    for op, e in chain.items():
        print(f"| {op} | `{e['kernel']}` | {e['grid']} x {e['block']} | {e['dispatches']} | {e['fetch_kib']} | "
              f"{e['write_kib']} | {e['traffic_bytes_per_launch']} | {e['algorithmic_bytes_per_launch']} | {e['ratio']:.3f} |")
    print("\n## Every kernel of the pass, by name and grid (means over its dispatches)\n")
    print("| kernel | grid x block | dispatches (fetch/write pass) | FETCH KiB | WRITE KiB | scaled HBM bytes |")
    print("|---|---|---|---|---|---|")
    for (name, grid, blk), (vf, vw) in sorted(table.items(), key=lambda kv: -statistics.fmean(kv[1][0] or [0])):
        if not vf or not vw:
            continue
        f, w = statistics.fmean(vf), statistics.fmean(vw)
        print(f"| `{name}` | {grid} x {blk} | {len(vf)}/{len(vw)} | {f:.1f} | {w:.1f} | {int(round(1024 * (f * sf + w * sw)))} |")
    print("\nbench.py reads the block below for `roofline.traffic` and the one-launch chain's "
          "`counter_traffic_bytes`, and drops an entry once the hash of its kernel's sources changes.\n")
    print("```json")
    print(json.dumps(dict(scale_fetch=round(sf, 6), scale_write=round(sw, 6), decode_chain=chain), indent=1))
    print("```")


SQ_PASSES = (
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_ANY",
    "SQ_INSTS_VALU SQ_INSTS_VMEM SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F SQ_CYCLES",
)


def sq_summary(cycles_dir: str, insts_dir: str):
    """Markdown summary of two `rocprofv3 --pmc` runs of `bench.py
    --pmc-pass` with the shader-sequencer counters of SQ_PASSES: per kernel
    and grid, the share of wave-cycles in VALU work, waiting and issue
    stalls, and instructions per wave."""
    import csv
    import glob

    def load(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        acc = {}
        for r in csv.DictReader(open(files[0])):
            name = r["Kernel_Name"]
            if "kcr::" not in name or "rope_table_kernel" in name:
                continue
            key = (name.replace("void kcr::", "").split("(")[0], _dim(r, "Grid_Size"), _dim(r, "Workgroup_Size"))
            acc.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return {k: {c: statistics.fmean(v) for c, v in cs.items()} for k, cs in acc.items()}

    cyc, ins = load(cycles_dir), load(insts_dir)
    print("# Shader-sequencer counters per dispatch (where waves spend their cycles)\n")
    print("Commands (two passes, then this summary; from the repository root on the MI355X machine, "
          "`REPO=$(pwd)`):\n")
    print("```")
    for tag, counters in zip(("SQ", "SQI"), SQ_PASSES):
        print(f"cd /tmp && timeout -s KILL 300 rocprofv3 --pmc {counters} --output-format csv "
              f"-d $REPO/gpurun_out/pmc_{tag} -o pmc -- python3 -u $REPO/bench.py --pmc-pass")
    print("cd $REPO && python3 bench.py --sq-summary gpurun_out/pmc_SQ gpurun_out/pmc_SQI")
    print("```\n")
    print("Means over all dispatches of each kernel and grid in the pass (eager launches of the decode chain, "
          "the one-launch chains, the large shapes). Wave-cycle counters are summed over waves. `VALU share` = "
          "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES, `waiting` = SQ_WAIT_ANY / SQ_WAVE_CYCLES (memory, barriers, "
          "dependencies), `issue stall` = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.\n")
    print("| kernel | grid x block | waves | VALU instr per wave | VMEM instr per wave | SALU instr per wave | "
          "LDS instr per wave | VALU share | waiting | issue stall |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for key in sorted(cyc, key=lambda k: -cyc[k].get("SQ_WAVES", 0) * k[1]):
        c, i = cyc[key], ins.get(key, {})
        w, wc = c.get("SQ_WAVES", 0.0), c.get("SQ_WAVE_CYCLES", 0.0)
        if w <= 0 or wc <= 0:
            continue
        per = lambda n: f"{i[n] / w:.1f}" if n in i else "-"
        print(f"| `{key[0]}` | {key[1]} x {key[2]} | {w:.0f} | {per('SQ_INSTS_VALU')} | {per('SQ_INSTS_VMEM')} | "
              f"{per('SQ_INSTS_SALU')} | {per('SQ_INSTS_LDS')} | {100 * c.get('SQ_ACTIVE_INST_VALU', 0) / wc:.1f}% | "
              f"{100 * c.get('SQ_WAIT_ANY', 0) / wc:.1f}% | {100 * c.get('SQ_WAIT_INST_ANY', 0) / wc:.1f}% |")


def trace_summary(trace_dir: str, steps: int):
    """Markdown summary of `rocprofv3 --kernel-trace --stats` over a default
    bench run: every library kernel by name and grid, then the launches
    split into segments at gaps over 200 us, where the timed region is the
    segment of `steps` graph replays of the 112-launch chain."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    ks = []
    for r in csv.DictReader(open(files[0])):
        name = r["Kernel_Name"]
        if "kcr::" not in name or "rope_table_kernel" in name:
            continue
        short = name.replace("void kcr::", "").split("(")[0]
        ks.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short, _dim(r, "Grid_Size"),
                   _dim(r, "Workgroup_Size")))
    ks.sort()

    def stats(v):
        v = sorted(v)
        return len(v), statistics.fmean(v), statistics.median(v), v[0], v[-1]

    groups = {}
    for a, b, n, g, w in ks:
        groups.setdefault((n, g, w), []).append((b - a) / 1e3)
    print("# rocprofv3 kernel trace of the default bench run\n")
    print("Command (from the repository root on the MI355X machine, `REPO=$(pwd)`), then this summary:\n")
    print("```")
    print("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/gpurun_out/prof_bench "
          "-o bench -- python3 -u $REPO/bench.py")
    print(f"cd $REPO && python3 bench.py --trace-summary gpurun_out/prof_bench --steps {steps}")
    print("```\n")
    print("Durations from the trace's own start/end stamps, in us. Under the profiler the dispatches of a "
          "graph replay are spaced further apart than unprofiled.\n")
    print("## Every library kernel, by name and grid\n")
    print("| kernel | grid x block | launches | mean us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (n, g, w), v in sorted(groups.items(), key=lambda kv: -statistics.fmean(kv[1])):
        c, mean, med, lo, hi = stats(v)
        print(f"| `{n}` | {g} x {w} | {c} | {mean:.2f} | {med:.2f} | {lo:.2f} | {hi:.2f} |")
    segs, cur = [], [ks[0]]
    for prev, k in zip(ks, ks[1:]):
        if k[0] - prev[1] > 200_000:
            segs.append(cur)
            cur = []
        cur.append(k)
    segs.append(cur)
    print("\n## Segments of at least 112 launches (split at gaps over 200 us)\n")
    print("| segment | launches | start-to-start us | kernels (n, mean us) |")
    print("|---|---|---|---|")
    timed = None
    for i, sg in enumerate(segs):
        if len(sg) < 112:
            continue
        per = {}
        for a, b, n, g, w in sg:
            per.setdefault(f"{n} {g}x{w}", []).append((b - a) / 1e3)
        gap = (sg[-1][0] - sg[0][0]) / 1e3 / max(1, len(sg) - 1)
        desc = "; ".join(f"`{k}` n={len(v)} {statistics.fmean(v):.2f}" for k, v in per.items())
        print(f"| {i} | {len(sg)} | {gap:.2f} | {desc} |")
        if len(sg) == 112 * steps and timed is None and len(per) == 3:
            timed = per
    # The timed graph replays end right before the launch-floor graph (the
    # 16-byte copy, grid 64): the 112 * steps chain launches before it.
    floor = next((i for i, k in enumerate(ks) if k[2].split("::")[-1] == "copy_kernel" and k[3] == 64), None)
    if floor is not None and floor >= 112 * steps:
        per = {}
        for a, b, n, g, w in ks[floor - 112 * steps:floor]:
            per.setdefault(f"{n} {g}x{w}", []).append((b - a) / 1e3)
        if len(per) == 3:
            timed = per
    if timed:
        print(f"\n## The timed region: {steps} graph replays of the 112-launch chain\n")
        print("| kernel | launches | launches per step | mean us | median us | us per step |")
        print("|---|---|---|---|---|---|")
        for k, v in sorted(timed.items(), key=lambda kv: -sum(kv[1])):
            c, mean, med, lo, hi = stats(v)
            print(f"| `{k}` | {c} | {c / steps:.0f} | {mean:.2f} | {med:.2f} | {mean * c / steps:.1f} |")


def library_source_sha() -> str:
    """sha256 over the library's sources (C ABI header, kernels, binding),
    file by file in name order: identifies the build a line was measured on
    where no git metadata travels with the tree."""
    h = hashlib.sha256()
    for d in ("include", os.path.join("kv_cache_rmsnorm_amd", "csrc"), "kv_cache_rmsnorm_amd"):
        full = os.path.join(ROOT, d)
        for f in sorted(os.listdir(full)):
            p = os.path.join(full, f)
            if os.path.isfile(p) and f.endswith((".h", ".hip", ".py")):
                h.update(f.encode())
                h.update(open(p, "rb").read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--skip-large", action="store_true", help="skip the per-kernel large shapes")
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-sweep", action="store_true", help="skip the [512, D] RMSNorm sweep")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="only launch each kernel eagerly (for rocprofv3 --pmc runs); no JSON line")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM byte-counter summary of two --pmc-pass runs (FETCH_SIZE, WRITE_SIZE)")
    ap.add_argument("--sq-summary", nargs=2, metavar=("SQ_DIR", "SQI_DIR"),
                    help="print the shader-sequencer counter summary of two --pmc-pass runs (SQ_PASSES)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="print the summary of a rocprofv3 --kernel-trace run of the default bench")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps)
        return
    if args.sq_summary:
        sq_summary(*args.sq_summary)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); the ops "
              "shard by rows and tokens with no exchange, so a multi-GPU run is not part of this "
              "benchmark", file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_rmsnorm_amd as kcr
    import workloads
    from kv_cache_rmsnorm_amd.chain import DecodeChain

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    if args.pmc_pass:
        pmc_pass()
        return
    # The small workloads first, while the process holds nothing else: run
    # after the chain (its 30 GB of caches and captured graphs alive), the
    # [512, D] sweep's smallest bf16 launches read 0.3 us slower, and the
    # batch-1 chain's one launch 63 -> 75 us per step.
    sweep = {} if args.skip_sweep else rmsnorm_sweep(kcr, max(10, args.steps // 5))
    token = decode_token_latency(kcr, max(10, args.steps // 2))
    chain_b1 = decode_chain_b1(kcr, max(20, args.steps))
    t0 = time.perf_counter()
    wl = workloads.decode_chain()
    log(f"generated workload in {time.perf_counter() - t0:.1f} s")
    chain = DecodeChain(wl, "cuda", sentinel_cache=False)
    nbytes = chain.bytes_per_step()
    B, inter = chain.h.shape[0], chain.inter
    log(f"step moves {nbytes['step']} algorithmic bytes over {4 * len(chain.layers)} launches")

    # eager warm-up and capture, then per-kernel durations inside whole steps
    chain.step_eager()
    torch.cuda.synchronize()
    chain.capture()
    per_op, sums = instrumented_steps(kcr, chain, max(3, args.steps // 5))
    kernel_sum_us = 1e3 * statistics.median(sums)

    # eager steps (one Python launch per op)
    for _ in range(3):
        chain.step_eager()
    torch.cuda.synchronize()
    e0, e1 = events(2)
    n_eager = max(5, args.steps // 5)
    e0.record()
    for _ in range(n_eager):
        chain.step_eager()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / n_eager

    # graph replay: the timed region
    for _ in range(args.warmup):
        chain.step_graph()
    torch.cuda.synchronize()
    e0, e1 = events(2)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        chain.step_graph()
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    value = nbytes["step"] / (ms * 1e-3) / 1e9
    log(f"graph step {ms * 1e3:.1f} us = {value:.0f} GB/s; eager {eager_ms * 1e3:.1f} us; "
        f"event-stamped kernel sum {kernel_sum_us:.1f} us")

    floor_us = launch_floor(kcr, 4 * len(chain.layers), max(10, args.steps // 2))
    log(f"launch floor: {floor_us:.2f} us per graph node of a 16-byte copy")
    op_graph = graph_op_us(kcr, chain, max(10, args.steps // 2))
    chain.reset_residual()
    log("in-graph per-launch us: " + ", ".join(f"{k} {v:.2f}" for k, v in op_graph.items()))
    chain_one = decode_chain_one_launch(kcr, chain, ms * 1e3, max(20, args.steps))
    chain.reset_residual()
    ceiling = copy_ceiling(kcr, args.kernel_iters)
    kernels = {} if args.skip_large else large_shapes(kcr, args.kernel_iters)

    copy_us = {op: graph_copy_us(kcr, b, len(chain.layers), max(10, args.steps // 2))
               for op, b in chain_op_bytes(chain).items()}
    copy_step_us = copy_equivalent_step_us(kcr, chain, max(20, args.steps))
    log(f"copy-equivalent step (112 plain copies of the ops' sizes): {copy_step_us:.1f} us")
    log("size-matched copies in a graph: " + ", ".join(f"{k} {v:.2f} us" for k, v in copy_us.items()))
    roofline = chain_roofline(chain, op_graph, per_op, len(sums), copy_us)
    log(f"roofline: dominant kernel {roofline['kernel']} ({100 * roofline['share_of_kernel_time']:.0f}% of the "
        f"step's kernel time), {roofline['mean_us']:.2f} us per launch, {roofline['achieved']:.0f} GB/s "
        f"({100 * roofline['frac']:.1f}% of peak)")

    cpu = None
    if not args.skip_cpu:
        cpu = cpu_baseline_run(wl, nbytes["step"], args.cpu_seconds)
        cpu["per_config"] = cpu_configs_run()
        log(f"cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    op_us = {k: round(1e3 * statistics.fmean(v), 3) for k, v in per_op.items()}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the Qwen2.5-1.5B decode workload)",
        "config": {"workload": "decode_chain: 28 layers x [add_rmsnorm, rope_kvstore, add_rmsnorm, swiglu], "
                               "batch 256, ctx 4096 cached, hidden 1536, inter 8960, 12q/2kv heads x128, "
                               "block 16, bf16",
                   "launch": "hipgraph replay of 112 kernels", "global_batch": B},
        "frac_of_peak": round(value / PEAK_GBS, 4),
        "copy_equivalent_step_us": round(copy_step_us, 2),
        "copy_equivalent_note": "a graph of 112 plain copies in the chain's order, each moving the bytes of the "
                                "op at its place (half read, half written): what a step of launches of these "
                                "sizes attains",
        "step_frac_of_copy_equivalent": round(copy_step_us / (ms * 1e3), 4),
        "step_bytes": nbytes["step"],
        "eager_ms_per_step": round(eager_ms, 5),
        "event_stamped_kernel_sum_us_per_step": round(kernel_sum_us, 2),
        "launch_floor_us_per_node": round(floor_us, 3),
        "launch_floor_share_of_step": round(4 * len(chain.layers) * floor_us / (ms * 1e3), 4),
        "op_event_stamped_mean_us": op_us,
        "op_in_graph_us": {k: round(v, 3) for k, v in op_graph.items()},
        "decode_token_b1": token,
        "decode_chain_b1": chain_b1,
        "decode_chain_b256_one_launch": chain_one,
        "timed_wall_s": round(wall_s, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ceiling": ceiling,
        "kernels": kernels,
        "rmsnorm_sweep_512xD": sweep,
        "device": torch.cuda.get_device_name(0),
        "source_sha256": library_source_sha(),
        "cus": kcr.device_cus(),
        "lds_per_block": torch.cuda.get_device_properties(0).shared_memory_per_block,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

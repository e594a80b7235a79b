"""Batched decode-step chain: the per-token ops of one decode step of a
Qwen2.5-1.5B-shaped model, every layer in turn:

    y_attn = add_rmsnorm(h, d_attn, w_attn)     (h <- h + d_attn)
    q_out  = rope_kvstore(q, k, v) ; K_rot, V -> this layer's paged cache
    y_mlp  = add_rmsnorm(h, d_mlp, w_mlp)       (h <- h + d_mlp)
    act    = swiglu(gate_up)

That is 4 launches per layer, 112 for 28 layers (the koas-w.github.io
2026-03-31 post counts 28 layers x 2 norms = 56 norm launches per step,
section 3; the GEMMs and attention that sit between these ops in a real
model are not part of this path, so each op reads its own seeded input).

The step runs eagerly (one launch per op from Python) or replayed from a
captured HIP graph, which removes the per-launch host cost that
m.lsln.cn/news/61269 (section 4) measures at 3-10 us per kernel.
"""
from __future__ import annotations

import torch

import kv_cache_rmsnorm_amd as kcr


class DecodeChain:
    def __init__(self, wl: dict, device="cuda", sentinel_cache: bool = True):
        """``wl`` is a workloads.decode_chain(...) dict (CPU tensors)."""
        dev = torch.device(device)
        self.device = dev
        self.wl = wl
        self.hq, self.hkv, self.dh = wl["hq"], wl["hkv"], wl["dh"]
        self.hidden, self.inter = wl["hidden"], wl["inter"]
        self.eps = wl["eps"]
        self.h0 = wl["h"].to(dev)
        self.h = self.h0.clone()
        self.positions = wl["positions"].to(dev)
        self.slot_mapping = wl["slot_mapping"].to(dev)
        self.cos, self.sin = kcr.rope_cos_sin(wl["max_pos"], self.dh, wl["theta"], device=dev)
        B = self.h.shape[0]
        self.layers = []
        for lw in wl["layers"]:
            qkv = lw["qkv"].to(dev)
            hq, hkv, dh = self.hq, self.hkv, self.dh
            cache = torch.empty(wl["cache_shape"], dtype=wl["dtype"], device=dev)
            if sentinel_cache:
                cache.view(torch.int16 if cache.element_size() == 2 else torch.int32).fill_(-1)
            gate_up = lw["gate_up"].to(dev)
            self.layers.append(dict(
                w_attn=lw["w_attn"].to(dev), w_mlp=lw["w_mlp"].to(dev),
                d_attn=lw["d_attn"].to(dev), d_mlp=lw["d_mlp"].to(dev), qkv=qkv,
                q=qkv[:, : hq * dh].unflatten(1, (hq, dh)),
                k=qkv[:, hq * dh:(hq + hkv) * dh].unflatten(1, (hkv, dh)),
                v=qkv[:, (hq + hkv) * dh:].unflatten(1, (hkv, dh)),
                gate=gate_up[:, : self.inter], up=gate_up[:, self.inter:], gate_up=gate_up,
                cache=cache,
                y_attn=torch.empty((B, self.hidden), dtype=wl["dtype"], device=dev),
                y_mlp=torch.empty((B, self.hidden), dtype=wl["dtype"], device=dev),
                q_out=torch.empty((B, hq, dh), dtype=wl["dtype"], device=dev),
                act=torch.empty((B, self.inter), dtype=wl["dtype"], device=dev)))
        self.graph = None
        self.graph_b1 = None
        self.graph_one = None
        self._b1 = None
        self._one = None

    def reset_residual(self):
        self.h.copy_(self.h0)

    def layer_ops(self, L: dict):
        """The four launches of one layer (on the current stream)."""
        kcr.add_rmsnorm(self.h, L["d_attn"], L["w_attn"], self.eps, out=L["y_attn"])
        kcr.rope_kvstore(L["q"], L["k"], L["v"], self.positions, self.cos, self.sin, L["cache"],
                         self.slot_mapping, q_out=L["q_out"])
        kcr.add_rmsnorm(self.h, L["d_mlp"], L["w_mlp"], self.eps, out=L["y_mlp"])
        kcr.swiglu(L["gate"], L["up"], out=L["act"])

    def step_eager(self):
        for L in self.layers:
            self.layer_ops(L)

    def step_b1(self):
        """Batch 1 only: the whole step's chain in one launch
        (kcr_decode_chain_b1), same ops in the same order."""
        if self._b1 is None:
            self._b1 = kcr.DecodeChainB1(self.layers, self.h, self.positions, self.slot_mapping, self.cos,
                                         self.sin, self.eps, self.hq, self.hkv)
        self._b1()

    def step_one_launch(self):
        """Any batch: the whole step's chain in one launch
        (kcr_decode_chain_batch), same ops with the same results."""
        if self._one is None:
            self._one = kcr.DecodeChainBatch(self.layers, self.h, self.positions, self.slot_mapping, self.cos,
                                             self.sin, self.eps, self.hq, self.hkv)
        self._one()

    def _capture(self, step):
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize(self.device)
        return g

    def capture_b1(self):
        """Capture the batch-1 one-launch step into a HIP graph."""
        self.graph_b1 = self._capture(self.step_b1)
        return self.graph_b1

    def capture_one_launch(self):
        """Capture the one-launch step of any batch into a HIP graph."""
        self.graph_one = self._capture(self.step_one_launch)
        return self.graph_one

    def capture(self):
        """Capture one step into a HIP graph (after one eager warm-up step on
        a side stream, as graph capture requires)."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            self.step_eager()
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step_eager()
        torch.cuda.synchronize(self.device)
        self.graph = g
        return g

    def step_graph(self):
        self.graph.replay()

    # Algorithmic bytes of one step (what the ops must move at least once).
    def bytes_per_step(self) -> dict:
        return chain_bytes(len(self.layers), self.h.shape[0], self.hidden, self.inter, self.hq,
                           self.hkv, self.dh, self.h.element_size(),
                           distinct_positions=int(torch.unique(self.positions).numel()))


def norm_bytes(rows: int, d: int, s: int, add: bool) -> int:
    """RMSNorm reads x and writes y; the add variant also reads delta and
    writes x back; the weight row is read once."""
    return (4 if add else 2) * rows * d * s + d * s


def rope_bytes(T: int, hq: int, hkv: int, dh: int, s: int, distinct_positions: int) -> int:
    """Per token: read q, k, v; write q_out, K_rot and V; plus the position
    and slot (8 B each). cos and sin rows (fp32) once per distinct position."""
    return T * ((2 * hq + 4 * hkv) * dh * s + 16) + distinct_positions * dh * 4


def swiglu_bytes(rows: int, inter: int, s: int) -> int:
    """Read gate and up, write out."""
    return 3 * rows * inter * s


def chain_bytes(layers, B, hidden, inter, hq, hkv, dh, s, distinct_positions=1) -> dict:
    per = dict(add_rmsnorm=2 * norm_bytes(B, hidden, s, True),
               rope_kvstore=rope_bytes(B, hq, hkv, dh, s, distinct_positions),
               swiglu=swiglu_bytes(B, inter, s))
    per_layer = sum(per.values())
    step = layers * per_layer
    # The one-launch chain (kcr_decode_chain_batch) keeps the residual h in
    # registers: it reads h once per token instead of once per add (2 adds
    # per layer), and the positions, slots and cos/sin rows once per step
    # instead of once per layer. Its stores are those of the separate ops.
    one = (step - (2 * layers - 1) * B * hidden * s
           - (layers - 1) * (B * 16 + distinct_positions * dh * 4))
    return dict(per_layer=per, layer=per_layer, step=step, one_launch_step=one)

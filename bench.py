#!/usr/bin/env python3
"""Benchmark of the hybrid GQA attention layer's hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
RoPE on the new keys, the KV-cache append, prefill attention (Q-RoPE fused in its
prologue, sigmoid gate in its epilogue), then the single-token decode (RoPE, append,
split-KV partials and their log-sum-exp combine).

Default workload (the 1M-context full layer, B=1): a cache holding positions
0..1044479, a chunked prefill of 4096 queries at positions 1044480..1048575, then one
decode at position 1048576 over 1048577 keys.  Other workloads (--workload 2..11):
2 the 32K sliding prefill, 3 the 128K full prefill, 4 the B=32 mixed decode at 128K,
6 the sliding-layer side of the 1M chunk (prefill against the 512-slot ring, append,
decode), 7 and 8 the 36-layer decode step and chunk prefill at 1M, 9 and 10 the decode
over the 8-bit KV cache at 1M and at B=32 x 128K, 11 the fused QKV + gate and output
projections on a 4096-token chunk.

Prints one JSON line.  `value` is the prefill attention throughput of the whole step
(algorithmic prefill FLOP / step time); the decode KV bandwidth and per-kernel rates,
measured with HIP events on the library's stream, are reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "prefill attn TFLOP/s (%MFMA peak); decode KV GB/s (%HBM) at 128K/1M"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
HQ, HKV, D, WINDOW = 16, 4, 256, 512
KV_BYTES_PER_TOKEN = 2 * HKV * D * 2   # K and V rows of one token, one layer
FLOP_PER_PAIR = 4 * D                  # QK^T and PV per visible (query, key, head)


def prefill_pairs(sq: int, pos0: int, kind: str) -> int:
    """Visible (query, key) pairs of one head for queries at pos0 .. pos0+sq-1."""
    if kind == "full":
        return sq * pos0 + sq * (sq + 1) // 2
    n_short = max(0, min(sq, WINDOW - pos0))
    return n_short * pos0 + n_short * (n_short + 1) // 2 + (sq - n_short) * WINDOW


class Timer:
    """HIP events around each launch of one stage, on the current stream."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.pairs.append((self.a, self.b))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


class Stages:
    def __init__(self, names):
        self.t = {n: [] for n in names}

    def time(self, name):
        s = Timer()
        self.t[name].append(s)
        return s

    def mean_ms(self, name):
        xs = self.t[name]
        return sum(x.mean_ms() for x in xs) / max(1, len(xs))

    def clear(self):
        for k in self.t:
            self.t[k] = []


# ------------------------------------------------------------------------ workloads --
def _cap(n: int) -> int:
    return synth.round_up(n, 64)


class PrefillWorkload:
    """Workloads 2 and 3: one layer's prefill from position 0; K/V consumed in place."""

    def __init__(self, idx: int, device="cuda"):
        from full_gqa_attention_hattn_amd import hattn
        self.h = hattn
        W = synth.WORKLOADS[idx]
        self.W, self.kind = W, W.params["kind"]
        B, S = W.params["B"], W.params["S"]
        self.B, self.S = B, S
        self.cfg = hattn.preset(self.kind)
        inp = synth.layer_inputs(W.seed, B, S, device)
        self.q, self.k_src, self.v, self.gate = inp["q"], inp["k"], inp["v"], inp["gate"]
        self.k = torch.empty_like(self.k_src)
        self.pos0 = synth.positions(0, B, device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(B, S, HQ, dtype=torch.float32, device=device)
        self.stages = Stages(["rope_k", "prefill"])
        self.prefill_flop = B * HQ * FLOP_PER_PAIR * prefill_pairs(S, 0, self.kind)
        self.decode_bytes = 0

    def step(self):
        h = self.h
        self.k.copy_(self.k_src)
        with self.stages.time("rope_k"):
            h.rope_qk(self.cfg, None, self.k, self.pos0)
        with self.stages.time("prefill"):
            h.prefill(self.cfg, self.q, self.k, self.v, self.pos0, self.gate, self.out, self.lse,
                      rope_q_fused=True)


class MixedDecodeWorkload:
    """Workload 4: B=32 new tokens at position 131072; one full layer reading a 131072-token
    cache and three sliding layers reading full 512-slot rings."""

    def __init__(self, device="cuda"):
        from full_gqa_attention_hattn_amd import hattn
        self.h = hattn
        W = synth.WORKLOADS[4]
        self.W = W
        B, p = W.params["B"], W.params["pos"]
        self.B, self.p = B, p
        self.cap = _cap(p + 1)
        self.layers = []
        for li, kind in enumerate(["full", "sliding", "sliding", "sliding"]):
            cfg = hattn.preset(kind)
            cap = self.cap if kind == "full" else WINDOW
            n_filled = p if kind == "full" else WINDOW
            cache = synth.cache_inputs(W.seed, B, cap, n_filled, device, layer=li)
            new = synth.layer_inputs(W.seed, B, 1, device, layer=li)
            L = dict(kind=kind, cfg=cfg, cap=cap, K=cache["cache_k"], V=cache["cache_v"],
                     q=new["q"], k_src=new["k"], v=new["v"], gate=new["gate"],
                     k=torch.empty_like(new["k"]),
                     out=torch.empty_like(new["q"]),
                     lse=torch.empty(B, 1, HQ, dtype=torch.float32, device=device),
                     ws=hattn.alloc_workspace(cfg, B, cap, device),
                     slots=torch.empty(B, 1, dtype=torch.int32, device=device))
            self.layers.append(L)
        self.pos = synth.positions(p, B, device)
        self.stages = Stages(["rope_k", "append", "decode_full", "decode_sliding"])
        self.prefill_flop = 0
        n_full = min(p + 1, self.cap)
        self.decode_bytes = B * KV_BYTES_PER_TOKEN * (n_full + 3 * min(p + 1, WINDOW))
        self.decode_bytes_full = B * KV_BYTES_PER_TOKEN * n_full

    def step(self):
        h = self.h
        for L in self.layers:
            L["k"].copy_(L["k_src"])
            with self.stages.time("rope_k"):
                h.rope_qk(L["cfg"], None, L["k"], self.pos)
            with self.stages.time("append"):
                h.kv_append(L["cfg"], L["k"], L["v"], L["K"], L["V"], self.pos, L["slots"])
            with self.stages.time("decode_full" if L["kind"] == "full" else "decode_sliding"):
                h.decode(L["cfg"], L["q"], L["K"], L["V"], self.pos, L["gate"], L["out"],
                         L["lse"], L["ws"], rope_q_fused=True)


class Full1MWorkload:
    """Workload 5: 1M-context full layer, B=1 -- chunked prefill then one decode."""

    def __init__(self, device="cuda"):
        from full_gqa_attention_hattn_amd import hattn
        self.h = hattn
        W = synth.WORKLOADS[5]
        self.W = W
        self.L0, self.C, self.pd = W.params["cache_len"], W.params["chunk"], W.params["decode_pos"]
        self.cap = _cap(self.pd + 1)
        self.cfg = hattn.preset("full")
        cache = synth.cache_inputs(W.seed, 1, self.cap, self.L0, device, layer=0)
        self.K, self.V = cache["cache_k"], cache["cache_v"]
        ch = synth.layer_inputs(W.seed, 1, self.C, device, layer=1)
        self.q, self.k_src, self.v, self.gate = ch["q"], ch["k"], ch["v"], ch["gate"]
        self.k = torch.empty_like(self.k_src)
        dc = synth.layer_inputs(W.seed, 1, 1, device, layer=2)
        self.qd, self.kd_src, self.vd, self.gd = dc["q"], dc["k"], dc["v"], dc["gate"]
        self.kd = torch.empty_like(self.kd_src)
        self.pos0 = synth.positions(self.L0, 1, device)
        self.posd = synth.positions(self.pd, 1, device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(1, self.C, HQ, dtype=torch.float32, device=device)
        self.outd = torch.empty_like(self.qd)
        self.lsed = torch.empty(1, 1, HQ, dtype=torch.float32, device=device)
        self.ws = hattn.alloc_workspace(self.cfg, 1, self.cap, device)
        self.slots = torch.empty(1, self.C, dtype=torch.int32, device=device)
        self.slotsd = torch.empty(1, 1, dtype=torch.int32, device=device)
        self.stages = Stages(["rope_k", "append", "prefill", "decode"])
        self.prefill_flop = HQ * FLOP_PER_PAIR * prefill_pairs(self.C, self.L0, "full")
        self.decode_bytes = KV_BYTES_PER_TOKEN * (self.pd + 1)

    def step(self):
        h = self.h
        self.k.copy_(self.k_src)
        with self.stages.time("rope_k"):
            h.rope_qk(self.cfg, None, self.k, self.pos0)
        with self.stages.time("append"):
            h.kv_append(self.cfg, self.k, self.v, self.K, self.V, self.pos0, self.slots)
        with self.stages.time("prefill"):
            h.prefill(self.cfg, self.q, self.K, self.V, self.pos0, self.gate, self.out, self.lse,
                      rope_q_fused=True)
        self.kd.copy_(self.kd_src)
        with self.stages.time("rope_k"):
            h.rope_qk(self.cfg, None, self.kd, self.posd)
        with self.stages.time("append"):
            h.kv_append(self.cfg, self.kd, self.vd, self.K, self.V, self.posd, self.slotsd)
        with self.stages.time("decode"):
            h.decode(self.cfg, self.qd, self.K, self.V, self.posd, self.gd, self.outd, self.lsed,
                     self.ws, rope_q_fused=True)


class SlidingRing1MWorkload:
    """Workload 6: the sliding-layer side of the 1M-context chunk, B=1 -- a chunk prefill
    that continues a full 512-slot ring, the chunk's append into the ring, then one
    ring decode."""

    def __init__(self, device="cuda"):
        from full_gqa_attention_hattn_amd import hattn
        self.h = hattn
        W = synth.WORKLOADS[6]
        self.W = W
        self.P, self.C, self.pd = W.params["ring_pos"], W.params["chunk"], W.params["decode_pos"]
        self.cfg = hattn.preset("sliding")
        ring = synth.cache_inputs(W.seed, 1, WINDOW, WINDOW, device, layer=0)
        self.K0, self.V0 = ring["cache_k"], ring["cache_v"]   # positions P-512 .. P-1
        self.K, self.V = self.K0.clone(), self.V0.clone()
        ch = synth.layer_inputs(W.seed, 1, self.C, device, layer=1)
        self.q, self.k_src, self.v, self.gate = ch["q"], ch["k"], ch["v"], ch["gate"]
        self.k = torch.empty_like(self.k_src)
        dc = synth.layer_inputs(W.seed, 1, 1, device, layer=2)
        self.qd, self.kd_src, self.vd, self.gd = dc["q"], dc["k"], dc["v"], dc["gate"]
        self.kd = torch.empty_like(self.kd_src)
        self.pos0 = synth.positions(self.P, 1, device)
        self.posd = synth.positions(self.pd, 1, device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(1, self.C, HQ, dtype=torch.float32, device=device)
        self.outd = torch.empty_like(self.qd)
        self.lsed = torch.empty(1, 1, HQ, dtype=torch.float32, device=device)
        self.ws = hattn.alloc_workspace(self.cfg, 1, WINDOW, device)
        self.stages = Stages(["rope_k", "append", "prefill", "decode"])
        self.prefill_flop = HQ * FLOP_PER_PAIR * prefill_pairs(self.C, self.P, "sliding")
        self.decode_bytes = KV_BYTES_PER_TOKEN * WINDOW

    def step(self):
        h = self.h
        self.K.copy_(self.K0)          # the ring as the previous chunk left it
        self.V.copy_(self.V0)
        self.k.copy_(self.k_src)
        with self.stages.time("rope_k"):
            h.rope_qk(self.cfg, None, self.k, self.pos0)
        with self.stages.time("prefill"):
            h.prefill_ring(self.cfg, self.q, self.k, self.v, self.K, self.V, self.pos0,
                           self.gate, self.out, self.lse, rope_q_fused=True)
        with self.stages.time("append"):
            h.kv_append(self.cfg, self.k, self.v, self.K, self.V, self.pos0)
        self.kd.copy_(self.kd_src)
        with self.stages.time("rope_k"):
            h.rope_qk(self.cfg, None, self.kd, self.posd)
        with self.stages.time("append"):
            h.kv_append(self.cfg, self.kd, self.vd, self.K, self.V, self.posd)
        with self.stages.time("decode"):
            h.decode(self.cfg, self.qd, self.K, self.V, self.posd, self.gd, self.outd, self.lsed,
                     self.ws, rope_q_fused=True)


class ModelWorkload:
    """Workloads 7 and 8: the whole 36-layer schedule on one GPU at a 1M context, through
    the library's driver (hattn_model_decode / hattn_model_prefill), B=1."""

    def __init__(self, idx: int, device="cuda"):
        from full_gqa_attention_hattn_amd import hattn
        self.h = hattn
        W = synth.WORKLOADS[idx]
        self.W, self.idx = W, idx
        self.n_layers = W.params["n_layers"]
        self.decode = idx == 7
        if self.decode:
            self.P, self.S = W.params["decode_pos"], 1          # history 0..P-1, token at P
        else:
            self.P, self.S = W.params["cache_len"], W.params["chunk"]
        self.cap = _cap(self.P + self.S)
        self.cfg = hattn.preset("full")
        self.layers, self.rings0 = [], []
        for l in range(self.n_layers):
            kind = hattn.model_layer_kind(l)
            rows = self.cap if kind == "full" else WINDOW
            filled = self.P if kind == "full" else WINDOW
            cache = synth.cache_inputs(W.seed, 1, rows, filled, device, layer=l)
            inp = synth.layer_inputs(W.seed, 1, self.S, device, layer=100 + l)
            L = dict(kind=kind, q=inp["q"], k=inp["k"], v=inp["v"], gate=inp["gate"],
                     k_cache=cache["cache_k"], v_cache=cache["cache_v"],
                     out=torch.empty_like(inp["q"]),
                     lse=torch.empty(1, self.S, HQ, dtype=torch.float32, device=device))
            self.layers.append(L)
            if kind == "sliding" and not self.decode:
                self.rings0.append((L, L["k_cache"].clone(), L["v_cache"].clone()))
        self.pos = synth.positions(self.P, 1, device)
        nbytes = (hattn.model_decode_workspace_bytes(self.n_layers, 1, self.cap) if self.decode
                  else hattn.model_prefill_workspace_bytes(self.n_layers, 1, self.S))
        self.ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=device)
        self.kv_per_layer, self.kv_total = hattn.model_kv_bytes(self.n_layers, 1, self.cap)
        n_full = sum(1 for L in self.layers if L["kind"] == "full")
        n_sl = self.n_layers - n_full
        self.stages = Stages(["model_step"])
        if self.decode:
            self.prefill_flop = 0
            self.decode_bytes = KV_BYTES_PER_TOKEN * (n_full * (self.P + 1) + n_sl * WINDOW)
        else:
            self.prefill_flop = HQ * FLOP_PER_PAIR * (
                n_full * prefill_pairs(self.S, self.P, "full")
                + n_sl * prefill_pairs(self.S, self.P, "sliding"))
            self.decode_bytes = 0

    def step(self):
        for L, K0, V0 in self.rings0:      # rings as the previous chunk left them
            L["k_cache"].copy_(K0)
            L["v_cache"].copy_(V0)
        with self.stages.time("model_step"):
            if self.decode:
                self.h.model_decode(self.layers, self.cap, self.pos, self.ws)
            else:
                self.h.model_prefill(self.layers, self.cap, self.pos, self.ws)

    def graph_ms(self, reps: int = 10):
        """The decode step captured once as a HIP graph and replayed (launch overhead of the
        108 kernels gone); mean ms per replay."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.h.model_decode(self.layers, self.cap, self.pos, self.ws)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps


class Kv8DecodeWorkload:
    """Workloads 9 and 10: full-layer decode over the 8-bit KV cache.  The history is drawn
    in bf16 and quantized once by the library's own append (untimed); a step appends the
    new token (rotated and quantized) and decodes it."""

    def __init__(self, idx: int, device="cuda", keep_source: bool = False):
        from full_gqa_attention_hattn_amd import hattn
        self.h = hattn
        W = synth.WORKLOADS[idx]
        self.W = W
        B, P = W.params["B"], W.params["decode_pos"]
        self.B, self.P = B, P
        self.cap = _cap(P + 1)
        self.cfg = hattn.preset("full")
        src = synth.cache_inputs(W.seed, B, self.cap, P, device, layer=0)
        self.K = torch.empty(B, self.cap, HKV, D, dtype=torch.uint8, device=device)
        self.V = torch.empty_like(self.K)
        self.Ks = torch.zeros(B, HKV, self.cap, dtype=torch.float32, device=device)
        self.Vs = torch.zeros_like(self.Ks)
        zero = synth.positions(0, B, device)
        # every row (those past P are zero and quantize to zero codes and scales)
        hattn.kv_append_fp8(self.cfg, src["cache_k"], src["cache_v"], self.K, self.V, self.Ks,
                            self.Vs, zero)
        torch.cuda.synchronize()
        self.source = src if keep_source else None
        del src
        new = synth.layer_inputs(W.seed, B, 1, device, layer=1)
        self.q, self.k, self.v, self.gate = new["q"], new["k"], new["v"], new["gate"]
        self.pos = synth.positions(P, B, device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(B, 1, HQ, dtype=torch.float32, device=device)
        self.ws = hattn.alloc_workspace_fp8(self.cfg, B, self.cap, device)
        self.stages = Stages(["append", "decode"])
        self.prefill_flop = 0
        self.kv8_bytes_per_token = 2 * HKV * D + 2 * HKV * 4
        self.decode_bytes = B * self.kv8_bytes_per_token * (P + 1)

    def step(self):
        h = self.h
        with self.stages.time("append"):
            h.kv_append_fp8(self.cfg, self.k, self.v, self.K, self.V, self.Ks, self.Vs, self.pos,
                            rope_k=True)
        with self.stages.time("decode"):
            h.decode_fp8(self.cfg, self.q, self.K, self.V, self.Ks, self.Vs, self.pos, self.gate,
                         self.out, self.lse, self.ws, rope_q_fused=True)


class ProjWorkload:
    """Workload 11: the fused QKV + gate projection and the output projection of one layer
    on a 4096-token chunk, with seeded synthetic weights."""

    def __init__(self, device="cuda"):
        from full_gqa_attention_hattn_amd import hattn
        import math
        self.h = hattn
        W = synth.WORKLOADS[11]
        self.W = W
        T, Hd = W.params["T"], W.params["hidden"]
        self.T = T

        def w(shape, s):
            return (synth.normal_bf16(shape, s, device).float() / math.sqrt(shape[1])).to(torch.bfloat16)
        self.w_qkv = w((6144, Hd), W.seed * 10 + 1)
        self.w_g = w((16, Hd), W.seed * 10 + 2)
        self.w_o = w((Hd, 4096), W.seed * 10 + 3)
        self.x = synth.normal_bf16((T, Hd), W.seed * 10 + 4, device)
        self.a = synth.normal_bf16((T, HQ, D), W.seed * 10 + 5, device)
        self.q = torch.empty(T, HQ, D, dtype=torch.bfloat16, device=device)
        self.k = torch.empty(T, HKV, D, dtype=torch.bfloat16, device=device)
        self.v = torch.empty_like(self.k)
        self.g = torch.empty(T, HQ, dtype=torch.bfloat16, device=device)
        self.y = torch.empty(T, Hd, dtype=torch.bfloat16, device=device)
        self.stages = Stages(["qkv_proj", "o_proj"])
        self.flop_qkv = 2 * T * Hd * (6144 + 16)
        self.flop_o = 2 * T * 4096 * Hd
        self.prefill_flop = 0
        self.decode_bytes = 0

    def step(self):
        with self.stages.time("qkv_proj"):
            self.h.qkv_proj(self.x, self.w_qkv, self.w_g, self.q, self.k, self.v, self.g)
        with self.stages.time("o_proj"):
            self.h.o_proj(self.a, self.w_o, self.y)


def make_workload(idx: int, device="cuda"):
    if idx in (2, 3):
        return PrefillWorkload(idx, device)
    if idx == 4:
        return MixedDecodeWorkload(device)
    if idx == 5:
        return Full1MWorkload(device)
    if idx == 6:
        return SlidingRing1MWorkload(device)
    if idx in (7, 8):
        return ModelWorkload(idx, device)
    if idx in (9, 10):
        return Kv8DecodeWorkload(idx, device)
    if idx == 11:
        return ProjWorkload(device)
    raise ValueError(f"no bench workload {idx} (1 is the parity-only tiny case)")


# ---------------------------------------------------------------------- cpu baseline --
def _blocks(rows, n=64):
    return [rows[i:i + n] for i in range(0, len(rows), n)]


def cpu_baseline(wl, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload, timed on the
    host's cores.  Reported in the metric's unit (TFLOP/s of attention work; GB/s of KV
    for the decode-only workload)."""
    import oracle as O
    torch.set_num_threads(os.cpu_count() or 1)
    cores = torch.get_num_threads()
    if isinstance(wl, Full1MWorkload):
        # the declared sample: the chunk's last 128 rows and 128 seeded random rows, the
        # oracle run on 64-row blocks (its own row blocking), until the budget is spent
        kc = wl.K[0, :wl.L0].cpu()
        vc = wl.V[0, :wl.L0].cpu()
        _, kr = O.rope_qk(None, wl.k_src[0].cpu(), wl.L0, "full")
        kc = torch.cat([kc.to(torch.float32), kr])
        vc = torch.cat([vc.to(torch.float32), wl.v[0].cpu().to(torch.float32)])
        q, g = wl.q[0].cpu(), wl.gate[0].cpu()
        gen = torch.Generator().manual_seed(1239)
        rand = sorted(torch.randperm(wl.C - 128, generator=gen)[:128].tolist())
        blocks = _blocks(list(range(wl.C - 128, wl.C))) + _blocks(rand)
        t0 = time.perf_counter()
        done = []
        for blk in blocks:
            O.prefill(q, kc, vc, g, wl.L0, "full", rows=torch.tensor(blk))
            done += blk
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        flop = sum(HQ * FLOP_PER_PAIR * (wl.L0 + r + 1) for r in done)
        rate = flop / dt
        return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"declared sample of the 4096-query chunk (last 128 rows, then 128 "
                          f"seeded random rows) over the full {wl.L0 + wl.C}-token cache, all "
                          f"16 heads, oracle on 64-row blocks: {len(done)} rows timed in "
                          f"{dt:.1f} s; the whole chunk extrapolated by visible-pair count "
                          f"would take {wl.prefill_flop / rate:.0f} s"}
    if isinstance(wl, ProjWorkload):
        t0 = time.perf_counter()
        rows, flop = 0, 0
        x, wq, wg = wl.x.cpu(), wl.w_qkv.cpu(), wl.w_g.cpu()
        while time.perf_counter() - t0 < min(budget_s, 10.0) and rows < wl.T:
            O.qkv_proj(x[rows:rows + 64], wq, wg)
            rows += 64
        flop = 2 * rows * 2560 * (6144 + 16)
        dt = time.perf_counter() - t0
        return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"fused QKV + gate projection of {rows} tokens ({dt:.1f} s)"}
    if isinstance(wl, Kv8DecodeWorkload):
        t0 = time.perf_counter()
        nbytes, done = 0, 0
        for b in range(wl.B):
            n = wl.P + 1
            kq, vq = wl.K[b, :n].cpu(), wl.V[b, :n].cpu()
            ks, vs = wl.Ks[b, :, :n].cpu().T, wl.Vs[b, :, :n].cpu().T
            O.decode_kv8(wl.q[b, 0].cpu(), kq, vq, ks, vs, wl.gate[b, 0].cpu(), wl.P, "full")
            nbytes += wl.kv8_bytes_per_token * n
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"8-bit full-layer decode of {done} of {wl.B} sequences, cache copy "
                          f"to host included ({dt:.1f} s)"}
    if isinstance(wl, ModelWorkload):
        # layer 3 (the first full layer) and layer 0 (sliding), the oracle as it stands
        full, sl = wl.layers[3], wl.layers[0]
        t0 = time.perf_counter()
        if wl.decode:
            done, nbytes = [], 0
            for L in (sl, full):
                kind = L["kind"]
                rows = wl.P if kind == "full" else WINDOW
                kc = L["k_cache"][0, :max(rows, WINDOW) if kind == "sliding" else wl.P + 1].cpu().float()
                vc = L["v_cache"][0, :kc.shape[0]].cpu().float()
                _, kn = O.rope_qk(None, L["k"][0].cpu(), wl.P, kind)
                slot = wl.P if kind == "full" else wl.P % WINDOW
                kc[slot] = kn[0]
                vc[slot] = L["v"][0, 0].cpu().float()
                O.decode(L["q"][0, 0].cpu(), kc, vc, L["gate"][0, 0].cpu(), wl.P, kind)
                nbytes += KV_BYTES_PER_TOKEN * ((wl.P + 1) if kind == "full" else WINDOW)
                done.append(kind)
            dt = time.perf_counter() - t0
            return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                    "sample": f"decode of layer 0 (sliding) and layer 3 (full, 2^20+1 keys), "
                              f"cache copy to host included ({dt:.1f} s)"}
        kc = full["k_cache"][0, :wl.P].cpu().float()
        vc = full["v_cache"][0, :wl.P].cpu().float()
        _, kr = O.rope_qk(None, full["k"][0].cpu(), wl.P, "full")
        kc = torch.cat([kc, kr])
        vc = torch.cat([vc, full["v"][0].cpu().float()])
        done, flop = [], 0
        for r in (wl.S - 1, wl.S - 2):
            O.prefill(full["q"][0].cpu(), kc, vc, full["gate"][0].cpu(), wl.P, "full",
                      rows=torch.tensor([r]))
            flop += HQ * FLOP_PER_PAIR * (wl.P + r + 1)
            done.append(r)
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"prefill rows {done} of layer 3 (full) over the 2^20-token cache, "
                          f"all 16 heads ({dt:.1f} s)"}
    if isinstance(wl, SlidingRing1MWorkload):
        rows = list(range(wl.C - 1, wl.C - 257, -1))
        q, g = wl.q[0].cpu(), wl.gate[0].cpu()
        _, kr = O.rope_qk(None, wl.k_src[0].cpu(), wl.P, "sliding")
        v, K0, V0 = wl.v[0].cpu(), wl.K0[0].cpu(), wl.V0[0].cpu()
        t0 = time.perf_counter()
        done = []
        for r in rows:
            O.prefill_ring(q, kr, v, K0, V0, g, wl.P, rows=torch.tensor([r]))
            done.append(r)
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        flop = len(done) * HQ * FLOP_PER_PAIR * WINDOW
        return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"{len(done)} prefill rows of the 4096-query chunk against the "
                          f"ring, all 16 heads ({dt:.1f} s)"}
    if isinstance(wl, PrefillWorkload):
        # sequence 0; full layer: the declared sample (last 1024 rows, 2048 seeded random
        # rows, first 1024 rows); sliding layer: every row in order.  64-row blocks until
        # the budget is spent, extrapolated by visible-pair count.
        b = 0
        S = wl.S
        if wl.kind == "full":
            gen = torch.Generator().manual_seed(1237)
            rand = sorted((torch.randperm(S - 2048, generator=gen)[:2048] + 1024).tolist())
            blocks = (_blocks(list(range(S - 1024, S))) + _blocks(rand)
                      + _blocks(list(range(1024))))
            what = "declared sample (last 1024, 2048 seeded random, first 1024 rows)"
        else:
            blocks = _blocks(list(range(S)))
            what = "every row in order"
        q, g = wl.q[b].cpu(), wl.gate[b].cpu()
        k_cpu, v = wl.k_src[b].cpu(), wl.v[b].cpu()
        _, kr = O.rope_qk(None, k_cpu, 0, wl.kind)
        t0 = time.perf_counter()
        done = []
        for blk in blocks:
            O.prefill(q, kr, v, g, 0, wl.kind, rows=torch.tensor(blk))
            done += blk
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        pairs = sum((r + 1) if wl.kind == "full" else min(r + 1, WINDOW) for r in done)
        rate = HQ * FLOP_PER_PAIR * pairs / dt
        return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"sequence 0, {what}, oracle on 64-row blocks: {len(done)} rows "
                          f"timed in {dt:.1f} s; the whole workload extrapolated by "
                          f"visible-pair count would take {wl.prefill_flop / rate:.0f} s"}
    # mixed decode: full-layer decode of a few sequences
    L = wl.layers[0]
    t0 = time.perf_counter()
    nbytes = 0
    done = 0
    for b in range(wl.B):
        kc = L["K"][b, :wl.p].cpu()
        vc = L["V"][b, :wl.p].cpu()
        _, kn = O.rope_qk(None, L["k_src"][b].cpu(), wl.p, "full")
        kc = torch.cat([kc.to(torch.float32), kn])
        vc = torch.cat([vc.to(torch.float32), L["v"][b].cpu().to(torch.float32)])
        O.decode(L["q"][b, 0].cpu(), kc, vc, L["gate"][b, 0].cpu(), wl.p, "full")
        nbytes += KV_BYTES_PER_TOKEN * (wl.p + 1)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"full-layer decode of {done} of {wl.B} sequences ({dt:.1f} s)"}


# --------------------------------------------------------------------------- traffic --
def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel_src: str, workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary (profiles/traffic_<workload>.txt, "key: value" lines), or None when that
    file is missing or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    src = os.path.join(ROOT, "full_gqa_attention_hattn_amd", "csrc", kernel_src)
    if rec.get("source_sha256") != _sha(src):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib: int):
    """One plain device-to-device copy of `mib` MiB (outside the timed region), so a
    counter pass over this run also records FETCH_SIZE / WRITE_SIZE for a copy of known
    size, which calibrates those counters to bytes."""
    if mib <= 0:
        return
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def model_fields(rec, wl, ms, stage_ms):
    """JSON fields of the whole-model workloads: the driver's step is timed as one unit
    (HIP events around the one library call), so the roofline line is the step's own
    rate over all its kernels, a lower bound for the dominant kernel."""
    step_ms = stage_ms["model_step"]
    rec["kv_cache_bytes"] = {"total": wl.kv_total,
                             "full_layer": max(wl.kv_per_layer),
                             "sliding_layer": min(wl.kv_per_layer),
                             "n_full": sum(1 for L in wl.layers if L["kind"] == "full"),
                             "n_sliding": sum(1 for L in wl.layers if L["kind"] == "sliding")}
    if wl.decode:
        rec["value"] = wl.decode_bytes / (ms * 1e-3) / 1e9
        rec["unit"] = "GB/s"
        ach = wl.decode_bytes / (step_ms * 1e-3) / 1e9
        g_ms = wl.graph_ms()
        rec["graph_ms_per_step"] = g_ms
        rec["graph_GBps"] = wl.decode_bytes / (g_ms * 1e-3) / 1e9
        rec["decode_steps_per_s"] = 1e3 / g_ms
        rec["roofline"] = {"bound": "hbm", "kernel": "hattn_model_decode step (all kernels)",
                           "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                           "frac": ach / PEAK_HBM_GBPS, "traffic": None}
    else:
        rec["value"] = wl.prefill_flop / (ms * 1e-3) / 1e12
        rec["unit"] = "TFLOP/s"
        ach = wl.prefill_flop / (step_ms * 1e-3) / 1e12
        rec["roofline"] = {"bound": "mfma", "kernel": "hattn_model_prefill step (all kernels)",
                           "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / PEAK_BF16_TFLOPS, "traffic": None}


# ------------------------------------------------------------------------------ main --
def measure(idx: int, steps: int, warmup: int, cpu_budget: float, calib_mib: int = 0):
    """Build workload idx, run `warmup` untimed steps, then time exactly `steps` steps
    between two device synchronisations; returns the workload's JSON record."""
    copy_calibration(calib_mib)
    wl = make_workload(idx)
    torch.cuda.synchronize()
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    wl.stages.clear()
    t0 = time.perf_counter()
    for _ in range(steps):
        wl.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps

    st = wl.stages
    rec = {"metric": METRIC, "n_gpus": 1, "steps": steps, "warmup": warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16; no weights needed)"}
    stage_ms = {k: st.mean_ms(k) for k in st.t if st.t[k]}
    rec["stage_ms"] = stage_ms
    if isinstance(wl, ProjWorkload):
        fq, fo = wl.flop_qkv, wl.flop_o
        rec["value"] = (fq + fo) / (ms * 1e-3) / 1e12
        rec["unit"] = "TFLOP/s"
        tq = fq / (stage_ms["qkv_proj"] * 1e-3) / 1e12
        to = fo / (stage_ms["o_proj"] * 1e-3) / 1e12
        rec["qkv_proj_TFLOPs"] = tq
        rec["o_proj_TFLOPs"] = to
        rec["roofline"] = {"bound": "mfma", "kernel": "proj_kernel (fused QKV + gate)",
                           "achieved": tq, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": tq / PEAK_BF16_TFLOPS,
                           "traffic": measured_traffic("proj.hip", "proj_qkv_t4096")}
    elif isinstance(wl, ModelWorkload):
        model_fields(rec, wl, ms, stage_ms)
    elif wl.prefill_flop:
        pf_ms = stage_ms["prefill"]
        rec["value"] = wl.prefill_flop / (ms * 1e-3) / 1e12
        rec["unit"] = "TFLOP/s"
        achieved = wl.prefill_flop / (pf_ms * 1e-3) / 1e12
        rec["prefill_TFLOPs_kernel"] = achieved
        rec["prefill_frac_mfma_peak"] = achieved / PEAK_BF16_TFLOPS
        tr_name = {5: "prefill_full_1m_chunk4096", 3: "prefill_full_b1_s131072",
                   2: "prefill_sliding_b4_s32768",
                   6: "prefill_sliding_ring_1m_chunk4096"}[idx]
        rec["roofline"] = {"bound": "mfma", "kernel": "prefill_kernel", "achieved": achieved,
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": achieved / PEAK_BF16_TFLOPS,
                           "traffic": measured_traffic("prefill.hip", tr_name)}
    if isinstance(wl, Kv8DecodeWorkload):
        dec_ms = stage_ms["decode"]
        gbps = wl.decode_bytes / (dec_ms * 1e-3) / 1e9
        rec["value"] = wl.decode_bytes / (ms * 1e-3) / 1e9
        rec["unit"] = "GB/s"
        rec["decode_GBps"] = gbps
        rec["decode_frac_hbm_peak"] = gbps / PEAK_HBM_GBPS
        rec["keys_per_s"] = wl.B * (wl.P + 1) / (dec_ms * 1e-3)
        rec["kv_bytes_per_token_layer"] = wl.kv8_bytes_per_token
        name = {9: "decode_fp8_full_1m", 10: "decode_fp8_full_b32_p131072"}[idx]
        rec["roofline"] = {"bound": "hbm", "kernel": "decode_split_fp8_kernel+combine",
                           "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                           "frac": gbps / PEAK_HBM_GBPS,
                           "traffic": measured_traffic("decode.hip", name)}
    elif wl.decode_bytes and not isinstance(wl, ModelWorkload):
        dec_ms = sum(stage_ms.get(k, 0.0) for k in ("decode", "decode_full", "decode_sliding"))
        if isinstance(wl, MixedDecodeWorkload):
            dec_ms = stage_ms["decode_full"] + 3 * stage_ms["decode_sliding"]
        gbps = wl.decode_bytes / (dec_ms * 1e-3) / 1e9
        rec["decode_GBps"] = gbps
        rec["decode_frac_hbm_peak"] = gbps / PEAK_HBM_GBPS
        if not wl.prefill_flop:
            rec["value"] = wl.decode_bytes / (ms * 1e-3) / 1e9
            rec["unit"] = "GB/s"
            full_ms = stage_ms["decode_full"]
            ach = wl.decode_bytes_full / (full_ms * 1e-3) / 1e9
            rec["roofline"] = {"bound": "hbm", "kernel": "decode_split_kernel+combine",
                               "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                               "frac": ach / PEAK_HBM_GBPS,
                               "traffic": measured_traffic("decode.hip", "decode_full_b32_p131072")}
    W = wl.W
    rec["config"] = {"workload": W.name, "desc": W.desc, **W.params}
    rec["cpu_baseline"] = cpu_baseline(wl, cpu_budget) if cpu_budget > 0 else None
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


# The metric names the 128K and 1M contexts: besides the headline 1M workload, the default
# run times the 32K sliding prefill, the 128K full prefill and the B=32 decode at 128K.
DEFAULT_EXTRA = (2, 3, 4)
_CONFIG_KEYS = ("ms_per_step", "value", "unit", "stage_ms", "roofline", "decode_GBps",
                "decode_frac_hbm_peak", "prefill_TFLOPs_kernel", "prefill_frac_mfma_peak",
                "config", "cpu_baseline")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5, choices=list(range(2, 12)))
    ap.add_argument("--extra", type=str, default=None,
                    help="comma-separated workloads also timed and reported under 'configs' "
                         "(default 2,3,4 with workload 5, none otherwise; 'none' for none)")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work for the cpu_baseline leg (0 skips it)")
    ap.add_argument("--extra-cpu-budget", type=float, default=4.0,
                    help="seconds of oracle work for each extra workload's cpu_baseline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the workload "
                         "(for calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU (no collectives or "
                                   "sharding are built); run with --gpus 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    if args.extra is None:
        extra = DEFAULT_EXTRA if args.workload == 5 else ()
    elif args.extra.strip().lower() in ("", "none"):
        extra = ()
    else:
        extra = tuple(int(x) for x in args.extra.split(","))

    rec = measure(args.workload, args.steps, args.warmup, args.cpu_budget,
                  args.copy_calibration_mib)
    if extra:
        rec["configs"] = []
        for idx in extra:
            r = measure(idx, args.steps, args.warmup, args.extra_cpu_budget)
            rec["configs"].append({k: r[k] for k in _CONFIG_KEYS if k in r})
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

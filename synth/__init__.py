"""Seeded synthetic inputs for the hybrid GQA attention layer's workloads.

Shared by the oracle-side tests and by the GPU tests and bench.  This module holds none
of the layer's arithmetic (no RoPE, masking, softmax or gating): only seeded normal
draws, position arrays, workload shapes and the placement of given values at given
indices.

Value distribution: i.i.d. N(0, 1) drawn in fp32 by torch's generator and rounded to
bf16, one independent generator per tensor (seed = 1000 * workload seed + stream).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

N_Q_HEADS = 16
N_KV_HEADS = 4
HEAD_DIM = 256

# Stream ids: one generator per tensor so tensors do not depend on each other's sizes.
STREAMS = {"q": 0, "k": 1, "v": 2, "gate": 3, "cache_k": 4, "cache_v": 5}


def normal_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    """N(0,1) bf16 tensor from a dedicated generator seeded with `seed`.
    Large tensors are drawn in slices along dim 0 so the fp32 draw stays small."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    if len(shape) == 0 or shape[0] == 0:
        return out
    per = max(1, (1 << 27) // max(1, out[0].numel()))  # <= 512 MiB fp32 per slice
    for s0 in range(0, shape[0], per):
        s1 = min(shape[0], s0 + per)
        out[s0:s1] = torch.randn((s1 - s0,) + shape[1:], generator=g, dtype=torch.float32,
                                 device=dev).to(torch.bfloat16)
    return out


def stream_seed(seed: int, name: str, layer: int = 0) -> int:
    return 1000 * int(seed) + 100 * int(layer) + STREAMS[name]


def layer_inputs(seed: int, B: int, S: int, device="cpu", layer: int = 0):
    """q [B,S,16,256], k/v [B,S,4,256], gate logits [B,S,16], all bf16 N(0,1)."""
    return {
        "q": normal_bf16((B, S, N_Q_HEADS, HEAD_DIM), stream_seed(seed, "q", layer), device),
        "k": normal_bf16((B, S, N_KV_HEADS, HEAD_DIM), stream_seed(seed, "k", layer), device),
        "v": normal_bf16((B, S, N_KV_HEADS, HEAD_DIM), stream_seed(seed, "v", layer), device),
        "gate": normal_bf16((B, S, N_Q_HEADS), stream_seed(seed, "gate", layer), device),
    }


def cache_inputs(seed: int, B: int, cap: int, n_filled: int, device="cpu", layer: int = 0):
    """KV cache pair [B, cap, 4, 256] bf16: rows < n_filled are N(0,1), the rest zero."""
    out = {}
    for name in ("cache_k", "cache_v"):
        t = torch.zeros((B, cap, N_KV_HEADS, HEAD_DIM), dtype=torch.bfloat16, device=device)
        for b in range(B):
            t[b, :n_filled] = normal_bf16((n_filled, N_KV_HEADS, HEAD_DIM),
                                          stream_seed(seed, name, layer) + 7919 * b, device)
        out[name] = t
    return out


def positions(pos0, B: int, device="cpu") -> torch.Tensor:
    """int32 [B] first position of each sequence (a scalar is broadcast)."""
    if isinstance(pos0, int):
        pos0 = [pos0] * B
    return torch.tensor(list(pos0), dtype=torch.int32, device=device)


def place(t: torch.Tensor, index, dims, values) -> None:
    """t[index][dims] = values, in place (index: a tuple addressing one row)."""
    row = t[index]
    row[..., list(dims)] = torch.as_tensor(values, dtype=t.dtype, device=t.device)


def plant_needle(q, k, b: int, i: int, j: int, dims, amp: float, zero_q: bool = True):
    """Make every query head of row (b, i) and every KV head of key (b, j) carry `amp`
    on `dims`; the query row's other dims are zeroed when zero_q.  The caller picks dims
    on which the layer's position encoding turns little, so the pair's logit is large."""
    if zero_q:
        q[b, i] = 0
    for h in range(q.shape[2]):
        place(q, (b, i, h), dims, [amp] * len(dims))
    for h in range(k.shape[2]):
        place(k, (b, j, h), dims, [amp] * len(dims))


# --- The five workloads ---------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    desc: str
    seed: int
    params: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload(1, "tiny_b1_s1024",
                "B=1, S=1024, one sliding and one full layer, positions 0..1023",
                1235, dict(B=1, S=1024, pos0=0)),
    2: Workload(2, "sliding_prefill_b4_s32768",
                "sliding layer prefill, B=4, S=32768, window 512, theta 1e4 on 256 dims",
                1236, dict(B=4, S=32768, pos0=0, kind="sliding")),
    3: Workload(3, "full_prefill_b1_s131072",
                "full-causal layer prefill, B=1, S=131072, theta 5e6 on dims 0..63",
                1237, dict(B=1, S=131072, pos0=0, kind="full")),
    4: Workload(4, "mixed_decode_b32_p131072",
                "decode step, B=32, new token at 131072: one full layer over a "
                "131072-token cache plus three sliding layers over 512-slot rings",
                1238, dict(B=32, pos=131072, n_sliding=3, window=512)),
    5: Workload(5, "full_1m_chunk4096_decode",
                "1M-context full layer, B=1: cache of positions 0..1044479, chunked "
                "prefill of 4096 queries at 1044480..1048575, then one decode at 1048576",
                1239, dict(B=1, cache_len=1044480, chunk=4096, decode_pos=1 << 20)),
    6: Workload(6, "sliding_ring_1m_chunk4096_decode",
                "1M-context sliding layer, B=1: 512-slot ring holding positions "
                "1043968..1044479, chunk prefill of 4096 queries at 1044480..1048575 "
                "against the ring, the chunk appended, then one ring decode at 1048576",
                1240, dict(B=1, ring_pos=1044480, chunk=4096, decode_pos=1 << 20,
                           window=512)),
    7: Workload(7, "model_36l_1m_decode",
                "36-layer hybrid schedule (9 full + 27 sliding), B=1: one decode step at "
                "position 1048576; full caches hold positions 0..1048575, rings the last 512",
                1241, dict(B=1, n_layers=36, decode_pos=1 << 20)),
    8: Workload(8, "model_36l_1m_chunk4096",
                "36-layer hybrid schedule (9 full + 27 sliding), B=1: one prefill chunk of "
                "4096 queries at 1044480..1048575; full caches hold positions 0..1044479, "
                "rings 1043968..1044479",
                1242, dict(B=1, n_layers=36, cache_len=1044480, chunk=4096)),
    9: Workload(9, "full_1m_decode_kv8",
                "1M-context full layer, B=1, 8-bit KV cache (E4M3 codes, per token-head "
                "scales) holding positions 0..1048575; one decode at 1048576",
                1243, dict(B=1, decode_pos=1 << 20, kv_format="e4m3+fp32 scale")),
    10: Workload(10, "full_decode_b32_p131072_kv8",
                 "full layer, B=32, 8-bit KV cache holding positions 0..131071 per sequence; "
                 "one decode at 131072",
                 1244, dict(B=32, decode_pos=131072, kv_format="e4m3+fp32 scale")),
    11: Workload(11, "projections_t4096",
                 "the layer's projections on the 1M context's 4096-token chunk: fused "
                 "QKV + gate (2560 -> 6144 + 16) and output (4096 -> 2560), seeded "
                 "synthetic weights N(0, 1/fan_in)",
                 1245, dict(T=4096, hidden=2560, qkv_out=6144, gate_out=16, o_in=4096)),
}


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m

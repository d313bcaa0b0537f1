"""GPU parity of the sliding-layer chunk prefill that continues a 512-slot ring
(hattn_prefill_ring), and of the guarantee that no kernel reads cache rows or ring slots
that no token has reached yet (those hold NaN here).  Expected values come only from
`oracle`; inputs from `synth`."""
import pytest
import torch

import oracle as O
import synth
from parity import check_outputs, say

pytestmark = pytest.mark.gpu

NAN = float("nan")


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from full_gqa_attention_hattn_amd import hattn
    return hattn


def _cpu(t):
    return t.detach().cpu()


def _ring_state(seed, B, pos0):
    """Rings as they stand after positions 0 .. pos0[b] - 1 were appended: slots no
    position has reached are NaN (they must never be read)."""
    ring = synth.cache_inputs(seed, B, 512, 512, "cuda")
    K, V = ring["cache_k"].clone(), ring["cache_v"].clone()
    for b, p in enumerate(pos0):
        if p < 512:
            K[b, p:] = NAN
            V[b, p:] = NAN
    return K, V


@pytest.mark.parametrize("fused", [True, False])
def test_prefill_ring_matches_oracle(h, fused):
    """Ragged chunk (300 rows) at chunk starts inside the first window, exactly at a
    wrap, past a wrap, unaligned to the 32-key tile, at 128K, and far past the model's
    context up to the last chunk the interface accepts (pos0 + Sq = 2^31 - 1)."""
    say(f"prefill_ring fused={fused}")
    pos0 = [0, 37, 511, 512, 1000, 131072 - 45, (1 << 30) + 7, (1 << 31) - 1 - 300]
    B, Sq = len(pos0), 300
    cfg = h.preset("sliding")
    inp = synth.layer_inputs(101, B, Sq, "cuda")
    K_ring, V_ring = _ring_state(102, B, pos0)
    pos = synth.positions(pos0, B, "cuda")
    k_new = inp["k"].clone()
    h.rope_qk(cfg, None, k_new, pos)
    q = inp["q"].clone()
    if not fused:
        h.rope_qk(cfg, q, None, pos)
    out = torch.empty_like(q)
    lse = torch.empty(B, Sq, 16, dtype=torch.float32, device="cuda")
    h.prefill_ring(cfg, q, k_new, inp["v"], K_ring, V_ring, pos, inp["gate"], out, lse,
                   rope_q_fused=fused)
    torch.cuda.synchronize()
    for b, p in enumerate(pos0):
        _, kr = O.rope_qk(None, _cpu(inp["k"][b]), p, "sliding")
        y, l = O.prefill_ring(_cpu(inp["q"][b]), kr, _cpu(inp["v"][b]), _cpu(K_ring[b]),
                              _cpu(V_ring[b]), _cpu(inp["gate"][b]), p)
        check_outputs(out[b], lse[b], y, l, f"ring pos0={p} fused={fused}")


@pytest.mark.parametrize("Sq", [1, 31, 33, 600])
def test_prefill_ring_chunk_sizes(h, Sq):
    """One-row chunks, chunks inside one tile, and a chunk longer than the window."""
    say(f"prefill_ring Sq={Sq}")
    pos0 = [70, 5000 + 17]
    B = len(pos0)
    cfg = h.preset("sliding")
    inp = synth.layer_inputs(111 + Sq, B, Sq, "cuda")
    K_ring, V_ring = _ring_state(112 + Sq, B, pos0)
    pos = synth.positions(pos0, B, "cuda")
    k_new = inp["k"].clone()
    h.rope_qk(cfg, None, k_new, pos)
    out = torch.empty_like(inp["q"])
    lse = torch.empty(B, Sq, 16, dtype=torch.float32, device="cuda")
    h.prefill_ring(cfg, inp["q"], k_new, inp["v"], K_ring, V_ring, pos, inp["gate"], out, lse)
    torch.cuda.synchronize()
    for b, p in enumerate(pos0):
        _, kr = O.rope_qk(None, _cpu(inp["k"][b]), p, "sliding")
        y, l = O.prefill_ring(_cpu(inp["q"][b]), kr, _cpu(inp["v"][b]), _cpu(K_ring[b]),
                              _cpu(V_ring[b]), _cpu(inp["gate"][b]), p)
        check_outputs(out[b], lse[b], y, l, f"ring Sq={Sq} pos0={p}")


def test_prefill_ring_chain_equals_one_shot(h):
    """A sequence prefilled chunk by chunk (rope K, prefill against the ring, then append
    the chunk to the ring) matches the oracle's one-shot prefill of the whole sequence."""
    say("prefill_ring chain")
    S, cuts = 1337, [0, 100, 700, 733, 1337]
    cfg = h.preset("sliding")
    inp = synth.layer_inputs(121, 1, S, "cuda")
    K_ring = torch.full((1, 512, 4, 256), NAN, dtype=torch.bfloat16, device="cuda")
    V_ring = torch.full_like(K_ring, NAN)
    out = torch.empty_like(inp["q"])
    lse = torch.empty(1, S, 16, dtype=torch.float32, device="cuda")
    for a, b in zip(cuts[:-1], cuts[1:]):
        pos = synth.positions(a, 1, "cuda")
        k = inp["k"][:, a:b].clone()      # RoPE runs in place; keep the source keys intact
        h.rope_qk(cfg, None, k, pos)
        o = torch.empty_like(inp["q"][:, a:b])
        l = torch.empty(1, b - a, 16, dtype=torch.float32, device="cuda")
        h.prefill_ring(cfg, inp["q"][:, a:b].contiguous(), k, inp["v"][:, a:b].contiguous(),
                       K_ring, V_ring, pos, inp["gate"][:, a:b].contiguous(), o, l)
        h.kv_append(cfg, k, inp["v"][:, a:b].contiguous(), K_ring, V_ring, pos)
        out[:, a:b] = o
        lse[:, a:b] = l
    torch.cuda.synchronize()
    _, kr = O.rope_qk(None, _cpu(inp["k"][0]), 0, "sliding")
    y, l = O.prefill(_cpu(inp["q"][0]), kr, _cpu(inp["v"][0]), _cpu(inp["gate"][0]), 0, "sliding")
    check_outputs(out[0], lse[0], y, l, "ring chain vs one-shot")


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_unwritten_cache_rows_are_never_read(h, kind):
    """Position-indexed caches hold NaN past the last query's position (rows not written
    yet); prefill and decode outputs stay finite and match the oracle."""
    say(f"unwritten rows {kind}")
    cfg = h.preset(kind)
    B, Sq, cap = 2, 100, 260
    pos0 = [0, 141]                          # last rows at 99 and 240; tiles reach 127, 255
    inp = synth.layer_inputs(131, B, Sq, "cuda")
    cache = synth.cache_inputs(132, B, cap, cap, "cuda")
    K, V = cache["cache_k"].clone(), cache["cache_v"].clone()
    for b, p in enumerate(pos0):
        K[b, p + Sq:] = NAN
        V[b, p + Sq:] = NAN
    out = torch.empty_like(inp["q"])
    lse = torch.empty(B, Sq, 16, dtype=torch.float32, device="cuda")
    h.prefill(cfg, inp["q"], K, V, synth.positions(pos0, B, "cuda"), inp["gate"], out, lse)
    # decode of the last chunk token, reading the same caches
    last = [p + Sq - 1 for p in pos0]
    qd = inp["q"][:, Sq - 1:Sq].contiguous()
    gd = inp["gate"][:, Sq - 1:Sq].contiguous()
    od = torch.empty_like(qd)
    ld = torch.empty(B, 1, 16, dtype=torch.float32, device="cuda")
    if kind == "full":
        ws = h.alloc_workspace(cfg, B, cap)
        h.decode(cfg, qd, K, V, synth.positions(last, B, "cuda"), gd, od, ld, ws, rope_q_fused=True)
    torch.cuda.synchronize()
    for b, p in enumerate(pos0):
        y, l = O.prefill(_cpu(inp["q"][b]), _cpu(K[b]), _cpu(V[b]), _cpu(inp["gate"][b]), p, kind,
                         q_rotated=False)
        check_outputs(out[b], lse[b], y, l, f"unwritten rows {kind} pos0={p}")
        if kind == "full":
            check_outputs(od[b, 0], ld[b, 0], y[Sq - 1], l[Sq - 1], f"decode unwritten rows p={last[b]}")

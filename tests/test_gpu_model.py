"""GPU parity of the rotating KV append and of the whole-model driver (the l % 4 == 3 layer
schedule) against the oracle, plus replay of a captured decode step.  Inputs from `synth`,
expected values only from `oracle`."""
import pytest
import torch

import oracle as O
import synth
from parity import assert_bf16_close, assert_rotated, check_outputs, say

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


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_append_rope_equals_rope_then_append(h, kind):
    """Rotating on the way into the cache gives the bits of rope_qk followed by kv_append,
    and rotated dims within one bf16 rounding of the oracle; the source keys stay as given."""
    say(f"append_rope {kind}")
    cfg = h.preset(kind)
    B, n = 3, 70
    cap = 512 if kind == "sliding" else 4096
    pos0 = [0, 1000, (1 << 20) - n + 1] if kind == "sliding" else [0, 1000, cap - n]
    new = synth.layer_inputs(141, B, n, "cuda")
    pos = synth.positions(pos0, B, "cuda")
    k_src = new["k"].clone()
    K1 = torch.zeros(B, cap, 4, 256, dtype=torch.bfloat16, device="cuda")
    V1, K2, V2 = torch.zeros_like(K1), torch.zeros_like(K1), torch.zeros_like(K1)
    s1 = torch.empty(B, n, dtype=torch.int32, device="cuda")
    s2 = torch.empty_like(s1)
    h.kv_append_rope(cfg, new["k"], new["v"], K1, V1, pos, s1)
    kr = new["k"].clone()
    h.rope_qk(cfg, None, kr, pos)
    h.kv_append(cfg, kr, new["v"], K2, V2, pos, s2)
    torch.cuda.synchronize()
    assert torch.equal(new["k"], k_src)
    assert torch.equal(s1, s2) and torch.equal(K1, K2) and torch.equal(V1, V2)
    r = O.KINDS[kind].rot_dim
    for b in range(B):
        _, ref = O.rope_qk(None, _cpu(k_src[b]), pos0[b], kind)
        slots = _cpu(s1[b]).long()
        keep = slots >= 0
        got = _cpu(K1[b])[slots[keep]]
        want = ref[keep]
        err = (got[..., :r].double() - want[..., :r].double()).abs()
        assert float((err - 2 ** -8 * want[..., :r].double().abs() - 1e-5).max()) <= 0
        assert torch.equal(got[..., r:], _cpu(k_src[b])[keep][..., r:])


def _model_layers(h, n_layers, B, S, cap, seed, device="cuda"):
    """Per-layer inputs and caches; full caches and rings start as NaN (never read before
    written) unless filled by the caller."""
    layers = []
    for l in range(n_layers):
        kind = h.model_layer_kind(l)
        inp = synth.layer_inputs(seed, B, S, device, layer=l)
        rows = cap if kind == "full" else 512
        layers.append(dict(kind=kind, q=inp["q"], k=inp["k"], v=inp["v"], gate=inp["gate"],
                           k_cache=torch.full((B, rows, 4, 256), NAN, dtype=torch.bfloat16, device=device),
                           v_cache=torch.full((B, rows, 4, 256), NAN, dtype=torch.bfloat16, device=device),
                           out=torch.empty_like(inp["q"]),
                           lse=torch.empty(B, S, 16, dtype=torch.float32, device=device)))
    return layers


def test_model_prefill_chunks_then_decode(h):
    """Two prefill chunks and one decode step through an 8-layer schedule (layers 3 and 7
    full) match the oracle's one-shot prefill and decode of every layer."""
    say("model prefill x2 + decode")
    n_layers, B, cap = 8, 2, 1024
    cuts = [0, 300, 813]
    S = cuts[-1]
    src = _model_layers(h, n_layers, B, S + 1, cap, 151)       # S prefill tokens + 1 decode
    ws = torch.empty(max(h.model_prefill_workspace_bytes(n_layers, B, 513),
                         h.model_decode_workspace_bytes(n_layers, B, cap)),
                     dtype=torch.uint8, device="cuda")
    outs = [torch.empty(B, S + 1, 16, 256, dtype=torch.bfloat16, device="cuda") for _ in src]
    lses = [torch.empty(B, S + 1, 16, dtype=torch.float32, device="cuda") for _ in src]
    for a, b in zip(cuts[:-1], cuts[1:]):
        chunk = [dict(q=L["q"][:, a:b].contiguous(), k=L["k"][:, a:b].contiguous(),
                      v=L["v"][:, a:b].contiguous(), gate=L["gate"][:, a:b].contiguous(),
                      k_cache=L["k_cache"], v_cache=L["v_cache"],
                      out=torch.empty(B, b - a, 16, 256, dtype=torch.bfloat16, device="cuda"),
                      lse=torch.empty(B, b - a, 16, dtype=torch.float32, device="cuda"))
                 for L in src]
        h.model_prefill(chunk, cap, synth.positions(a, B, "cuda"), ws)
        for l, c in enumerate(chunk):
            outs[l][:, a:b] = c["out"]
            lses[l][:, a:b] = c["lse"]
    step = [dict(q=L["q"][:, S:].contiguous(), k=L["k"][:, S:].contiguous(),
                 v=L["v"][:, S:].contiguous(), gate=L["gate"][:, S:].contiguous(),
                 k_cache=L["k_cache"], v_cache=L["v_cache"],
                 out=torch.empty(B, 1, 16, 256, dtype=torch.bfloat16, device="cuda"),
                 lse=torch.empty(B, 1, 16, dtype=torch.float32, device="cuda")) for L in src]
    h.model_decode(step, cap, synth.positions(S, B, "cuda"), ws)
    for l, c in enumerate(step):
        outs[l][:, S:] = c["out"]
        lses[l][:, S:] = c["lse"]
    torch.cuda.synchronize()
    for l, L in enumerate(src):
        kind = L["kind"]
        for b in range(B):
            _, kr = O.rope_qk(None, _cpu(L["k"][b]), 0, kind)
            y, lse = O.prefill(_cpu(L["q"][b]), kr, _cpu(L["v"][b]), _cpu(L["gate"][b]), 0, kind)
            check_outputs(outs[l][b], lses[l][b], y, lse, f"model layer {l} ({kind}) b={b}")


@pytest.mark.parametrize("positions", [[1000], [5, 1000, 2000],
                                       [5, 100, 511, 512, 1000, 1500, 2000, 2047, 7, 700]])
def test_model_decode_graph_replay(h, positions):
    """A captured decode step of a 4-layer schedule replays to the eager result, several
    times, with other work and synchronisations in between.  The ring steps' counters are
    cleared by a kernel in the graph; B = 1 and 3 split each ring 8 ways, B = 10 4 ways."""
    say(f"model decode graph replay B={len(positions)}")
    n_layers, B, cap = 4, len(positions), 2048
    layers = _model_layers(h, n_layers, B, 1, cap, 161)
    for l, L in enumerate(layers):      # history: random rotated keys at every slot
        hist = synth.cache_inputs(162, B, L["k_cache"].shape[1], L["k_cache"].shape[1], "cuda", layer=l)
        L["k_cache"].copy_(hist["cache_k"])
        L["v_cache"].copy_(hist["cache_v"])
    pos = synth.positions(positions, B, "cuda")
    ws = torch.empty(h.model_decode_workspace_bytes(n_layers, B, cap), dtype=torch.uint8, device="cuda")
    before = [(_cpu(L["k_cache"]).clone(), _cpu(L["v_cache"]).clone()) for L in layers]
    h.model_decode(layers, cap, pos, ws)
    torch.cuda.synchronize()
    ref = [(L["out"].clone(), L["lse"].clone()) for L in layers]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            h.model_decode(layers, cap, pos, ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for L in layers:
            L["out"].zero_()
            L["lse"].zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, L in enumerate(layers):
            assert torch.equal(L["out"], ref[l][0]), (rep, l)
            assert torch.equal(L["lse"], ref[l][1]), (rep, l)
        del junk
    # and the eager result matches the oracle's decode over the caches as they were before
    # the step, with the oracle's own append of the oracle-rotated new key; every other
    # cache row is unchanged by the replays
    p = positions
    for l, L in enumerate(layers):
        kind = L["kind"]
        for b in range(B):
            _, kn = O.rope_qk(None, _cpu(L["k"][b]), p[b], kind)
            kc, vc = before[l][0][b].clone(), before[l][1][b].clone()
            O.kv_append(kc, vc, kn.to(torch.bfloat16), _cpu(L["v"][b]), p[b], kind)
            slot = p[b] if kind == "full" else p[b] % 512
            other = torch.arange(kc.shape[0]) != slot
            got_k, got_v = _cpu(L["k_cache"][b]), _cpu(L["v_cache"][b])
            assert torch.equal(got_k[other], kc[other]) and torch.equal(got_v, vc), (l, b)
            assert_rotated(got_k[slot], kn[0], L["k"][b, 0], O.KINDS[kind].rot_dim,
                           f"graph layer {l} b={b} appended key")
            y, lse = O.decode(_cpu(L["q"][b, 0]), kc, vc, _cpu(L["gate"][b, 0]), p[b], kind)
            check_outputs(ref[l][0][b, 0], ref[l][1][b, 0], y, lse, f"graph layer {l} b={b}")


@pytest.mark.parametrize("positions", [
    [(1 << 30) + 5, (1 << 31) - 1],                       # far past the context, to int32 max
    [0, 1, 31, 32, 63, 300, 511],                         # 8 splits, rings partly filled
    [0, 1, 31, 32, 63, 64, 300, 511, 512, 131072, (1 << 30) + 5, (1 << 31) - 1],  # 4 splits
    [(37 * b * b + 11 * b) % 1500 for b in range(40)],   # 640 workgroups: several rounds
])
def test_model_decode_sliding_steps(h, positions):
    """Three sliding layers (the fused ring step: append, attention, merge) at positions
    from 0 up to the largest int32 position: the rotated key lands in slot p mod 512, the
    token attends the ring's filled slots (unfilled ones hold NaN here and must not reach
    the output), as the oracle's decode over the same ring."""
    B = len(positions)
    say(f"model decode sliding steps B={B}")
    n_layers = 3
    layers = _model_layers(h, n_layers, B, 1, 512, 171)
    before = []
    for l, L in enumerate(layers):
        ring = synth.cache_inputs(172 + l, B, 512, 512, "cuda")
        for b, p in enumerate(positions):
            if p < 511:     # slots p + 1 .. 511 have never been written
                ring["cache_k"][b, p + 1:] = NAN
                ring["cache_v"][b, p + 1:] = NAN
        L["k_cache"].copy_(ring["cache_k"])
        L["v_cache"].copy_(ring["cache_v"])
        before.append((_cpu(L["k_cache"]).clone(), _cpu(L["v_cache"]).clone()))
    ws = torch.empty(h.model_decode_workspace_bytes(n_layers, B, 512), dtype=torch.uint8,
                     device="cuda")
    h.model_decode(layers, 512, synth.positions(positions, B, "cuda"), ws)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)     # NaN-safe equality of bf16 rows
    for l, L in enumerate(layers):
        for b, p in enumerate(positions):
            _, kr = O.rope_qk(None, _cpu(L["k"][b]), p, "sliding")
            K, V = before[l][0][b].clone(), before[l][1][b].clone()
            K[p % 512] = kr[0].to(torch.bfloat16)
            V[p % 512] = _cpu(L["v"][b, 0])
            got_k = _cpu(L["k_cache"][b])
            other = torch.arange(512) != p % 512
            assert torch.equal(bits(got_k[other]), bits(K[other]))
            assert torch.equal(bits(_cpu(L["v_cache"][b])), bits(V))
            assert_bf16_close(got_k[p % 512], kr[0], f"ring key layer {l} p={p}")
            assert_rotated(got_k[p % 512], kr[0], got_k[p % 512], 256, f"ring key layer {l} p={p}")
            # the oracle attends over its own ring: the snapshot with its own rotated key
            y, lse = O.decode(_cpu(L["q"][b, 0]), K, V, _cpu(L["gate"][b, 0]), p, "sliding")
            check_outputs(L["out"][b, 0], L["lse"][b, 0], y, lse, f"model step layer {l} p={p}")

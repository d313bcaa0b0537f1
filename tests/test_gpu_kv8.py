"""GPU parity of the 8-bit KV cache: quantized codes and scales bit-exact against the
oracle's quantizer, the rotating variant bit-identical to rotate-then-quantize, and the
8-bit decode against the oracle's decode of the dequantized cache.  Inputs from `synth`
(and, for the decode, codes made by the oracle's quantizer); expected values only from
`oracle`."""
import pytest
import torch

import oracle as O
import synth
from parity import check_outputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from full_gqa_attention_hattn_amd import hattn
    return hattn


def _cpu(t):
    return t.detach().cpu()


def _empty8(B, cap):
    codes = torch.full((B, cap, 4, 256), 0x55, dtype=torch.uint8, device="cuda")
    scales = torch.full((B, 4, cap), -1.0, dtype=torch.float32, device="cuda")
    return codes, scales


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_append_fp8_codes_and_scales_bit_exact(h, kind):
    say(f"append_fp8 {kind}")
    cfg = h.preset(kind)
    B, n = 2, 600 if kind == "sliding" else 300          # a ring append longer than 512
    cap = 512 if kind == "sliding" else 1024
    new = synth.layer_inputs(171, B, n, "cuda")
    k, v = new["k"].clone(), new["v"].clone()
    k[0, 5, 2] = 0                                      # all-zero head row
    v[1, 7] *= 1000                                     # large values
    k[1, 9, 1] *= 1e-30                                 # tiny values
    pos0 = [0, 700] if kind == "full" else [3, 131000]
    pos = synth.positions(pos0, B, "cuda")
    Kc, Ks = _empty8(B, cap)
    Vc, Vs = _empty8(B, cap)
    slots = torch.empty(B, n, dtype=torch.int32, device="cuda")
    h.kv_append_fp8(cfg, k, v, Kc, Vc, Ks, Vs, pos, slots)
    torch.cuda.synchronize()
    for b in range(B):
        ref_slots = O.append_slots(pos0[b], n, kind, cap)
        assert torch.equal(_cpu(slots[b]), ref_slots)
        kq, ksc = O.kv_quantize(_cpu(k[b]))
        vq, vsc = O.kv_quantize(_cpu(v[b]))
        # last writer per slot
        last = {}
        for t, s in enumerate(ref_slots.tolist()):
            if s >= 0:
                last[s] = t
        sl = torch.tensor(sorted(last))
        tt = torch.tensor([last[s] for s in sorted(last)])
        assert torch.equal(_cpu(Kc[b])[sl], kq[tt]) and torch.equal(_cpu(Vc[b])[sl], vq[tt])
        assert torch.equal(_cpu(Ks[b]).T[sl], ksc[tt]) and torch.equal(_cpu(Vs[b]).T[sl], vsc[tt])
        untouched = torch.ones(cap, dtype=torch.bool)
        untouched[sl] = False
        assert bool((_cpu(Kc[b])[untouched] == 0x55).all())


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_append_fp8_rope_equals_rope_then_append(h, kind):
    say(f"append_fp8 rope {kind}")
    cfg = h.preset(kind)
    B, n = 2, 64
    cap = 512 if kind == "sliding" else 2048
    new = synth.layer_inputs(172, B, n, "cuda")
    pos = synth.positions([0, 1500], B, "cuda")
    K1, S1 = _empty8(B, cap)
    V1, T1 = _empty8(B, cap)
    K2, S2 = _empty8(B, cap)
    V2, T2 = _empty8(B, cap)
    h.kv_append_fp8(cfg, new["k"], new["v"], K1, V1, S1, T1, pos, rope_k=True)
    kr = new["k"].clone()
    h.rope_qk(cfg, None, kr, pos)
    h.kv_append_fp8(cfg, kr, new["v"], K2, V2, S2, T2, pos)
    torch.cuda.synchronize()
    assert torch.equal(K1, K2) and torch.equal(S1, S2) and torch.equal(V1, V2) and torch.equal(T1, T2)


def _oracle_cache8(kc, vc):
    """Codes / scales by the oracle's quantizer, in the library's layouts."""
    kq, ks = O.kv_quantize(kc)
    vq, vs = O.kv_quantize(vc)
    return kq, vq, ks.T.contiguous(), vs.T.contiguous()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_decode_fp8_matches_oracle(h, kind, fused):
    say(f"decode_fp8 {kind} fused={fused}")
    cfg = h.preset(kind)
    # sliding: up to the largest int32 position (its key count must not overflow)
    positions = ([0, 31, 511, 512, 2999] if kind == "full"
                 else [0, 5, 511, 512, 1 << 20, (1 << 30) + 9, (1 << 31) - 1])
    B = len(positions)
    cap = 3000 if kind == "full" else 512
    new = synth.layer_inputs(173, B, 1, "cuda")
    cache = synth.cache_inputs(174, B, cap, cap, "cpu")
    Kc = torch.empty(B, cap, 4, 256, dtype=torch.uint8)
    Vc = torch.empty_like(Kc)
    Ks = torch.empty(B, 4, cap)
    Vs = torch.empty_like(Ks)
    for b in range(B):
        Kc[b], Vc[b], Ks[b], Vs[b] = _oracle_cache8(cache["cache_k"][b], cache["cache_v"][b])
    Kd, Vd, Ksd, Vsd = Kc.cuda(), Vc.cuda(), Ks.cuda(), Vs.cuda()
    q = new["q"].clone()
    pos = synth.positions(positions, B, "cuda")
    if not fused:
        h.rope_qk(cfg, q, None, pos)
    out = torch.empty_like(q)
    lse = torch.empty(B, 1, 16, dtype=torch.float32, device="cuda")
    ws = h.alloc_workspace_fp8(cfg, B, cap)
    h.decode_fp8(cfg, q, Kd, Vd, Ksd, Vsd, pos, new["gate"], out, lse, ws, rope_q_fused=fused)
    torch.cuda.synchronize()
    for b, p in enumerate(positions):
        y, l = O.decode_kv8(_cpu(new["q"][b, 0]), Kc[b], Vc[b], Ks[b].T, Vs[b].T,
                            _cpu(new["gate"][b, 0]), p, kind)
        check_outputs(out[b, 0], lse[b, 0], y, l, f"decode_fp8 {kind} p={p} fused={fused}")


@pytest.mark.parametrize("cap", [3000, 3001])
def test_decode_fp8_unwritten_rows_and_odd_cap(h, cap):
    """Rows past each sequence's position hold NaN codes (0x7F) and NaN scales, as a cache
    whose tail was never written may: they must not reach the output.  cap 3000 takes the
    16-byte scale loads, cap 3001 (rows not 16-byte aligned) the per-key ones."""
    say(f"decode_fp8 unwritten rows cap={cap}")
    cfg = h.preset("full")
    positions = [0, 31, 1000, cap - 2]
    B = len(positions)
    new = synth.layer_inputs(177, B, 1, "cuda")
    cache = synth.cache_inputs(178, B, cap, cap, "cpu")
    Kc = torch.empty(B, cap, 4, 256, dtype=torch.uint8)
    Vc = torch.empty_like(Kc)
    Ks = torch.empty(B, 4, cap)
    Vs = torch.empty_like(Ks)
    for b, p in enumerate(positions):
        Kc[b], Vc[b], Ks[b], Vs[b] = _oracle_cache8(cache["cache_k"][b], cache["cache_v"][b])
        Kc[b, p + 1:] = 0x7F
        Vc[b, p + 1:] = 0x7F
        Ks[b, :, p + 1:] = float("nan")
        Vs[b, :, p + 1:] = float("nan")
    Kd, Vd, Ksd, Vsd = Kc.cuda(), Vc.cuda(), Ks.cuda(), Vs.cuda()
    out = torch.empty_like(new["q"])
    lse = torch.empty(B, 1, 16, dtype=torch.float32, device="cuda")
    ws = h.alloc_workspace_fp8(cfg, B, cap)
    h.decode_fp8(cfg, new["q"], Kd, Vd, Ksd, Vsd, synth.positions(positions, B, "cuda"),
                 new["gate"], out, lse, ws, rope_q_fused=True)
    torch.cuda.synchronize()
    for b, p in enumerate(positions):
        y, l = O.decode_kv8(_cpu(new["q"][b, 0]), Kc[b], Vc[b], Ks[b].T, Vs[b].T,
                            _cpu(new["gate"][b, 0]), p, "full")
        check_outputs(out[b, 0], lse[b, 0], y, l, f"decode_fp8 unwritten cap={cap} p={p}")


def test_decode_fp8_follows_append_fp8(h):
    """End to end: append a sequence with the rotating 8-bit append, decode its last token;
    the result matches the oracle's decode over the oracle-quantized rotated keys."""
    say("append_fp8 -> decode_fp8")
    cfg = h.preset("full")
    B, S, cap = 2, 900, 1024
    inp = synth.layer_inputs(175, B, S, "cuda")
    pos0 = synth.positions(0, B, "cuda")
    Kc, Ks = _empty8(B, cap)
    Vc, Vs = _empty8(B, cap)
    h.kv_append_fp8(cfg, inp["k"], inp["v"], Kc, Vc, Ks, Vs, pos0, rope_k=True)
    p = S - 1
    q = inp["q"][:, p:p + 1].contiguous()
    g = inp["gate"][:, p:p + 1].contiguous()
    out = torch.empty_like(q)
    lse = torch.empty(B, 1, 16, dtype=torch.float32, device="cuda")
    ws = h.alloc_workspace_fp8(cfg, B, cap)
    h.decode_fp8(cfg, q, Kc, Vc, Ks, Vs, synth.positions(p, B, "cuda"), g, out, lse, ws,
                 rope_q_fused=True)
    torch.cuda.synchronize()
    for b in range(B):
        _, kr = O.rope_qk(None, _cpu(inp["k"][b]), 0, "full")
        kq, vq, ks, vs = _oracle_cache8(kr.to(torch.bfloat16), _cpu(inp["v"][b]))
        y, l = O.decode_kv8(_cpu(inp["q"][b, p]), kq, vq, ks.T, vs.T, _cpu(inp["gate"][b, p]),
                            p, "full")
        check_outputs(out[b, 0], lse[b, 0], y, l, f"append->decode fp8 b={b}")

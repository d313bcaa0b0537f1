"""Full-size workloads, run through bench.py's step (the launch configuration it times) and
checked against the oracle.

Every oracle input comes from the seeded sources or from a snapshot of the caches taken
before the step; nothing the step wrote is fed back to the oracle.  After the step, every
cache row the step must not touch is compared with its snapshot bit for bit, and every
row it appends with the oracle's own append of the oracle's rotated key.  Outputs are
compared on as many rows as the oracle computes in seconds: every row of the sliding
workloads, declared row subsets of the long full-causal ones (first, last and seeded
random rows), with the fraction checked printed; planted needles make the outputs O(1)
where long rows would average them away."""
import gc
import math

import pytest
import torch

import oracle as O
import synth
from parity import Coverage, assert_rotated, check_needle_row, check_outputs, row_blocks, say

pytestmark = pytest.mark.gpu

WINDOW = 512


def _cpu(t):
    return t.detach().cpu()


@pytest.fixture(scope="module")
def bench():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench as B
    return B


def _free(*objs):
    for o in objs:
        del o
    gc.collect()
    torch.cuda.empty_cache()


def _needle_target(V_b_j, g):
    return [_cpu(V_b_j[hq // 4]).double() / (1 + math.exp(-float(g[hq]))) for hq in range(16)]


def _rows_unchanged(after, before, slot, name):
    """Every row but `slot` of the caches [B, rows, 4, 256] equal to the snapshot, bit for
    bit (device tensors, compared in place)."""
    assert torch.equal(after[:, :slot], before[:, :slot]), f"{name}: rows below the append changed"
    assert torch.equal(after[:, slot + 1:], before[:, slot + 1:]), \
        f"{name}: rows above the append changed"


# ------------------------------------------------------------------ workload 2 --
def test_sliding_prefill_b4_s32768(bench):
    """Every output row of all four sequences (131072 rows x 16 heads), plus a visible
    needle at distance 511 and an invisible one at 512."""
    say("workload 2: sliding prefill B=4 S=32768")
    wl = bench.make_workload(2)
    wl.q[1, 20000] = 0
    synth.plant_needle(wl.q, wl.k_src, 1, 20000, 20000 - 511, (127, 255), 16.0)
    synth.plant_needle(wl.q, wl.k_src, 2, 25000, 25000 - 512, (127, 255), 16.0)
    wl.step()
    torch.cuda.synchronize()
    S = wl.S
    for b in range(wl.B):
        _, kr = O.rope_qk(None, _cpu(wl.k_src[b]), 0, "sliding")
        assert_rotated(_cpu(wl.k[b]), kr, wl.k_src[b], 256, f"w2 b={b} rotated keys")
        q, v, g = _cpu(wl.q[b]), _cpu(wl.v[b]), _cpu(wl.gate[b])
        out, lse = _cpu(wl.out[b]), _cpu(wl.lse[b])
        cov = Coverage(f"w2 b={b}", S)
        for rows in row_blocks(range(S)):
            y, l = O.prefill(q, kr, v, g, 0, "sliding", rows=rows)
            cov.check(out[rows], lse[rows], y, l)
        cov.report()
    tgt = _needle_target(wl.v[1, 20000 - 511], wl.gate[1, 20000])
    for hq in range(16):
        got = _cpu(wl.out[1, 20000, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    tgt = _needle_target(wl.v[2, 25000 - 512], wl.gate[2, 25000])
    for hq in range(16):
        got = _cpu(wl.out[2, 25000, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) > 0.5
    _free(wl)


# ------------------------------------------------------------------ workload 3 --
def test_full_prefill_b1_s131072(bench):
    """Rows 0..1023, the last 1024 rows and 2048 seeded random rows (the declared subset),
    plus a needle at key 0 owning the last row."""
    say("workload 3: full prefill B=1 S=131072")
    wl = bench.make_workload(3)
    S = wl.S
    last = S - 1
    wl.q[0, last] = 0
    synth.plant_needle(wl.q, wl.k_src, 0, last, 0, (128, 200), 16.0)
    wl.step()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(6)
    rows = (list(range(1024)) + list(range(S - 1024, S))
            + torch.randperm(S - 2048, generator=gen)[:2048].add(1024).tolist())
    _, kr = O.rope_qk(None, _cpu(wl.k_src[0]), 0, "full")
    assert_rotated(_cpu(wl.k[0]), kr, wl.k_src[0], 64, "w3 rotated keys")
    q, v, g = _cpu(wl.q[0]), _cpu(wl.v[0]), _cpu(wl.gate[0])
    out, lse = _cpu(wl.out[0]), _cpu(wl.lse[0])
    cov = Coverage("w3", S)
    for blk in row_blocks(rows):
        y, l = O.prefill(q, kr, v, g, 0, "full", rows=blk)
        cov.check(out[blk], lse[blk], y, l)
    cov.report()
    tgt = _needle_target(wl.v[0, 0], wl.gate[0, last])
    for hq in range(16):
        got = _cpu(wl.out[0, last, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    _free(wl)


# ------------------------------------------------------------------ workload 4 --
def test_mixed_decode_b32_p131072(bench):
    """All 32 sequences of all four layers.  The oracle's caches are the pre-step snapshot
    with the oracle's own append of the oracle-rotated new key."""
    say("workload 4: mixed decode B=32 at 131072")
    wl = bench.make_workload(4)
    snaps = [(L["K"].clone(), L["V"].clone()) for L in wl.layers]
    wl.step()
    torch.cuda.synchronize()
    p, B = wl.p, wl.B
    for li, L in enumerate(wl.layers):
        kind = L["kind"]
        K0, V0 = snaps[li]
        slot = p if kind == "full" else p % WINDOW
        slots = _cpu(L["slots"])
        assert torch.equal(slots, O.append_slots(p, 1, kind, L["cap"]).expand(B, 1)), li
        _rows_unchanged(L["K"], K0, slot, f"w4 layer {li} K")
        _rows_unchanged(L["V"], V0, slot, f"w4 layer {li} V")
        assert torch.equal(L["V"][:, slot], L["v"][:, 0])
        rot = O.KINDS[kind].rot_dim
        cov = Coverage(f"w4 layer {li} ({kind})", B, unit="sequences")
        for b in range(B):
            _, kn = O.rope_qk(None, _cpu(L["k_src"][b]), p, kind)
            assert_rotated(_cpu(L["K"][b, slot]), kn[0], L["k_src"][b, 0], rot,
                           f"w4 layer {li} b={b} appended key")
            n_hist = p if kind == "full" else WINDOW
            kc = _cpu(K0[b, :n_hist]).clone()
            vc = _cpu(V0[b, :n_hist]).clone()
            if kind == "full":
                kc = torch.cat([kc, torch.zeros_like(kc[:1])])
                vc = torch.cat([vc, torch.zeros_like(vc[:1])])
            O.kv_append(kc, vc, kn.to(torch.bfloat16), _cpu(L["v"][b]), p, kind)
            y, l = O.decode(_cpu(L["q"][b, 0]), kc, vc, _cpu(L["gate"][b, 0]), p, kind)
            cov.check(_cpu(L["out"][b]), _cpu(L["lse"][b]), y[None], l[None])
        cov.report()
        del K0, V0
    snaps.clear()
    _free(wl)


# ------------------------------------------------------------------ workload 5 --
def test_full_1m_chunk_and_decode(bench):
    """The last 128 rows and 128 seeded random rows of the 4096-query chunk (the declared
    subset) plus rows 0..3, the decode at 2^20, and decode == prefill row at 2^20 - 1."""
    say("workload 5: 1M full layer chunk + decode")
    wl = bench.make_workload(5)
    row = wl.C - 1
    wl.q[0, row] = 0
    synth.plant_needle(wl.q, wl.K, 0, row, 0, (128, 200), 16.0)    # cache row 0 as the needle
    K0, V0 = wl.K.clone(), wl.V.clone()
    wl.step()
    torch.cuda.synchronize()
    slots = _cpu(wl.slots)[0]
    assert torch.equal(slots, torch.arange(wl.L0, wl.L0 + wl.C, dtype=torch.int32))
    assert int(_cpu(wl.slotsd)[0, 0]) == wl.pd
    _, kr = O.rope_qk(None, _cpu(wl.k_src[0]), wl.L0, "full")
    _, kd = O.rope_qk(None, _cpu(wl.kd_src[0]), wl.pd, "full")
    # the chunk at L0 .. L0 + C - 1 and the decode token at pd = L0 + C, nothing else
    L0, pd = wl.L0, wl.pd
    for name, T, T0, chunk, tok in (("K", wl.K, K0, wl.k, wl.kd), ("V", wl.V, V0, wl.v, wl.vd)):
        assert torch.equal(T[:, :L0], T0[:, :L0]), f"w5 {name}: history rows changed"
        assert torch.equal(T[:, L0:pd], chunk), f"w5 {name}: chunk rows are not the appended tokens"
        assert torch.equal(T[:, pd], tok[:, 0]), f"w5 {name}: decode row is not the appended token"
        assert torch.equal(T[:, pd + 1:], T0[:, pd + 1:]), f"w5 {name}: rows past the append changed"
    assert_rotated(_cpu(wl.k[0]), kr, wl.k_src[0], 64, "w5 rotated chunk keys")
    assert_rotated(_cpu(wl.kd[0]), kd, wl.kd_src[0], 64, "w5 rotated decode key")
    # oracle caches: the pre-step history, then the oracle's append of its rotated keys
    kc = _cpu(K0[0, :wl.pd + 1]).clone()
    vc = _cpu(V0[0, :wl.pd + 1]).clone()
    del K0, V0
    torch.cuda.empty_cache()
    O.kv_append(kc, vc, kr.to(torch.bfloat16), _cpu(wl.v[0]), wl.L0, "full")
    O.kv_append(kc, vc, kd.to(torch.bfloat16), _cpu(wl.vd[0]), wl.pd, "full")
    kc, vc = kc.float(), vc.float()
    gen = torch.Generator().manual_seed(7)
    rand = torch.randperm(wl.C - 128, generator=gen)[:128].tolist()
    rows = [0, 1, 2, 3] + list(range(wl.C - 128, wl.C)) + rand
    q, g = _cpu(wl.q[0]), _cpu(wl.gate[0])
    out, lse = _cpu(wl.out[0]), _cpu(wl.lse[0])
    cov = Coverage("w5 prefill", wl.C)
    for blk in row_blocks(rows):
        y, l = O.prefill(q, kc, vc, g, wl.L0, "full", rows=blk)
        cov.check(out[blk], lse[blk], y, l)
        say(f"  w5 rows {int(blk[0])}..{int(blk[-1])} ok")
    cov.report()
    tgt = _needle_target(wl.V[0, 0], wl.gate[0, row])
    for hq in range(16):
        got = _cpu(wl.out[0, row, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    yd, ld = O.decode(_cpu(wl.qd[0, 0]), kc, vc, _cpu(wl.gd[0, 0]), wl.pd, "full")
    check_outputs(_cpu(wl.outd[0, 0]), _cpu(wl.lsed[0, 0]), yd, ld, "w5 decode p=2^20")
    del kc, vc
    # cross-path: decode of the chunk's last query (p = 2^20 - 1) equals prefill row 4095
    h = wl.h
    od = torch.empty_like(wl.qd)
    lsed = torch.empty_like(wl.lsed)
    h.decode(wl.cfg, wl.q[:, row:row + 1].contiguous(), wl.K, wl.V,
             synth.positions(wl.L0 + row, 1, "cuda"), wl.gate[:, row:row + 1].contiguous(), od,
             lsed, wl.ws, rope_q_fused=True)
    torch.cuda.synchronize()
    assert float((od[0, 0].float() - wl.out[0, row].float()).abs().max()) < 1e-2
    assert float((lsed[0, 0] - wl.lse[0, row]).abs().max()) < 1e-3
    _free(wl)


# ------------------------------------------------------------------ workload 6 --
def test_sliding_ring_1m_chunk_and_decode(bench):
    """Every row of the 4096-query chunk against the ring (needle rows against their
    targets), the ring after the chunk's append, and the ring decode at 2^20."""
    say("workload 6: 1M sliding layer, chunk against the ring + decode")
    wl = bench.make_workload(6)
    synth.plant_needle(wl.q, wl.k_src, 0, 1500, 1500 - 511, (127, 255), 16.0)
    synth.plant_needle(wl.q, wl.k_src, 0, 2500, 2500 - 512, (127, 255), 16.0)
    wl.step()
    torch.cuda.synchronize()
    P = wl.P
    _, kr = O.rope_qk(None, _cpu(wl.k_src[0]), P, "sliding")
    assert_rotated(_cpu(wl.k[0]), kr, wl.k_src[0], 256, "w6 rotated chunk keys")
    q, v, g = _cpu(wl.q[0]), _cpu(wl.v[0]), _cpu(wl.gate[0])
    K0, V0 = _cpu(wl.K0[0]), _cpu(wl.V0[0])     # the ring as the previous chunk left it
    out, lse = _cpu(wl.out[0]), _cpu(wl.lse[0])
    cov = Coverage("w6 prefill", wl.C)
    needles = {1500, 2500}
    for blk in row_blocks(range(wl.C)):
        keep = torch.tensor([int(r) not in needles for r in blk])
        blk = blk[keep]
        y, l = O.prefill_ring(q, kr, v, K0, V0, g, P, rows=blk)
        cov.check(out[blk], lse[blk], y, l)
    cov.report()
    for r in sorted(needles):
        yn, ln = O.prefill_ring(q, kr, v, K0, V0, g, P, rows=torch.tensor([r]))
        check_needle_row(_cpu(wl.out[0, r]), _cpu(wl.lse[0, r]), yn[0], ln[0], f"w6 needle row {r}")
    tgt = _needle_target(wl.v[0, 1500 - 511], wl.gate[0, 1500])
    for hq in range(16):
        got = _cpu(wl.out[0, 1500, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    tgt = _needle_target(wl.v[0, 2500 - 512], wl.gate[0, 2500])
    for hq in range(16):
        got = _cpu(wl.out[0, 2500, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) > 0.5
    # the ring after the chunk and the decode token, built by the oracle's own appends:
    # in fp32 for the key rotation bound, in bf16 (the cache format) for the decode
    _, kd = O.rope_qk(None, _cpu(wl.kd_src[0]), wl.pd, "sliding")
    ring_k, ring_v = K0.clone(), V0.clone()
    ring_kf, ring_vf = K0.float(), V0.float()
    for kk, vv, pos in ((kr, v, P), (kd, _cpu(wl.vd[0]), wl.pd)):
        O.kv_append(ring_k, ring_v, kk.to(torch.bfloat16), vv, pos, "sliding")
        O.kv_append(ring_kf, ring_vf, kk, vv.float(), pos, "sliding")
    assert torch.equal(_cpu(wl.V[0]), ring_v), "w6 ring values after the appends"
    assert_rotated(_cpu(wl.K[0]), ring_kf, ring_k, 256, "w6 ring keys after the appends")
    yd, ld = O.decode(_cpu(wl.qd[0, 0]), ring_k, ring_v, _cpu(wl.gd[0, 0]), wl.pd, "sliding")
    check_outputs(_cpu(wl.outd[0, 0]), _cpu(wl.lsed[0, 0]), yd, ld, "w6 ring decode p=2^20")
    _free(wl)


# ------------------------------------------------------------------ workload 8 --
def test_model_36_layers_1m_chunk(bench):
    """Sliding layers 0, 1, 2 and 34 on every row of the chunk, full layers 3 and 35 on the
    last 64 and 64 seeded random rows; each checked layer's cache or ring against the
    oracle's append of the chunk onto its pre-step snapshot."""
    say("workload 8: 36-layer chunk of 4096 at 1M")
    wl = bench.make_workload(8)
    full_ids, sl_ids = (3, 35), (0, 1, 2, 34)
    snaps = {l: (wl.layers[l]["k_cache"].clone(), wl.layers[l]["v_cache"].clone())
             for l in full_ids}
    wl.step()
    torch.cuda.synchronize()
    P, C = wl.P, wl.S
    gen = torch.Generator().manual_seed(8)
    for l in sl_ids + full_ids:
        L = wl.layers[l]
        kind = L["kind"]
        assert kind == ("full" if l in full_ids else "sliding")
        _, kr = O.rope_qk(None, _cpu(L["k"][0]), P, kind)
        q, v, g = _cpu(L["q"][0]), _cpu(L["v"][0]), _cpu(L["gate"][0])
        out, lse = _cpu(L["out"][0]), _cpu(L["lse"][0])
        cov = Coverage(f"w8 layer {l} ({kind})", C)
        if kind == "sliding":
            K0, V0 = next((_cpu(k[0]), _cpu(vv[0])) for (LL, k, vv) in wl.rings0 if LL is L)
            for blk in row_blocks(range(C)):
                y, lo = O.prefill_ring(q, kr, v, K0, V0, g, P, rows=blk)
                cov.check(out[blk], lse[blk], y, lo)
            ring_kf, ring_v = K0.float(), V0.clone()
            O.kv_append(ring_kf, ring_v, kr, v, P, "sliding")
            assert torch.equal(_cpu(L["v_cache"][0]), ring_v), f"w8 layer {l} ring values"
            assert_rotated(_cpu(L["k_cache"][0]), ring_kf, K0, 256, f"w8 layer {l} ring keys")
        else:
            K0, V0 = snaps[l]
            kc = _cpu(K0[0, :P + C]).clone()
            vc = _cpu(V0[0, :P + C]).clone()
            assert torch.equal(L["k_cache"][:, :P], K0[:, :P]), f"w8 layer {l} history keys"
            assert torch.equal(L["v_cache"][:, :P], V0[:, :P]), f"w8 layer {l} history values"
            assert torch.equal(L["k_cache"][:, P + C:], K0[:, P + C:])
            assert torch.equal(L["v_cache"][:, P:P + C], L["v"]), f"w8 layer {l} appended values"
            assert_rotated(_cpu(L["k_cache"][0, P:P + C]), kr, L["k"][0], 64,
                           f"w8 layer {l} appended keys")
            del K0, V0
            snaps.pop(l)
            O.kv_append(kc, vc, kr.to(torch.bfloat16), v, P, "full")
            kc, vc = kc.float(), vc.float()
            rows = list(range(C - 64, C)) + torch.randperm(C - 64, generator=gen)[:64].tolist()
            for blk in row_blocks(rows):
                y, lo = O.prefill(q, kc, vc, g, P, "full", rows=blk)
                cov.check(out[blk], lse[blk], y, lo)
            del kc, vc
        cov.report()
    _free(wl)


# ------------------------------------------------------------------ workload 7 --
def test_model_36_layers_1m_decode(bench):
    """All 27 sliding layers and full layers 3, 19 and 35: output against the oracle's
    decode over the pre-step cache with the oracle's append of the new token, and the
    cache after the step against the same append."""
    say("workload 7: 36-layer decode at 2^20")
    wl = bench.make_workload(7)
    p = wl.P
    full_ids = (3, 19, 35)
    checked = [l for l, L in enumerate(wl.layers) if L["kind"] == "sliding"] + list(full_ids)
    snaps = {l: (wl.layers[l]["k_cache"].clone(), wl.layers[l]["v_cache"].clone())
             for l in checked}
    wl.step()
    torch.cuda.synchronize()
    cov = Coverage("w7", len(wl.layers), unit="layers")
    for l in checked:
        L = wl.layers[l]
        kind = L["kind"]
        K0, V0 = snaps.pop(l)
        slot = p if kind == "full" else p % WINDOW
        _rows_unchanged(L["k_cache"], K0, slot, f"w7 layer {l} K")
        _rows_unchanged(L["v_cache"], V0, slot, f"w7 layer {l} V")
        assert torch.equal(L["v_cache"][:, slot], L["v"][:, 0]), f"w7 layer {l} appended value"
        _, kn = O.rope_qk(None, _cpu(L["k"][0]), p, kind)
        assert_rotated(_cpu(L["k_cache"][0, slot]), kn[0], L["k"][0, 0], O.KINDS[kind].rot_dim,
                       f"w7 layer {l} appended key")
        n = p + 1 if kind == "full" else WINDOW
        kc, vc = _cpu(K0[0, :n]).clone(), _cpu(V0[0, :n]).clone()
        del K0, V0
        O.kv_append(kc, vc, kn.to(torch.bfloat16), _cpu(L["v"][0]), p, kind)
        y, lse = O.decode(_cpu(L["q"][0, 0]), kc, vc, _cpu(L["gate"][0, 0]), p, kind)
        cov.check(_cpu(L["out"][0]), _cpu(L["lse"][0]), y[None], lse[None])
        del kc, vc
    cov.report()
    _free(wl)


# ------------------------------------------------------------------ workloads 9, 10 --
def _oracle_kv8_rows(src_rows, chunk=65536):
    """The oracle's dequantized values of a [n, 4, 256] bf16 history, quantized by the
    oracle itself, chunk by chunk (fp32 [n, 4, 256])."""
    outs = []
    for r0 in range(0, src_rows.shape[0], chunk):
        c, s = O.kv_quantize(src_rows[r0:r0 + chunk])
        outs.append(O.kv_dequantize(c, s))
    say(f"  oracle quantized {src_rows.shape[0]} rows")
    return torch.cat(outs)


def _check_kv8_workload(bench, idx, seqs, sample_rows):
    wl = bench.Kv8DecodeWorkload(idx, keep_source=True)
    wl.step()
    torch.cuda.synchronize()
    P = wl.P
    gen = torch.Generator().manual_seed(9 + idx)
    cov = Coverage(f"w{idx} kv8 decode", wl.B, unit="sequences")
    for b in seqs:
        src_k, src_v = _cpu(wl.source["cache_k"][b, :P]), _cpu(wl.source["cache_v"][b, :P])
        # codes and scales of sampled rows, bit for bit
        rows = torch.unique(torch.cat([torch.randint(0, P, (sample_rows,), generator=gen),
                                       torch.arange(P - 64, P)]))
        kq, ks = O.kv_quantize(src_k[rows])
        vq, vs = O.kv_quantize(src_v[rows])
        assert torch.equal(_cpu(wl.K[b])[rows], kq) and torch.equal(_cpu(wl.V[b])[rows], vq)
        assert torch.equal(_cpu(wl.Ks[b]).T[rows], ks) and torch.equal(_cpu(wl.Vs[b]).T[rows], vs)
        # the decode over the whole history, every code made by the oracle
        _, kn = O.rope_qk(None, _cpu(wl.k[b]), P, "full")
        kc = torch.cat([_oracle_kv8_rows(src_k), O.kv_dequantize(*O.kv_quantize(kn.to(torch.bfloat16)))])
        vc = torch.cat([_oracle_kv8_rows(src_v), O.kv_dequantize(*O.kv_quantize(_cpu(wl.v[b])))])
        y, lse = O.decode(_cpu(wl.q[b, 0]), kc, vc, _cpu(wl.gate[b, 0]), P, "full")
        cov.check(_cpu(wl.out[b]), _cpu(wl.lse[b]), y[None], lse[None])
        del kc, vc
    cov.report()
    _free(wl)


def test_kv8_decode_b32_p131072(bench):
    say("workload 10: 8-bit KV decode, B=32 at 131072")
    _check_kv8_workload(bench, 10, (0, 7, 19, 31), 2048)


def test_kv8_decode_1m(bench):
    say("workload 9: 8-bit KV decode at 2^20")
    _check_kv8_workload(bench, 9, (0,), 16384)

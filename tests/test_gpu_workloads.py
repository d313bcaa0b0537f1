"""Full-size workloads, run through bench.py's step (the launch configuration it times),
checked against the oracle on sampled rows the oracle can compute one by one, plus planted
needles whose outputs are O(1) and a decode-vs-prefill cross-check at 1M positions."""
import gc
import math

import pytest
import torch

import oracle as O
import synth
from parity import check_needle_row, check_outputs, say

pytestmark = pytest.mark.gpu


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


def test_sliding_prefill_b4_s32768(bench):
    say("workload 2: sliding prefill B=4 S=32768")
    wl = bench.make_workload(2)
    # needles: (b, i, j) visible at distance 511 and invisible at 512, dims turning slowest
    wl.q[1, 20000] = 0
    synth.plant_needle(wl.q, wl.k_src, 1, 20000, 20000 - 511, (127, 255), 16.0)
    synth.plant_needle(wl.q, wl.k_src, 2, 25000, 25000 - 512, (127, 255), 16.0)
    wl.step()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(5)
    for b in (0, 1, 2, 3):
        rows = sorted(set(list(range(0, 40)) + list(range(500, 530)) + list(range(32768 - 40, 32768))
                          + torch.randint(0, 32768, (24,), generator=gen).tolist()
                          + ([20000] if b == 1 else []) + ([25000] if b == 2 else [])))
        rows_t = torch.tensor(rows)
        _, kr = O.rope_qk(None, _cpu(wl.k_src[b]), 0, "sliding")
        y, l = O.prefill(_cpu(wl.q[b]), kr, _cpu(wl.v[b]), _cpu(wl.gate[b]), 0, "sliding",
                         rows=rows_t)
        check_outputs(_cpu(wl.out[b])[rows_t], _cpu(wl.lse[b])[rows_t], y, l,
                      f"w2 b={b} ({len(rows)} rows)")
    # the visible needle owns row 20000 of sequence 1
    tgt = _needle_target(wl.v[1, 20000 - 511], wl.gate[1, 20000])
    for hq in range(16):
        got = _cpu(wl.out[1, 20000, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    tgt = _needle_target(wl.v[2, 25000 - 512], wl.gate[2, 25000])
    for hq in range(16):
        got = _cpu(wl.out[2, 25000, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) > 0.5
    _free(wl)


def test_full_prefill_b1_s131072(bench):
    say("workload 3: full prefill B=1 S=131072")
    wl = bench.make_workload(3)
    last = 131071
    wl.q[0, last] = 0
    synth.plant_needle(wl.q, wl.k_src, 0, last, 0, (128, 200), 16.0)
    wl.step()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(6)
    rows = sorted(set(list(range(0, 24)) + list(range(131072 - 24, 131072))
                      + torch.randint(0, 131072, (24,), generator=gen).tolist()))
    rows_t = torch.tensor(rows)
    _, kr = O.rope_qk(None, _cpu(wl.k_src[0]), 0, "full")
    y, l = O.prefill(_cpu(wl.q[0]), kr, _cpu(wl.v[0]), _cpu(wl.gate[0]), 0, "full", rows=rows_t)
    check_outputs(_cpu(wl.out[0])[rows_t], _cpu(wl.lse[0])[rows_t], y, l, f"w3 ({len(rows)} rows)")
    tgt = _needle_target(wl.v[0, 0], wl.gate[0, last])
    for hq in range(16):
        got = _cpu(wl.out[0, last, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    _free(wl)


def test_mixed_decode_b32_p131072(bench):
    say("workload 4: mixed decode B=32 at 131072")
    wl = bench.make_workload(4)
    wl.step()
    torch.cuda.synchronize()
    p = wl.p
    for li, L in enumerate(wl.layers):
        kind = L["kind"]
        seqs = range(wl.B) if kind == "sliding" else (0, 13, 31)
        slots = _cpu(L["slots"])
        assert torch.equal(slots, O.append_slots(p, 1, kind, L["cap"]).expand(wl.B, 1)), li
        for b in seqs:
            _, kn = O.rope_qk(None, _cpu(L["k_src"][b]), p, kind)
            if kind == "full":
                kc = torch.cat([_cpu(L["K"][b, :p]).float(), kn])
                vc = torch.cat([_cpu(L["V"][b, :p]).float(), _cpu(L["v"][b]).float()])
            else:
                kc = _cpu(L["K"][b]).float()
                vc = _cpu(L["V"][b]).float()
                s = p % 512
                # the ring slot of the new token holds what the oracle rotates itself
                kc[s] = kn[0]
                vc[s] = _cpu(L["v"][b, 0]).float()
            y, l = O.decode(_cpu(L["q"][b, 0]), kc, vc, _cpu(L["gate"][b, 0]), p, kind)
            check_outputs(_cpu(L["out"][b, 0]), _cpu(L["lse"][b, 0]), y, l,
                          f"w4 layer {li} ({kind}) b={b}")
    _free(wl)


def test_full_1m_chunk_and_decode(bench):
    say("workload 5: 1M full layer chunk + decode")
    wl = bench.make_workload(5)
    row = wl.C - 1
    wl.q[0, row] = 0
    synth.plant_needle(wl.q, wl.K, 0, row, 0, (128, 200), 16.0)    # cache row 0 as the needle
    wl.step()
    torch.cuda.synchronize()
    slots = _cpu(wl.slots)[0]
    assert torch.equal(slots, torch.arange(wl.L0, wl.L0 + wl.C, dtype=torch.int32))
    assert int(_cpu(wl.slotsd)[0, 0]) == wl.pd
    # oracle keys: cached rows as given, then the chunk and the decode token rotated by it
    _, kr = O.rope_qk(None, _cpu(wl.k_src[0]), wl.L0, "full")
    _, kd = O.rope_qk(None, _cpu(wl.kd_src[0]), wl.pd, "full")
    kc = torch.cat([_cpu(wl.K[0, :wl.L0]).float(), kr, kd])
    vc = torch.cat([_cpu(wl.V[0, :wl.L0]).float(), _cpu(wl.v[0]).float(), _cpu(wl.vd[0]).float()])
    gen = torch.Generator().manual_seed(7)
    rows = sorted(set([0, 1, 2, 3, row - 3, row - 2, row - 1, row]
                      + torch.randint(0, wl.C, (6,), generator=gen).tolist()))
    rows_t = torch.tensor(rows)
    y, l = O.prefill(_cpu(wl.q[0]), kc, vc, _cpu(wl.gate[0]), wl.L0, "full", rows=rows_t)
    check_outputs(_cpu(wl.out[0])[rows_t], _cpu(wl.lse[0])[rows_t], y, l, f"w5 prefill {rows}")
    tgt = _needle_target(wl.V[0, 0], wl.gate[0, row])
    for hq in range(16):
        got = _cpu(wl.out[0, row, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    yd, ld = O.decode(_cpu(wl.qd[0, 0]), kc, vc, _cpu(wl.gd[0, 0]), wl.pd, "full")
    check_outputs(_cpu(wl.outd[0, 0]), _cpu(wl.lsed[0, 0]), yd, ld, "w5 decode p=2^20")
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


def test_sliding_ring_1m_chunk_and_decode(bench):
    say("workload 6: 1M sliding layer, chunk against the ring + decode")
    wl = bench.make_workload(6)
    # needles among the chunk's own keys: visible at distance 511, invisible at 512
    synth.plant_needle(wl.q, wl.k_src, 0, 1500, 1500 - 511, (127, 255), 16.0)
    synth.plant_needle(wl.q, wl.k_src, 0, 2500, 2500 - 512, (127, 255), 16.0)
    wl.step()
    torch.cuda.synchronize()
    P = wl.P
    _, kr = O.rope_qk(None, _cpu(wl.k_src[0]), P, "sliding")
    gen = torch.Generator().manual_seed(8)
    rows = sorted(set(list(range(0, 40)) + list(range(495, 530))
                      + list(range(wl.C - 20, wl.C))
                      + torch.randint(0, wl.C, (24,), generator=gen).tolist()) - {1500, 2500})
    rows_t = torch.tensor(rows)
    y, l = O.prefill_ring(_cpu(wl.q[0]), kr, _cpu(wl.v[0]), _cpu(wl.K0[0]), _cpu(wl.V0[0]),
                          _cpu(wl.gate[0]), P, rows=rows_t)
    check_outputs(_cpu(wl.out[0])[rows_t], _cpu(wl.lse[0])[rows_t], y, l,
                  f"w6 prefill ({len(rows)} rows)")
    for r in (1500, 2500):
        yn, ln = O.prefill_ring(_cpu(wl.q[0]), kr, _cpu(wl.v[0]), _cpu(wl.K0[0]), _cpu(wl.V0[0]),
                                _cpu(wl.gate[0]), P, rows=torch.tensor([r]))
        check_needle_row(_cpu(wl.out[0, r]), _cpu(wl.lse[0, r]), yn[0], ln[0], f"w6 needle row {r}")
    tgt = _needle_target(wl.v[0, 1500 - 511], wl.gate[0, 1500])
    for hq in range(16):
        got = _cpu(wl.out[0, 1500, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) < 2e-2
    tgt = _needle_target(wl.v[0, 2500 - 512], wl.gate[0, 2500])
    for hq in range(16):
        got = _cpu(wl.out[0, 2500, hq]).double()
        assert float((got - tgt[hq]).norm() / tgt[hq].norm()) > 0.5
    # decode at 2^20 over the ring after the chunk and the new token were appended
    ring_k = _cpu(wl.K0[0]).float()
    ring_v = _cpu(wl.V0[0]).float()
    O.kv_append(ring_k, ring_v, kr, _cpu(wl.v[0]).float(), P, "sliding")
    _, kd = O.rope_qk(None, _cpu(wl.kd_src[0]), wl.pd, "sliding")
    O.kv_append(ring_k, ring_v, kd, _cpu(wl.vd[0]).float(), wl.pd, "sliding")
    yd, ld = O.decode(_cpu(wl.qd[0, 0]), ring_k, ring_v, _cpu(wl.gd[0, 0]), wl.pd, "sliding")
    check_outputs(_cpu(wl.outd[0, 0]), _cpu(wl.lsed[0, 0]), yd, ld, "w6 ring decode p=2^20")
    _free(wl)


def _oracle_layer_rows(wl, L, rows):
    """Oracle prefill rows of one layer of a whole-model chunk workload (B=1)."""
    kind = L["kind"]
    _, kr = O.rope_qk(None, _cpu(L["k"][0]), wl.P, kind)
    if kind == "full":
        kc = torch.cat([_cpu(L["k_cache"][0, :wl.P]).float(), kr])
        vc = torch.cat([_cpu(L["v_cache"][0, :wl.P]).float(), _cpu(L["v"][0]).float()])
        return O.prefill(_cpu(L["q"][0]), kc, vc, _cpu(L["gate"][0]), wl.P, kind, rows=rows)
    K0, V0 = next((k, v) for (LL, k, v) in wl.rings0 if LL is L)
    return O.prefill_ring(_cpu(L["q"][0]), kr, _cpu(L["v"][0]), _cpu(K0[0]), _cpu(V0[0]),
                          _cpu(L["gate"][0]), wl.P, rows=rows)


def test_model_36_layers_1m_chunk(bench):
    say("workload 8: 36-layer chunk of 4096 at 1M")
    wl = bench.make_workload(8)
    wl.step()
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 511, 512, 2047, 4094, 4095])
    for l in (0, 3, 34, 35):          # sliding and full, first and last of the schedule
        L = wl.layers[l]
        y, lse = _oracle_layer_rows(wl, L, rows)
        check_outputs(_cpu(L["out"][0])[rows], _cpu(L["lse"][0])[rows], y, lse,
                      f"w8 layer {l} ({L['kind']})")
    _free(wl)


def test_model_36_layers_1m_decode(bench):
    say("workload 7: 36-layer decode at 2^20")
    wl = bench.make_workload(7)
    wl.step()
    torch.cuda.synchronize()
    p = wl.P
    for l in (0, 3, 34, 35):
        L = wl.layers[l]
        kind = L["kind"]
        _, kn = O.rope_qk(None, _cpu(L["k"][0]), p, kind)
        if kind == "full":
            kc = torch.cat([_cpu(L["k_cache"][0, :p]).float(), kn])
            vc = torch.cat([_cpu(L["v_cache"][0, :p]).float(), _cpu(L["v"][0]).float()])
        else:
            kc, vc = _cpu(L["k_cache"][0]).float(), _cpu(L["v_cache"][0]).float()
            kc[p % 512] = kn[0]
            vc[p % 512] = _cpu(L["v"][0, 0]).float()
        y, lse = O.decode(_cpu(L["q"][0, 0]), kc, vc, _cpu(L["gate"][0, 0]), p, kind)
        check_outputs(_cpu(L["out"][0, 0]), _cpu(L["lse"][0, 0]), y, lse, f"w7 layer {l} ({kind})")
    _free(wl)


def _oracle_kv8_rows(src_rows, chunk=65536):
    """The oracle's dequantized values of a [n, 4, 256] bf16 history, quantized by the
    oracle itself, chunk by chunk (fp32 [n, 4, 256])."""
    outs = []
    for r0 in range(0, src_rows.shape[0], chunk):
        c, s = O.kv_quantize(src_rows[r0:r0 + chunk])
        outs.append(O.kv_dequantize(c, s))
        say(f"  oracle quantized rows {r0}..{min(r0 + chunk, src_rows.shape[0]) - 1}")
    return torch.cat(outs)


def _check_kv8_workload(bench, idx, seqs, sample_rows):
    wl = bench.Kv8DecodeWorkload(idx, keep_source=True)
    wl.step()
    torch.cuda.synchronize()
    P = wl.P
    gen = torch.Generator().manual_seed(9 + idx)
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
        check_outputs(_cpu(wl.out[b, 0]), _cpu(wl.lse[b, 0]), y, lse, f"w{idx} kv8 decode b={b}")
        del kc, vc
    _free(wl)


def test_kv8_decode_b32_p131072(bench):
    say("workload 10: 8-bit KV decode, B=32 at 131072")
    _check_kv8_workload(bench, 10, (0, 31), 4096)


def test_kv8_decode_1m(bench):
    say("workload 9: 8-bit KV decode at 2^20")
    _check_kv8_workload(bench, 9, (0,), 16384)

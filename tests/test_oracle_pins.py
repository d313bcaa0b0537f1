"""Pins for the CPU oracle: closed forms, the pages' printed constants and figures, a
library attention routine, brute force on tiny inputs, and invariants.  Each test is
chosen so that a plausible slip in the oracle (a wrong sign, pairing, frequency base,
scale, window edge, head mapping, ring slot or dropped gate) fails at least one of them.
CPU only."""
import cmath
import json
import math
import pathlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synth

GOLD = pathlib.Path(__file__).parent / "golden"


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32)


# ----------------------------------------------------------------- page constants --
def test_constants_match_pages():
    g = json.loads((GOLD / "page_constants.json").read_text())
    assert O.N_Q_HEADS == g["num_attention_heads"]
    assert O.N_KV_HEADS == g["num_key_value_heads"]
    assert O.N_Q_HEADS // O.N_KV_HEADS == g["num_key_value_groups"]
    assert O.HEAD_DIM == g["head_dim"]
    assert O.WINDOW == g["sliding_window"]
    full, sl = g["rope"]["full_attention"], g["rope"]["sliding_attention"]
    assert O.FULL.rope_theta == full["rope_theta"]
    assert O.SLIDING.rope_theta == sl["rope_theta"]
    assert O.FULL.rot_dim == int(g["head_dim"] * full["partial_rotary_factor"]) == full["rotated_dims"]
    assert O.SLIDING.rot_dim == int(g["head_dim"] * sl["partial_rotary_factor"]) == sl["rotated_dims"]
    sched = O.layer_schedule(g["num_hidden_layers"])
    assert [i for i, s in enumerate(sched) if s == "full"] == g["full_layer_indices"]
    assert sched.count("full") == g["n_full_layers"]
    assert sched.count("sliding") == g["n_sliding_layers"]
    assert sched[-1] == "full"


# ---------------------------------------------------------------------------- RoPE --
@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_frequencies_closed_form(kind):
    k = O.KINDS[kind]
    w = O.rope_inv_freq(k.rope_theta, k.rot_dim).to(torch.float64)
    r = k.rot_dim
    assert w.numel() == r // 2
    assert float(w[0]) == 1.0
    # omega_1 = theta^(-2/r), omega_last = theta^(-(r-2)/r), from the page constants
    assert float(w[1]) == pytest.approx(math.pow(k.rope_theta, -2.0 / r), rel=1e-7)
    assert float(w[-1]) == pytest.approx(math.pow(k.rope_theta, -(r - 2.0) / r), rel=1e-7)
    assert bool((w[1:] < w[:-1]).all())


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_is_complex_multiplication(kind):
    """Rotate-half RoPE == multiplying z_i = x_i + j x_{i+r/2} by exp(j * angle_i)."""
    k = O.KINDS[kind]
    r, half = k.rot_dim, k.rot_dim // 2
    x = _rand((5, 3, O.HEAD_DIM), 1)
    pos = torch.tensor([0, 1, 777, 131072, 1048575])
    y = O.rope_rotate(x, pos, kind).numpy().astype(np.float64)
    ang = O.rope_angles(pos, k.rope_theta, r).numpy().astype(np.float64)
    xn = x.numpy().astype(np.float64)
    for n in range(5):
        for h in range(3):
            for i in range(half):
                z = complex(xn[n, h, i], xn[n, h, i + half]) * cmath.exp(1j * ang[n, i])
                assert y[n, h, i] == pytest.approx(z.real, abs=2e-6)
                assert y[n, h, i + half] == pytest.approx(z.imag, abs=2e-6)


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_basis_vector_turns_by_position(kind):
    """omega_0 = 1, so e_0 at position p lands on (cos p, sin p) in dims (0, r/2)."""
    k = O.KINDS[kind]
    for p in (3, 131072, 1048576):
        x = torch.zeros(1, 1, O.HEAD_DIM)
        x[0, 0, 0] = 1.0
        y = O.rope_rotate(x, torch.tensor([p]), kind)
        assert float(y[0, 0, 0]) == pytest.approx(math.cos(p), abs=1e-7)
        assert float(y[0, 0, k.rot_dim // 2]) == pytest.approx(math.sin(p), abs=1e-7)
        others = torch.cat([y[0, 0, 1:k.rot_dim // 2], y[0, 0, k.rot_dim // 2 + 1:]])
        assert float(others.abs().max()) == 0.0


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_identity_norms_and_passthrough(kind):
    k = O.KINDS[kind]
    r, half = k.rot_dim, k.rot_dim // 2
    x = _rand((4, 16, O.HEAD_DIM), 2).to(torch.bfloat16)
    y0 = O.rope_rotate(x, torch.zeros(4, dtype=torch.int64), kind)
    assert torch.equal(y0, x.to(torch.float32))
    pos = torch.tensor([1, 511, 65537, 1048576])
    y = O.rope_rotate(x, pos, kind).to(torch.float64)
    xf = x.to(torch.float64)
    n_in = xf[..., :half] ** 2 + xf[..., half:r] ** 2
    n_out = y[..., :half] ** 2 + y[..., half:r] ** 2
    assert torch.allclose(n_in, n_out, rtol=1e-6, atol=1e-9)
    # dims r..255 pass through bit-exactly (full layers: 64..255)
    assert torch.equal(y[..., r:].to(torch.float32), x[..., r:].to(torch.float32))


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_rope_relative_position(kind):
    """<R(m) q, R(n) k> == <q, R(n - m) k>."""
    q = _rand((1, 1, O.HEAD_DIM), 3)
    kk = _rand((1, 1, O.HEAD_DIM), 4)
    for m, n in ((5, 300), (700, 12), (999, 999)):
        lhs = float((O.rope_rotate(q, torch.tensor([m]), kind).double()
                     * O.rope_rotate(kk, torch.tensor([n]), kind).double()).sum())
        d = n - m
        kr = O.rope_rotate(kk, torch.tensor([abs(d)]), kind)
        if d < 0:  # R(-d) k = R(d)^T k: rotate q by |d| instead
            rhs = float((O.rope_rotate(q, torch.tensor([abs(d)]), kind).double() * kk.double()).sum())
        else:
            rhs = float((q.double() * kr.double()).sum())
        scale = float(q.norm() * kk.norm())
        assert abs(lhs - rhs) <= 2e-3 * scale


# -------------------------------------------------------------- attention pins --
def _rows(S, pos0=0):
    return torch.arange(S, dtype=torch.int64) + pos0


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_matches_library_sdpa(kind):
    """Special case that reduces to torch's scaled_dot_product_attention (fp64, GQA by
    repeat-interleave, explicit band built with tril/triu) times the sigmoid gate."""
    S = 700
    q = _rand((S, 16, 256), 5)
    k = _rand((S, 4, 256), 6)
    v = _rand((S, 4, 256), 7)
    g = _rand((S, 16), 8)
    pos = _rows(S)
    y, lse = O.attend(q, k, v, g, pos, pos, kind)
    ones = torch.ones(S, S, dtype=torch.bool)
    band = torch.tril(ones) if kind == "full" else torch.tril(ones) & torch.triu(ones, diagonal=-511)
    ref = F.scaled_dot_product_attention(
        q.double().permute(1, 0, 2)[None], k.double().permute(1, 0, 2)[None],
        v.double().permute(1, 0, 2)[None], attn_mask=band, scale=1.0 / 16, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2) * torch.sigmoid(g.double())[..., None]
    assert torch.allclose(y, ref, rtol=1e-4, atol=1e-5)
    # LSE against logsumexp of the library's own scores
    s = torch.einsum("qhd,khd->hqk", q.double(), k.double().repeat_interleave(4, dim=1)) / 16
    s = s.masked_fill(~band[None], float("-inf"))
    assert torch.allclose(lse.T, torch.logsumexp(s, dim=-1), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_zero_query_uniform_weights_lse_closed_form(kind):
    """q = 0: every visible key weighs the same, so y_i = sigmoid(g_i) * mean(v visible)
    and LSE_i = ln(n_i) with n_i = min(i+1, 512) sliding, i+1 full."""
    S = 1100
    q = torch.zeros(S, 16, 256)
    k = _rand((S, 4, 256), 9)
    v = _rand((S, 4, 256), 10)
    g = _rand((S, 16), 11)
    pos = _rows(S)
    y, lse = O.attend(q, k, v, g, pos, pos, kind)
    i = torch.arange(S, dtype=torch.float64)
    n = torch.minimum(i + 1, torch.tensor(512.0)) if kind == "sliding" else i + 1
    assert torch.allclose(lse, torch.log(n)[:, None].expand(S, 16), atol=1e-9)
    for row in (0, 1, 510, 511, 512, 513, 1099):
        lo = max(0, row - 511) if kind == "sliding" else 0
        mean = v[lo:row + 1].double().mean(dim=0)  # [4, 256]
        for h in range(16):
            expect = mean[h // 4] / (1 + math.exp(-float(g[row, h])))
            assert torch.allclose(y[row, h], expect, rtol=1e-5, atol=1e-6)


def test_gqa_head_mapping_and_mha_equivalence():
    """Query head h reads KV head h // 4; GQA equals MHA with KV heads repeated 4x."""
    S = 64
    q = torch.zeros(S, 16, 256)
    k = _rand((S, 4, 256), 12)
    v = torch.zeros(S, 4, 256)
    for kvh in range(4):
        v[:, kvh, :] = kvh + 1.0
    g = torch.zeros(S, 16)
    y, _ = O.attend(q, k, v, g, _rows(S), _rows(S), "full")
    for h in range(16):
        assert torch.allclose(y[:, h, :], torch.full((S, 256), 0.5 * (h // 4 + 1), dtype=torch.float64))
    q = _rand((S, 16, 256), 13)
    v = _rand((S, 4, 256), 14)
    g = _rand((S, 16), 15)
    y1, l1 = O.attend(q, k, v, g, _rows(S), _rows(S), "full")
    y2, l2 = O.attend(q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), g,
                      _rows(S), _rows(S), "full")
    assert torch.allclose(y1, y2, atol=1e-12) and torch.allclose(l1, l2, atol=1e-12)


def test_first_row_sees_only_itself():
    S = 40
    q = _rand((S, 16, 256), 16)
    k = _rand((S, 4, 256), 17)
    v = _rand((S, 4, 256), 18)
    g = _rand((S, 16), 19)
    for kind in ("sliding", "full"):
        y, _ = O.attend(q, k, v, g, _rows(S), _rows(S), kind)
        for h in range(16):
            expect = v[0, h // 4].double() / (1 + math.exp(-float(g[0, h])))
            assert torch.allclose(y[0, h], expect, atol=1e-6)


def test_two_key_closed_form_pins_scale():
    """Full layer, content only in dims >= 64 (no rotation there): row 1 has logits
    (0, q.k/16) = (0, 4*8/16 = 2), so p = (1, e^2)/(1+e^2) and LSE = ln(1+e^2).
    Goes through the prefill entry (q unrotated)."""
    q = torch.zeros(2, 16, 256)
    q[1, :, 100] = 4.0
    kc = torch.zeros(2, 4, 256)
    kc[1, :, 100] = 8.0
    vc = _rand((2, 4, 256), 20)
    g = _rand((2, 16), 21)
    y, lse = O.prefill(q, kc, vc, g, 0, "full")
    p1 = math.exp(2) / (1 + math.exp(2))
    for h in range(16):
        sig = 1 / (1 + math.exp(-float(g[1, h])))
        expect = sig * ((1 - p1) * vc[0, h // 4].double() + p1 * vc[1, h // 4].double())
        assert torch.allclose(y[1, h], expect, atol=1e-6)
        assert float(lse[1, h]) == pytest.approx(math.log(1 + math.exp(2)), abs=1e-9)
        assert float(lse[0, h]) == pytest.approx(0.0, abs=1e-12)


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_probabilities_gate_and_linearity(kind):
    S = 600
    q = _rand((S, 16, 256), 22)
    k = _rand((S, 4, 256), 23)
    v = _rand((S, 4, 256), 24)
    pos = _rows(S)
    g0 = torch.zeros(S, 16)
    y0, _, p = O.attend(q, k, v, g0, pos, pos, kind, return_probs=True)
    assert torch.allclose(p.sum(dim=-1), torch.ones(16, S, dtype=torch.float64), atol=1e-12)
    vis = O.visible(pos, pos, kind)
    assert float(p[:, ~vis].abs().max()) == 0.0
    assert float(O.sigmoid64(torch.zeros(1))[0]) == 0.5
    g = _rand((S, 16), 25) * 4
    sg = O.sigmoid64(g)
    assert bool(((sg > 0) & (sg < 1)).all())
    y, _ = O.attend(q, k, v, g, pos, pos, kind)
    # output is linear in sigmoid(g): y(g) / sigmoid(g) == y(0) / 0.5
    assert torch.allclose(y / sg[..., None], y0 / 0.5, atol=1e-9)


def test_sliding_equals_full_when_short():
    S = 512
    q = _rand((S, 16, 256), 26)
    k = _rand((S, 4, 256), 27)
    v = _rand((S, 4, 256), 28)
    g = _rand((S, 16), 29)
    a = O.attend(q, k, v, g, _rows(S), _rows(S), "sliding")
    b = O.attend(q, k, v, g, _rows(S), _rows(S), "full")
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _brute_force(q, k, v, g, pos0, kind):
    """Naive fp64 loops with Python floats: rope, masked softmax, gate."""
    kd = O.KINDS[kind]
    r, half, th = kd.rot_dim, kd.rot_dim // 2, kd.rope_theta
    S = q.shape[0]
    qn, kn, vn, gn = (t.double().tolist() for t in (q, k, v, g))

    def rot(x, p):
        out = list(x)
        for i in range(half):
            w = np.float32(math.pow(th, -2.0 * i / r))
            a = float(np.float32(np.float32(p) * w))
            c, s = math.cos(a), math.sin(a)
            out[i] = x[i] * c - x[i + half] * s
            out[i + half] = x[i + half] * c + x[i] * s
        return out

    ys, lses = [], []
    for i in range(S):
        pi = pos0 + i
        yrow, lrow = [], []
        for h in range(16):
            qr = rot(qn[i][h], pi)
            sc = []
            for j in range(pos0 + S):
                if j > pi or (kd.window is not None and pi - j > kd.window - 1):
                    continue
                kr = rot(kn[j][h // 4], j)
                sc.append((j, math.fsum(a * b for a, b in zip(qr, kr)) / 16.0))
            mx = max(s for _, s in sc)
            den = math.fsum(math.exp(s - mx) for _, s in sc)
            sig = 1.0 / (1.0 + math.exp(-gn[i][h]))
            yrow.append([sig * math.fsum(math.exp(s - mx) / den * vn[j][h // 4][d] for j, s in sc)
                         for d in range(256)])
            lrow.append(mx + math.log(den))
        ys.append(yrow)
        lses.append(lrow)
    return torch.tensor(ys, dtype=torch.float64), torch.tensor(lses, dtype=torch.float64)


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_brute_force_tiny(kind):
    S = 6
    q = _rand((S, 16, 256), 30).to(torch.bfloat16)
    k = _rand((S, 4, 256), 31).to(torch.bfloat16)
    v = _rand((S, 4, 256), 32).to(torch.bfloat16)
    g = _rand((S, 16), 33).to(torch.bfloat16)
    _, kr = O.rope_qk(None, k, 0, kind)
    y, lse = O.prefill(q, kr, v, g, 0, kind)
    yb, lb = _brute_force(q, k, v, g, 0, kind)
    assert torch.allclose(y, yb, rtol=1e-4, atol=1e-5)
    assert torch.allclose(lse, lb, atol=1e-4)


# ---------------------------------------------------------------------- needles --
def test_needles_pin_window_edge_and_relative_rotation():
    """A planted key with a logit near 32 takes all the weight: visible at distance 511
    (sliding) or 5000 (full, on non-rotating dims); invisible at distance 512."""
    S, i = 1200, 1100
    for kind, j, dims, seen in (("sliding", i - 511, (127, 255), True),
                                ("sliding", i - 512, (127, 255), False),
                                ("full", 0, (128, 200), True)):
        base = synth.layer_inputs(77, 1, S)
        q, k, v, g = (base[n][0].clone() for n in ("q", "k", "v", "gate"))
        qb, kb = q[None], k[None]
        synth.plant_needle(qb, kb, 0, i, j, dims, 16.0)
        _, kr = O.rope_qk(None, k, 0, kind)
        y, _ = O.prefill(q, kr, v, g, 0, kind, rows=torch.tensor([i]))
        for h in range(16):
            target = v[j, h // 4].double() / (1 + math.exp(-float(g[i, h])))
            err = float((y[0, h] - target).norm() / target.norm())
            if seen:
                assert err < 1e-3
            else:
                assert err > 0.5


# ------------------------------------------------------------------ cache & decode --
def test_ring_slots_closed_form():
    assert int(O.append_slots(131072, 1, "sliding", 512)[0]) == 0
    assert int(O.append_slots(1044480, 1, "sliding", 512)[0]) == 0
    assert O.append_slots(1000, 30, "sliding", 512).tolist() == [(1000 + t) % 512 for t in range(30)]
    assert O.append_slots(5, 4, "full", 8).tolist() == [5, 6, 7, -1]
    held = O.ring_positions(1023)
    assert held.tolist() == list(range(512, 1024))
    held = O.ring_positions(300)
    assert held[:301].tolist() == list(range(301)) and bool((held[301:] == -1).all())
    held = O.ring_positions(1300)
    assert sorted(held.tolist()) == list(range(1300 - 511, 1301))


def test_ring_append_last_writer_wins():
    kn = _rand((1024, 4, 256), 34).to(torch.bfloat16)
    vn = _rand((1024, 4, 256), 35).to(torch.bfloat16)
    kc = torch.zeros(512, 4, 256, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    slots = O.kv_append(kc, vc, kn, vn, 0, "sliding")
    assert slots.tolist() == [t % 512 for t in range(1024)]
    assert torch.equal(kc, kn[512:]) and torch.equal(vc, vn[512:])


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_decode_equals_prefill_row_and_ring_equals_window(kind):
    S, pos = 900, 899
    base = synth.layer_inputs(78, 1, S)
    q, k, v, g = (base[n][0] for n in ("q", "k", "v", "gate"))
    _, kr = O.rope_qk(None, k, 0, kind)
    kr = kr.to(torch.bfloat16)
    yp, lp = O.prefill(q, kr, v, g, 0, kind, rows=torch.tensor([pos]))
    if kind == "full":
        yd, ld = O.decode(q[pos], kr, v, g[pos], pos, kind)
    else:
        kc = torch.zeros(512, 4, 256, dtype=torch.bfloat16)
        vc = torch.zeros_like(kc)
        O.kv_append(kc, vc, kr, v, 0, kind)
        yd, ld = O.decode(q[pos], kc, vc, g[pos], pos, kind)
    assert torch.allclose(yd, yp[0], atol=1e-6) and torch.allclose(ld, lp[0], atol=1e-6)


def test_ring_chunks_equal_one_shot_prefill():
    """Prefilling a sequence chunk by chunk, each chunk reading the ring that the previous
    chunks filled, gives the rows of one prefill over a position-indexed cache.  The ring
    starts as NaN, so reading a slot that no token has reached would poison the result."""
    S, cuts = 1337, [0, 100, 700, 733, 1337]   # chunks of 100, 600, 33 and 604 tokens
    base = synth.layer_inputs(79, 1, S)
    q, k, v, g = (base[n][0] for n in ("q", "k", "v", "gate"))
    _, kr = O.rope_qk(None, k, 0, "sliding")
    kr = kr.to(torch.bfloat16)
    y1, l1 = O.prefill(q, kr, v, g, 0, "sliding")
    ring_k = torch.full((512, 4, 256), float("nan"), dtype=torch.bfloat16)
    ring_v = torch.full_like(ring_k, float("nan"))
    for a, b in zip(cuts[:-1], cuts[1:]):
        yc, lc = O.prefill_ring(q[a:b], kr[a:b], v[a:b], ring_k, ring_v, g[a:b], a)
        assert torch.allclose(yc, y1[a:b], atol=1e-6, rtol=0), (a, b)
        assert torch.allclose(lc, l1[a:b], atol=1e-9, rtol=0), (a, b)
        O.kv_append(ring_k, ring_v, kr[a:b], v[a:b], a, "sliding")


def test_ring_prefill_brute_force_slot_lookup():
    """Naive per-(row, head, key) evaluation that locates each visible position by
    scanning the ring for the slot holding it, at a chunk that starts past one wrap."""
    pos0, n = 530, 3
    base = synth.layer_inputs(80, 1, pos0 + n)
    q, k, v, g = (base[nm][0] for nm in ("q", "k", "v", "gate"))
    _, kr = O.rope_qk(None, k, 0, "sliding")
    kr = kr.to(torch.bfloat16)
    ring_k = torch.zeros(512, 4, 256, dtype=torch.bfloat16)
    ring_v = torch.zeros_like(ring_k)
    for t in range(pos0):           # ring state after appending positions 0 .. pos0 - 1
        ring_k[t % 512], ring_v[t % 512] = kr[t], v[t]
    y, lse = O.prefill_ring(q[pos0:], kr[pos0:], v[pos0:], ring_k, ring_v, g[pos0:], pos0)
    qr, _ = O.rope_qk(q[pos0:], None, pos0, "sliding")
    for i in range(n):
        p = pos0 + i
        for h in range(16):
            scores, vals = [], []
            for j in range(max(0, p - 511), p + 1):
                if j >= pos0:
                    kj, vj = kr[j], v[j]
                else:
                    slot = [s for s in range(512) if s == j % 512 and j >= pos0 - 512][0]
                    kj, vj = ring_k[slot], ring_v[slot]
                kh = kj[h // 4].double().numpy()
                scores.append(float(np.dot(qr[i, h].double().numpy(), kh)) / 16.0)
                vals.append(vj[h // 4].double().numpy())
            sc = np.array(scores)
            w = np.exp(sc - sc.max())
            ref = (w[:, None] * np.stack(vals)).sum(0) / w.sum() / (1 + math.exp(-float(g[p, h])))
            assert np.allclose(y[i, h].numpy(), ref, atol=1e-5, rtol=1e-5)
            assert abs(float(lse[i, h]) - (sc.max() + math.log(w.sum()))) < 1e-5


# ---------------------------------------------------------------- 8-bit KV cache --
def test_e4m3_code_values_closed_form():
    """Code values from the E4M3 definition: bias 7, 3 mantissa bits, subnormals below
    2^-6, largest finite 448, 0x7F / 0xFF NaN."""
    codes = torch.tensor([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x77, 0x7E, 0x80, 0xB8, 0xFE],
                         dtype=torch.uint8)
    want = [0.0, 2 ** -9, 7 * 2 ** -9, 2 ** -6, 1.0, 1.5, 240.0, 448.0, -0.0, -1.0, -448.0]
    got = O.e4m3_decode(codes).tolist()
    assert got == want
    assert math.copysign(1, O.e4m3_decode(torch.tensor([0x80], dtype=torch.uint8))[0]) == -1
    nan = O.e4m3_decode(torch.tensor([0x7F, 0xFF], dtype=torch.uint8))
    assert bool(torch.isnan(nan).all())


def test_e4m3_encode_matches_library_and_round_trips():
    """Encoding matches torch's float8_e4m3fn conversion (round to nearest, ties to even)
    on random values and on every midpoint between neighbouring codes; every finite code
    decodes and re-encodes to itself."""
    g = torch.Generator().manual_seed(90)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-12, 9, (200000,), generator=g).float())
    x = x.clamp(-448, 448)
    fin = torch.tensor([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=torch.uint8)
    vals = O.e4m3_decode(fin).double()
    pos = torch.sort(vals[vals > 0]).values
    mids = ((pos[1:] + pos[:-1]) / 2).float()                 # exact ties in fp32
    for t in (x, mids, -mids):
        assert torch.equal(O.e4m3_encode(t), t.to(torch.float8_e4m3fn).view(torch.uint8))
    assert torch.equal(O.e4m3_encode(O.e4m3_decode(fin)), fin)


def test_kv_quantize_scale_and_error_bound():
    g = torch.Generator().manual_seed(91)
    x = (torch.randn(64, 4, 256, generator=g) * 3).to(torch.bfloat16)
    x[5, 2] = 0                                                # an all-zero row
    codes, scale = O.kv_quantize(x)
    xf = x.float()
    amax = xf.abs().amax(-1)
    assert torch.equal(scale, amax / 448.0)
    assert float(scale[5, 2]) == 0 and bool((codes[5, 2] == 0).all())
    # the largest element of every non-zero row lands on +-448 exactly
    idx = xf.abs().argmax(-1, keepdim=True)
    top = torch.gather(O.e4m3_decode(codes).abs(), -1, idx).squeeze(-1)
    assert bool((top[amax > 0] == 448.0).all())
    # half an E4M3 step: 2^-4 relative on normals, 2^-10 * scale absolute below them
    deq = O.kv_dequantize(codes, scale)
    err = (deq - xf).abs()
    bound = torch.maximum(2 ** -4 * xf.abs(), 2 ** -10 * scale[..., None]) * (1 + 1e-6)
    assert bool((err <= bound).all())
    assert O.kv8_bytes_per_token_layer() == 2080


@pytest.mark.parametrize("kind", ["sliding", "full"])
def test_decode_kv8_is_decode_of_dequantized_cache(kind):
    """decode_kv8 equals decode() on the dequantized cache, and stays within the noise
    that 3-bit mantissas put on N(0,1) data of the bf16 decode (a dropped or misapplied
    scale would move it by orders of magnitude)."""
    S, pos = 700, 699
    base = synth.layer_inputs(92, 1, S)
    q, k, v, g = (base[n][0] for n in ("q", "k", "v", "gate"))
    _, kr = O.rope_qk(None, k, 0, kind)
    kr = kr.to(torch.bfloat16)
    if kind == "sliding":
        kc = torch.zeros(512, 4, 256, dtype=torch.bfloat16)
        vc = torch.zeros_like(kc)
        O.kv_append(kc, vc, kr, v, 0, kind)
    else:
        kc, vc = kr, v
    kq, ks = O.kv_quantize(kc)
    vq, vs = O.kv_quantize(vc)
    y8, l8 = O.decode_kv8(q[pos], kq, vq, ks, vs, g[pos], pos, kind)
    yd, ld = O.decode(q[pos], O.kv_dequantize(kq, ks), O.kv_dequantize(vq, vs), g[pos], pos, kind)
    assert torch.equal(y8, yd) and torch.equal(l8, ld)
    y, l = O.decode(q[pos], kc, vc, g[pos], pos, kind)
    rel = (y8 - y).norm(dim=-1) / y.norm(dim=-1)
    assert float(rel.max()) < 0.08 and float((l8 - l).abs().max()) < 0.02


# ------------------------------------------------------------------- projections --
def test_qkv_slicing_with_selector_weights():
    """Weights whose rows pick single input columns: q, k, v and the gate come out as
    those columns, which fixes the slice order and offsets of the fused projection."""
    T = 5
    x = _rand((T, O.HIDDEN), 95).to(torch.bfloat16)
    sel = torch.randint(0, O.HIDDEN, (O.Q_DIM + 2 * O.KV_DIM + 16,), generator=torch.Generator().manual_seed(94))
    w = torch.zeros(O.Q_DIM + 2 * O.KV_DIM, O.HIDDEN, dtype=torch.bfloat16)
    w[torch.arange(w.shape[0]), sel[:w.shape[0]]] = 1
    wg = torch.zeros(16, O.HIDDEN, dtype=torch.bfloat16)
    wg[torch.arange(16), sel[w.shape[0]:]] = 1
    q, k, v, g = O.qkv_proj(x, w, wg)
    xf = x.float()
    assert torch.equal(q.reshape(T, -1), xf[:, sel[:O.Q_DIM]])
    assert torch.equal(k.reshape(T, -1), xf[:, sel[O.Q_DIM:O.Q_DIM + O.KV_DIM]])
    assert torch.equal(v.reshape(T, -1), xf[:, sel[O.Q_DIM + O.KV_DIM:w.shape[0]]])
    assert torch.equal(g, xf[:, sel[w.shape[0]:]])
    # head h of q is columns 256 h .. 256 h + 255 of the fused output
    assert torch.equal(q[:, 3, 7], xf[:, sel[3 * 256 + 7]])


def test_projections_match_library_linear_and_brute_force():
    g = torch.Generator().manual_seed(93)
    x = torch.randint(-3, 4, (4, O.HIDDEN), generator=g).to(torch.bfloat16)
    w = torch.randint(-2, 3, (O.Q_DIM + 2 * O.KV_DIM, O.HIDDEN), generator=g).to(torch.bfloat16)
    wg = torch.randint(-2, 3, (16, O.HIDDEN), generator=g).to(torch.bfloat16)
    q, k, v, gl = O.qkv_proj(x, w, wg)
    full = F.linear(x.double(), w.double())                     # exact: small integers
    assert torch.equal(torch.cat([q.reshape(4, -1), k.reshape(4, -1), v.reshape(4, -1)], 1).double(), full)
    assert torch.equal(gl.double(), F.linear(x.double(), wg.double()))
    # o_proj against a plain loop on two outputs
    a = torch.randint(-3, 4, (2, 16, 256), generator=g).to(torch.bfloat16)
    wo = torch.randint(-2, 3, (O.HIDDEN, O.Q_DIM), generator=g).to(torch.bfloat16)
    y = O.o_proj(a, wo)
    af = a.reshape(2, -1).tolist()
    for (t, n) in ((0, 0), (1, 2559), (1, 1234)):
        ref = sum(af[t][i] * float(wo[n, i]) for i in range(O.Q_DIM))
        assert float(y[t, n]) == ref


# ------------------------------------------------------------------ closed forms --
def test_kv_memory_matches_page_figures():
    m = json.loads((GOLD / "kv_memory.json").read_text())
    tol = m["rel_tol_printed"]
    assert O.kv_bytes_per_token_layer() == m["bytes_per_token_layer"]
    full36 = O.kv_cache_bytes(m["all_full_1m_tokens"], ["full"] * 36)
    assert full36 / 1e9 == pytest.approx(m["all_full_1m_GB"], rel=tol)
    assert O.kv_cache_bytes(m["all_full_32k_tokens"], ["full"] * 36) / 1e9 == pytest.approx(
        m["all_full_32k_GB"], rel=0.02)
    assert O.kv_cache_bytes(1 << 20, ["sliding"] * m["page_sliding_layers"]) / 1e6 == pytest.approx(
        m["page_sliding_MB"], rel=tol)
    assert O.kv_cache_bytes(1 << 20, ["full"] * m["page_full_layers"]) / 1e9 == pytest.approx(
        m["page_full_1m_GB"], rel=tol)
    # the 9 full / 27 sliding schedule: 38.65 GB + 56.6 MB at 1M tokens
    hybrid = O.kv_cache_bytes(1 << 20)
    assert hybrid == 9 * 4096 * (1 << 20) + 27 * 4096 * 512


@pytest.mark.parametrize("kind,sq,pos0", [("full", 37, 0), ("full", 50, 1000), ("sliding", 700, 0),
                                          ("sliding", 64, 300), ("sliding", 64, 5000)])
def test_pair_count_matches_mask(kind, sq, pos0):
    qp = torch.arange(sq) + pos0
    kp = torch.arange(pos0 + sq)
    assert O.attention_pairs_prefill(sq, pos0, kind) == int(O.visible(qp, kp, kind).sum())

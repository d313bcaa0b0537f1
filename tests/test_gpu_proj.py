"""GPU parity of the fused QKV + gate projection and of the output projection (bf16 MFMA
GEMMs) against the oracle's fp32 products: ragged token counts, exact selector weights,
and the 4096-token chunk.  Weights are seeded synthetic (no trained weights exist here)."""
import math

import pytest
import torch

import oracle as O
import synth
from parity import assert_bf16_close, check_outputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def h():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from full_gqa_attention_hattn_amd import hattn
    return hattn


def _cpu(t):
    return t.detach().cpu()


def _weights(seed, device="cuda"):
    """N(0, 1/fan_in) weights in the linear-layer layout, bf16."""
    def w(shape, s):
        return (synth.normal_bf16(shape, s, device).float() / math.sqrt(shape[1])).to(torch.bfloat16)
    return (w((O.Q_DIM + 2 * O.KV_DIM, O.HIDDEN), seed), w((16, O.HIDDEN), seed + 1),
            w((O.HIDDEN, O.Q_DIM), seed + 2))


def _run_qkv(h, x, w_qkv, w_g):
    T = x.shape[0]
    q = torch.empty(T, 16, 256, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(T, 4, 256, dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    g = torch.empty(T, 16, dtype=torch.bfloat16, device="cuda")
    h.qkv_proj(x, w_qkv, w_g, q, k, v, g)
    return q, k, v, g


def _rel_l2(gpu, ref, name, tol=2e-2):
    g, r = _cpu(gpu).double(), ref.double()
    rel = (g - r).norm(dim=-1) / r.norm(dim=-1).clamp_min(1e-30)
    assert float(rel.max()) <= tol, f"{name}: rel-L2 {float(rel.max()):.3e}"


@pytest.mark.parametrize("T", [1, 16, 17, 32, 37, 300])
def test_qkv_and_o_proj_match_oracle(h, T):
    say(f"projections T={T}")
    w_qkv, w_g, w_o = _weights(181)
    x = synth.normal_bf16((T, O.HIDDEN), 182, "cuda")
    q, k, v, g = _run_qkv(h, x, w_qkv, w_g)
    a = synth.normal_bf16((T, 16, 256), 183, "cuda")
    y = torch.empty(T, O.HIDDEN, dtype=torch.bfloat16, device="cuda")
    h.o_proj(a, w_o, y)
    torch.cuda.synchronize()
    rq, rk, rv, rg = O.qkv_proj(_cpu(x), _cpu(w_qkv), _cpu(w_g))
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("gate", g, rg)):
        assert_bf16_close(got, ref, f"{name} T={T}")
        _rel_l2(got, ref, f"{name} T={T}")
    ry = O.o_proj(_cpu(a), _cpu(w_o))
    assert_bf16_close(y, ry, f"o_proj T={T}")
    _rel_l2(y, ry, f"o_proj T={T}")


def test_qkv_selector_weights_exact(h):
    """Rows of one-hot weights: every output is an input value, so the GPU result must be
    bit-exact, which pins the slicing into q, k, v and the gate."""
    say("projections selector")
    T = 130
    x = synth.normal_bf16((T, O.HIDDEN), 184, "cuda")
    sel = torch.randint(0, O.HIDDEN, (O.Q_DIM + 2 * O.KV_DIM + 16,),
                        generator=torch.Generator().manual_seed(185))
    w = torch.zeros(O.Q_DIM + 2 * O.KV_DIM, O.HIDDEN, dtype=torch.bfloat16)
    w[torch.arange(w.shape[0]), sel[:w.shape[0]]] = 1
    wg = torch.zeros(16, O.HIDDEN, dtype=torch.bfloat16)
    wg[torch.arange(16), sel[w.shape[0]:]] = 1
    q, k, v, g = _run_qkv(h, x, w.cuda(), wg.cuda())
    torch.cuda.synchronize()
    rq, rk, rv, rg = O.qkv_proj(_cpu(x), w, wg)
    for got, ref in ((q, rq), (k, rk), (v, rv), (g, rg)):
        assert torch.equal(_cpu(got), ref.to(torch.bfloat16))


def test_projections_chunk_4096(h):
    """The 4096-token chunk (the launch configuration the bench times), sampled rows."""
    say("projections T=4096")
    T = 4096
    w_qkv, w_g, w_o = _weights(186)
    x = synth.normal_bf16((T, O.HIDDEN), 187, "cuda")
    q, k, v, g = _run_qkv(h, x, w_qkv, w_g)
    a = synth.normal_bf16((T, 16, 256), 188, "cuda")
    y = torch.empty(T, O.HIDDEN, dtype=torch.bfloat16, device="cuda")
    h.o_proj(a, w_o, y)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 127, 128, 2047, 4094, 4095])
    rq, rk, rv, rg = O.qkv_proj(_cpu(x)[rows], _cpu(w_qkv), _cpu(w_g))
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("gate", g, rg)):
        assert_bf16_close(_cpu(got)[rows], ref, f"{name} T=4096")
    ry = O.o_proj(_cpu(a)[rows], _cpu(w_o))
    assert_bf16_close(_cpu(y)[rows], ry, "o_proj T=4096")
    _rel_l2(_cpu(y)[rows], ry, "o_proj T=4096")


@pytest.mark.parametrize("T", [2048, 2100, 4000, 4096])
def test_projections_every_output_written(h, T):
    """Token counts where the 192 x 256 / 160 x 256 tiles (and the separate gate rows) may be
    chosen, with ragged last tiles: outputs start as NaN, every element must be written, and
    sampled rows at tile edges match the oracle."""
    say(f"projections coverage T={T}")
    w_qkv, w_g, w_o = _weights(191)
    x = synth.normal_bf16((T, O.HIDDEN), 192, "cuda")
    nan = float("nan")
    q = torch.full((T, 16, 256), nan, dtype=torch.bfloat16, device="cuda")
    k = torch.full((T, 4, 256), nan, dtype=torch.bfloat16, device="cuda")
    v = torch.full((T, 4, 256), nan, dtype=torch.bfloat16, device="cuda")
    g = torch.full((T, 16), nan, dtype=torch.bfloat16, device="cuda")
    h.qkv_proj(x, w_qkv, w_g, q, k, v, g)
    a = synth.normal_bf16((T, 16, 256), 193, "cuda")
    y = torch.full((T, O.HIDDEN), nan, dtype=torch.bfloat16, device="cuda")
    h.o_proj(a, w_o, y)
    torch.cuda.synchronize()
    for name, got in (("q", q), ("k", k), ("v", v), ("gate", g), ("o_proj", y)):
        assert not bool(torch.isnan(got).any()), f"{name} T={T}: unwritten outputs"
    last = (T - 1) // 256 * 256
    rows = torch.tensor(sorted({0, 1, 127, 128, 255, 256, 257, T // 2, last - 1, last, T - 2, T - 1}))
    rq, rk, rv, rg = O.qkv_proj(_cpu(x)[rows], _cpu(w_qkv), _cpu(w_g))
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("gate", g, rg)):
        assert_bf16_close(_cpu(got)[rows], ref, f"{name} T={T}")
    ry = O.o_proj(_cpu(a)[rows], _cpu(w_o))
    assert_bf16_close(_cpu(y)[rows], ry, f"o_proj T={T}")
    _rel_l2(_cpu(y)[rows], ry, f"o_proj T={T}")


def test_projections_past_a_million_tokens(h):
    """T = 2^20 + 40 tokens: more token blocks than a grid's y extent holds, so the launch
    geometry of every kernel the shape choice can pick is exercised at this size (about 32 GB
    of activations); sampled rows at the start and at the ragged end match the oracle."""
    T = (1 << 20) + 40
    say(f"projections T={T}")
    w_qkv, w_g, w_o = _weights(196)
    x = synth.normal_bf16((T, O.HIDDEN), 197, "cuda")
    q, k, v, g = _run_qkv(h, x, w_qkv, w_g)
    a = synth.normal_bf16((T, 16, 256), 198, "cuda")
    y = torch.empty(T, O.HIDDEN, dtype=torch.bfloat16, device="cuda")
    h.o_proj(a, w_o, y)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 255, 256, T // 2, T - 41, T - 40, T - 2, T - 1])
    rq, rk, rv, rg = O.qkv_proj(_cpu(x[rows]), _cpu(w_qkv), _cpu(w_g))
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("gate", g, rg)):
        assert_bf16_close(_cpu(got[rows.cuda()]), ref, f"{name} T={T}")
    ry = O.o_proj(_cpu(a[rows.cuda()]), _cpu(w_o))
    assert_bf16_close(_cpu(y[rows.cuda()]), ry, f"o_proj T={T}")

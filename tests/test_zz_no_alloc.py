"""The allocation-free decode entry point (hattn_decode_noalloc), called through the C ABI,
against the existing entry point (hattn_decode with a caller workspace) on the same
inputs: two calls in a row per layer kind, the second smaller than the first, each held
to the parity bar against hattn_decode's output (and, since both run the same kernels and
split plan, to its bits) and to the oracle."""
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


# (kind, positions, cap): per kind, a larger call then a smaller one.  Sliding: B = 2 and
# 1 (8 ring splits), then B = 12 (4 splits); the partials and arrival counters live in
# the scratch.
CASES = {
    "full": [([131072, 70000, 5, 131071, 100000, 2, 90000, 131000], 131136),
             ([4000, 777], 4096)],
    "sliding": [([131072, 600], 512), ([300], 512),
                ([5000, 1 << 20, 40, 0, 511, 512, 131072, 77, 300, 9999, (1 << 31) - 1, 1000], 512)],
}


@pytest.mark.parametrize("kind", ["full", "sliding"])
def test_noalloc_matches_workspace_decode(h, kind):
    cfg = h.preset(kind)
    for i, (positions, cap) in enumerate(CASES[kind]):
        B = len(positions)
        say(f"noalloc {kind} call {i}: B={B} cap={cap}")
        new = synth.layer_inputs(300 + i, B, 1, "cuda")
        cache = synth.cache_inputs(310 + i, B, cap, cap, "cuda")
        K, V = cache["cache_k"], cache["cache_v"]
        pos = synth.positions(positions, B, "cuda")
        ref_out = torch.empty_like(new["q"])
        ref_lse = torch.empty(B, 1, 16, dtype=torch.float32, device="cuda")
        ws = h.alloc_workspace(cfg, B, cap)
        h.decode(cfg, new["q"], K, V, pos, new["gate"], ref_out, ref_lse, ws, rope_q_fused=True)
        out = torch.full_like(new["q"], float("nan"))
        lse = torch.full((B, 1, 16), float("nan"), dtype=torch.float32, device="cuda")
        h.decode_noalloc(cfg, new["q"], K, V, pos, new["gate"], out, lse, rope_q_fused=True)
        torch.cuda.synchronize()
        assert_bf16_close(out, ref_out.float(), f"noalloc {kind} call {i} vs workspace decode")
        assert float((lse - ref_lse).abs().max()) <= 1e-2
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), \
            "same kernels and plan, so the same bits"
        for b, p in enumerate(positions):
            y, l = O.decode(_cpu(new["q"][b, 0]), _cpu(K[b]), _cpu(V[b]), _cpu(new["gate"][b, 0]),
                            p, kind)
            check_outputs(out[b, 0], lse[b, 0], y, l, f"noalloc {kind} call {i} b={b} p={p}")

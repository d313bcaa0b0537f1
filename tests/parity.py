"""Comparison helpers for GPU-vs-oracle parity (imported by the gpu tests).

Bar (from the layer's specification): bf16 outputs within |err| <= 2e-2 + 2e-2 |ref| per
element; integer outputs bit-exact.  Because long rows of N(0,1) data have outputs far
below 2e-2, two more checks discriminate: the fp32 LSE within 1e-2 and, per (row, head),
the relative L2 error of the 256-dim output within 2e-2.
"""
import sys

import torch

ATOL = 2e-2
RTOL = 2e-2
LSE_TOL = 1e-2
REL_L2_TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_bf16_close(gpu, ref, name, atol=ATOL, rtol=RTOL):
    g = gpu.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    err = (g - r).abs()
    bound = atol + rtol * r.abs()
    bad = err > bound
    n_bad = int(bad.sum())
    assert torch.isfinite(g).all(), f"{name}: non-finite GPU output"
    assert n_bad == 0, (f"{name}: {n_bad} of {bad.numel()} elements out of tolerance; "
                        f"max err {float(err.max()):.3e}")
    return float(err.max())


def assert_lse_close(gpu, ref, name, tol=LSE_TOL):
    g = gpu.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    err = (g - r).abs()
    assert float(err.max()) <= tol, f"{name}: LSE max err {float(err.max()):.3e}"
    return float(err.max())


def assert_rel_l2(gpu, ref, name, tol=REL_L2_TOL):
    """Per (row, head) relative L2 error over the head dim (last axis)."""
    g = gpu.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    num = (g - r).norm(dim=-1)
    den = r.norm(dim=-1).clamp_min(1e-30)
    rel = num / den
    worst = float(rel.max())
    at = [int(i) for i in torch.nonzero(rel == rel.max())[0]]
    assert worst <= tol, f"{name}: worst per-row relative L2 error {worst:.3e} at index {at}"
    return worst


def check_outputs(gpu_out, gpu_lse, ref_out, ref_lse, name):
    e1 = assert_bf16_close(gpu_out, ref_out, name)
    e2 = assert_rel_l2(gpu_out, ref_out, name)
    e3 = assert_lse_close(gpu_lse, ref_lse, name) if gpu_lse is not None else None
    say(f"{name}: max abs err {e1:.2e}, worst rel-L2 {e2:.2e}, LSE err {e3}")


def check_needle_row(gpu_out, gpu_lse, ref_out, ref_lse, name):
    """A planted-needle row: element tolerance as usual; its LSE, set by a logit of ~32
    or by logits spread far wider than N(0, 1), is held to 1e-2 + 2^-7 |LSE|.  The bf16
    operands of a needle (amplitude 16 on two rotated dims) carry a rounding error that
    scales the row's logits by a common 1 + O(2^-9) each, which moves the LSE in
    proportion to its size; a leaked or missed needle moves it by ~25."""
    e1 = assert_bf16_close(gpu_out, ref_out, name)
    g = gpu_lse.detach().to("cpu", torch.float64)
    r = ref_lse.detach().to("cpu", torch.float64)
    err = (g - r).abs()
    assert bool((err <= 1e-2 + 2 ** -7 * r.abs()).all()), f"{name}: LSE err {float(err.max()):.3e}"
    say(f"{name}: max abs err {e1:.2e}, LSE err {float(err.max()):.2e}")


def assert_rotated(gpu, ref, src, rot_dim, name):
    """Keys or queries rotated on the GPU (bf16) against the oracle's rotation of the same
    source (fp32): the rotated dims within one bf16 rounding and, for more than 98% of
    them, equal to the round-to-nearest of the oracle; the pass-through dims equal to the
    source bit for bit."""
    g = gpu.detach().cpu()
    r = ref.detach().cpu()
    err = (g[..., :rot_dim].double() - r[..., :rot_dim].double()).abs()
    bound = 2 ** -8 * r[..., :rot_dim].double().abs() + 1e-5
    assert bool((err <= bound).all()), f"{name}: rotated dims off by {float((err - bound).max()):.3e}"
    exact = float((g[..., :rot_dim] == r[..., :rot_dim].to(torch.bfloat16)).double().mean())
    assert exact > 0.98, f"{name}: only {exact:.3f} of rotated dims round-to-nearest"
    if rot_dim < g.shape[-1]:
        assert torch.equal(g[..., rot_dim:], src.detach().cpu()[..., rot_dim:]), \
            f"{name}: pass-through dims changed"


def row_blocks(rows, block=64):
    """Sorted distinct query rows in blocks of `block`, so the oracle's key range and its
    score matrices stay those of one block."""
    rows = sorted(set(int(r) for r in rows))
    for i in range(0, len(rows), block):
        yield torch.tensor(rows[i:i + block])


class Coverage:
    """Counts the (row, head) outputs an oracle comparison covered, for the report."""

    def __init__(self, name, total_rows, unit="rows"):
        self.name, self.total, self.rows, self.unit = name, int(total_rows), 0, unit
        self.worst_abs = self.worst_rel = self.worst_lse = 0.0

    def check(self, gpu_out, gpu_lse, ref_out, ref_lse):
        e1 = assert_bf16_close(gpu_out, ref_out, self.name)
        e2 = assert_rel_l2(gpu_out, ref_out, self.name)
        e3 = assert_lse_close(gpu_lse, ref_lse, self.name)
        self.rows += int(ref_out.shape[0])
        self.worst_abs = max(self.worst_abs, e1)
        self.worst_rel = max(self.worst_rel, e2)
        self.worst_lse = max(self.worst_lse, e3)

    def report(self):
        say(f"{self.name}: checked {self.rows} of {self.total} {self.unit} "
            f"({100.0 * self.rows / self.total:.2f}%), every head and dim; max abs err "
            f"{self.worst_abs:.2e}, worst rel-L2 {self.worst_rel:.2e}, LSE err {self.worst_lse:.2e}")
